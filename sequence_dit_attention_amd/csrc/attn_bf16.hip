// bf16 flash attention of a rank's local queries against the full K/V, gfx950.
//
// Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", section 机制一: the
// local shard provides Q, K/V span the whole sequence, no mask.  Scale 1/sqrt(d)
// is passed in (page "NPU HunyuanImage-3.0模型推理优化实践", 消除FA中scale的冗余计算).
//
// Design (MI355X / CDNA4):
//  * One work-group = 4 waves = BM query rows of one head; each wave owns
//    32*QB rows whose Q fragments stay in VGPRs for the whole key loop.
//  * Keys stream through LDS in tiles of 64 (K and V, double buffered, 16-byte
//    chunks XOR-swizzled per row so MFMA operand reads spread over the banks).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of ONE query column, so the softmax max and sum
//    are lane-local except for one exchange between the two wave halves.
//  * The probabilities are converted to bf16 in place (v_cvt_pk_bf16_f32) and
//    feed O^T += V^T P^T directly as the MFMA B operand; the matching V^T
//    operand is read from the row-major V tile with the gfx950 transposing LDS
//    read ds_read_b64_tr_b16.  The k index of that MFMA is a permutation of
//    the keys (the layout the S^T accumulator already has); the same
//    permutation is applied to V, so the contraction is unchanged.
//  * Online softmax in float32, base 2, scale folded into log2(e).
//  * Work-group ids are remapped so that the work-groups resident on one XCD
//    (dispatch is round-robin over the 8 XCDs) work on neighbouring query
//    tiles of the same head and share that head's K/V stream in their L2.
// Per output row the arithmetic depends only on that query row and on K/V in
// a fixed key order, so results are deterministic and independent of sq and
// of the row's position inside a tile.
#include "internal.h"

namespace spattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;         // keys per tile
constexpr int kKB = kBN / 32;   // 32-key blocks per tile
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
struct Geo {
  static constexpr int kCh = D / 8;                      // 16-byte chunks per K/V row
  static constexpr int kDC = D / 16;                     // k-steps of the Q.K MFMA
  static constexpr int kND = D / 32;                     // 32-row d-blocks of O^T
  static constexpr int kRowB = D * 2;                    // bytes per K/V row
  static constexpr int kTileB = kBN * kRowB;             // bytes per K or V tile
  static constexpr int kStage = kBN * kCh / kThreads;    // 16-byte chunks per lane per tile
  // K rows: chunk c of row r lives at c ^ (r mod kCh): the 32 rows one
  // MFMA operand read touches land on distinct chunk columns.
  static __device__ int swz_k(int r, int c) { return c ^ (r & (kCh - 1)); }
  // V rows: the transposing read takes 4 rows x 32 bytes per 16 lanes; XOR
  // with 4*(r mod kCh/4) moves those rows to different 64-byte bank groups.
  static __device__ int swz_v(int r, int c) { return c ^ ((r & (kCh / 4 - 1)) << 2); }
};

__device__ inline float other_half(float x) { return __shfl_xor(x, 32); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, nearest-even
  return __builtin_bit_cast(uint32_t, h);
}

template <int D, int QB>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int sq, int skv, int H, float c,
    int nqt, int nwg, int per_xcd) {
  using G = Geo<D>;
  constexpr int BM = kWaves * 32 * QB;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * G::kTileB];

  // XCD-aware remap: hardware block b runs on XCD b % 8.
  const int b = blockIdx.x;
  const int L = (b & 7) * per_xcd + (b >> 3);
  if (L >= nwg) return;
  const int h = L / nqt;
  const int qt = L - h * nqt;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column inside a 32-block / row inside an MFMA A operand
  const int hf = lane >> 5;    // wave half
  const int64_t rowstride = int64_t(H) * D;  // elements between consecutive tokens

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds 8 d-values of one query.
  bf16x8 qf[QB][G::kDC];
  const int qrow0 = qt * BM + wave * 32 * QB;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + col;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + int64_t(row) * rowstride + int64_t(h) * D + 8 * hf);
#pragma unroll
    for (int cc = 0; cc < G::kDC; ++cc) {
      u32x4 t = row < sq ? src[2 * cc] : u32x4{0, 0, 0, 0};
      qf[qb][cc] = __builtin_bit_cast(bf16x8, t);
    }
  }

  f32x16 acc_o[G::kND][QB];
#pragma unroll
  for (int db = 0; db < G::kND; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][qb][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  // ---- K/V staging: global -> VGPRs -> LDS, one tile ahead.
  const uint16_t* kh = k + int64_t(h) * D;
  const uint16_t* vh = v + int64_t(h) * D;
  u32x4 stk[G::kStage], stv[G::kStage];
  auto stage_load = [&](int t) {
    const int kv0 = t * kBN;
#pragma unroll
    for (int i = 0; i < G::kStage; ++i) {
      const int cidx = tid + i * kThreads;
      const int r = cidx / G::kCh, cch = cidx % G::kCh;
      const int j = kv0 + r;
      if (j < skv) {
        stk[i] = *reinterpret_cast<const u32x4*>(kh + int64_t(j) * rowstride + cch * 8);
        stv[i] = *reinterpret_cast<const u32x4*>(vh + int64_t(j) * rowstride + cch * 8);
      } else {
        stk[i] = u32x4{0, 0, 0, 0};
        stv[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto stage_store = [&](int buf) {
    char* kb = smem + buf * 2 * G::kTileB;
    char* vb = kb + G::kTileB;
#pragma unroll
    for (int i = 0; i < G::kStage; ++i) {
      const int cidx = tid + i * kThreads;
      const int r = cidx / G::kCh, cch = cidx % G::kCh;
      *reinterpret_cast<u32x4*>(kb + r * G::kRowB + G::swz_k(r, cch) * 16) = stk[i];
      *reinterpret_cast<u32x4*>(vb + r * G::kRowB + G::swz_v(r, cch) * 16) = stv[i];
    }
  };

  const int nT = (skv + kBN - 1) / kBN;
  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int t = 0; t < nT; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < nT;
    if (more) stage_load(t + 1);
    const char* kb_lds = smem + buf * 2 * G::kTileB;
    const char* vb_lds = kb_lds + G::kTileB;

    // ---- S^T = K Q^T for 64 keys x 32*QB queries.
    f32x16 s[kKB][QB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < G::kDC; ++cc) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const int r = kb * 32 + col;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_lds + r * G::kRowB + G::swz_k(r, 2 * cc + hf) * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][cc], s[kb][qb], 0, 0, 0);
      }
    }

    // ---- keys past the end of the sequence (last tile only) get -inf.
    const int kv0 = t * kBN;
    if (kv0 + kBN > skv) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= skv)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = -INFINITY;
        }
    }

    // ---- online softmax (base 2) per query column; P in bf16 as MFMA B operand.
    u32x4 pb[kKB][QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, other_half(mx));
      const float m_new = fmaxf(m_run[qb], mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c, -m_new));
          s[kb][qb][r] = p;
          rs += p;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[kb][qb][u][e] = pack_bf16x2(s[kb][qb][8 * u + 2 * e], s[kb][qb][8 * u + 2 * e + 1]);
      }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < G::kND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][qb][r] *= alpha;
    }

    // ---- O^T += V^T P^T.  MFMA (kb, u) contracts keys kb*32 + 16u + {4hf..4hf+3, 8+4hf..8+4hf+3}
    // in k-slots 8hf..8hf+7, the order in which the S^T accumulator holds them.
    const int g16 = lane >> 4, j16 = lane & 15;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = kb * 32 + 16 * u + 4 * hf + (j16 >> 2);
#pragma unroll
        for (int db = 0; db < G::kND; ++db) {
          const int dcol = db * 32 + 16 * (g16 & 1) + 4 * (j16 & 3);
          const int ch = dcol >> 3, inb = (dcol & 7) * 2;
          const lds_i16x4* p0 = (const lds_i16x4*)(vb_lds + r0 * G::kRowB + G::swz_v(r0, ch) * 16 + inb);
          const lds_i16x4* p1 = (const lds_i16x4*)(vb_lds + (r0 + 8) * G::kRowB + G::swz_v(r0 + 8, ch) * 16 + inb);
          const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p0));
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p1));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc_o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, __builtin_bit_cast(bf16x8, pb[kb][qb][u]), acc_o[db][qb], 0, 0, 0);
        }
      }
    }

    if (more) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, rows past sq are dropped.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + other_half(l_run[qb]);
    const float inv = 1.f / lt;
    const int row = qrow0 + qb * 32 + col;
    if (row < sq) {
      uint16_t* dst = o + int64_t(row) * rowstride + int64_t(h) * D;
#pragma unroll
      for (int db = 0; db < G::kND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          u32x2 w;
          w[0] = pack_bf16x2(acc_o[db][qb][4 * g] * inv, acc_o[db][qb][4 * g + 1] * inv);
          w[1] = pack_bf16x2(acc_o[db][qb][4 * g + 2] * inv, acc_o[db][qb][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + d0) = w;
        }
      if (lse && hf == 0) lse[int64_t(h) * sq + row] = (m_run[qb] + __log2f(lt)) * kLn2;
    }
  }
}

template <int D, int QB>
hipError_t launch_cfg(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                      int64_t skv, int H, float c, hipStream_t stream) {
  constexpr int BM = kWaves * 32 * QB;
  const int64_t nqt = (sq + BM - 1) / BM;
  const int64_t nwg = nqt * H;
  const int64_t per = (nwg + 7) / 8;
  const int64_t grid = per * 8;
  if (grid > kMaxGrid) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_bf16_kernel<D, QB>), dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, int(sq), int(skv), H,
                     c, int(nqt), int(nwg), int(per));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                            int64_t skv, int H, int d, float scale, hipStream_t stream) {
  if (sq > (int64_t(1) << 31) - 1024) return hipErrorInvalidValue;
  const float c = scale * 1.4426950408889634f;
  if (d == 64) return launch_cfg<64, 1>(q, k, v, o, lse, sq, skv, H, c, stream);
  return launch_cfg<128, 1>(q, k, v, o, lse, sq, skv, H, c, stream);
}

}  // namespace spattn

// bf16 flash attention of a rank's local queries against the full K/V, gfx950:
// the kernel for head size 64, the merge of split-key partials, and the
// dispatch by head size (128 and 512 have kernels of their own, attn_d128.hip
// and attn_d512.hip).
//
// Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", section 机制一: the
// local shard provides Q, K/V span the whole sequence, no mask.  Scale 1/sqrt(d)
// is passed in (page "NPU HunyuanImage-3.0模型推理优化实践", 消除FA中scale的冗余计算).
//
// Design (MI355X / CDNA4):
//  * One work-group = 4 waves (one per SIMD) = 256 query rows of one head; each
//    wave owns 64 rows (two 32-column MFMA blocks), whose Q fragments stay in
//    VGPRs for the whole key loop.  Two query blocks per wave halve the LDS
//    operand reads per MFMA flop, which bound a 32-row-per-wave layout.
//  * Keys stream through LDS in tiles of 64, K and V double buffered, filled
//    by global_load_lds_dwordx4 straight from HBM/L2 (no VGPR staging).  Each
//    row's 16-byte chunks are XOR-swizzled; because an LDS-direct load writes
//    lane i at base + 16*i, the swizzle is applied to the global addresses.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of ONE query column, so the softmax max and sum
//    are lane-local except for one v_permlane32_swap between wave halves.
//  * The probabilities are converted to bf16 in place (v_cvt_pk_bf16_f32) and
//    feed O^T += V^T P^T as the MFMA B operand; the V^T operand is read from
//    the row-major V tile with the transposing LDS read ds_read_b64_tr_b16.
//    The k index of that MFMA is a permutation of the keys (the order in
//    which the S^T accumulator holds them); V is read in the same order, so
//    the contraction is unchanged.
//  * Online softmax in float32, base 2, scale folded into log2(e).  The
//    reference maximum starts at the first block's maximum and is only raised
//    when a block would hold a probability above 2^kTau: probabilities then
//    stay <= 2^8, harmless in float32 sums and bf16 operands.  Instead of a
//    maximum per block, the probabilities are computed against the current
//    reference and a lane's block sum (needed anyway) is compared with 2^kTau
//    before the block enters P*V; only when that check fires (a handful of
//    times per row) is the block's maximum taken, O rescaled and the block
//    redone.  The result O = sum(p v) / sum(p) does not depend on the
//    reference.  Row sums add the bf16 probabilities the P*V product uses
//    (v_dot2 with ones), so O is normalised by exactly the weights it was
//    built from.
//  * Software pipeline: while the softmax of tile t runs on the VALU, the
//    MFMAs already compute S^T of tile t+1 (independent registers), then P*V
//    of tile t follows.  The loop is unrolled by two so the two S^T register
//    sets alternate roles without copies.
//  * Work-groups are ordered head-major, so at any time all XCDs work on the
//    same head: its K+V stays in the 256 MB Infinity Cache and each XCD's L2
//    serves its co-resident query tiles.
//  * Head size 64.  (This layout also ran head size 128 at one wave per SIMD;
//    the eight-wave kernel of attn_d128.hip, two waves per SIMD with one
//    wave's softmax under the other's MFMAs, replaced it there.)
// Per output row the arithmetic depends only on that query row and on K/V in
// a fixed key order, so results are deterministic and independent of sq and
// of the row's position inside a tile.
#include "internal.h"

#include <mutex>
#include <type_traits>
#include <utility>

namespace spattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Build-time shape knobs.  The defaults are the configuration the library is
// built, tested and measured with; other values compile (they were used to
// time alternatives) but are not part of the tested product.
#ifndef SPATTN_WAVES
#define SPATTN_WAVES 4
#endif
#ifndef SPATTN_QB
#define SPATTN_QB 2
#endif
constexpr int kWaves = SPATTN_WAVES;   // waves per work-group
constexpr int kThreads = 64 * kWaves;
#ifndef SPATTN_RA
#define SPATTN_RA 2  // LDS operand reads are issued this many MFMA groups ahead of their use
#endif
constexpr int kRA = SPATTN_RA;
#ifndef SPATTN_LEAD
#define SPATTN_LEAD 1  // K/V tiles loaded ahead of the one in use (head sizes 64, 128)
#endif
#ifndef SPATTN_EOFF
#define SPATTN_EOFF 2  // P*V slots before the first probability word of the next block is made
#endif
#ifndef SPATTN_EARLY
#define SPATTN_EARLY 4  // of the 8 words per query block, those made one step early
#endif
#ifndef SPATTN_BN
#define SPATTN_BN 64  // keys per tile (head sizes 64, 128)
#endif
constexpr int pow2_ceil(int x) { return x <= 1 ? 1 : 2 * pow2_ceil((x + 1) / 2); }
constexpr float kTau = 8.0f;           // lazy-rescale threshold (log2 units)
constexpr float kCheck = 256.0f;       // 2^kTau: a lane's block sum above it triggers the reference check
constexpr float kLn2 = 0.69314718055994531f;

// Shape of the kernel for head size D (64): two 32-query blocks per wave
// (QB), 64-key tiles, every output column.
template <int D>
struct Geo {
  static_assert(D == 64, "head size 64 (128 and 512 have kernels of their own)");
  static constexpr int kD = D;
  static constexpr int QB = SPATTN_QB;                    // 32-query MFMA blocks per wave
  static constexpr int BM = kWaves * 32 * QB;             // query rows per work-group
  static constexpr int kBN = SPATTN_BN;                   // keys per tile
  static constexpr int kSteps = kBN / 32;                 // 32-key steps per tile
  static_assert(kSteps == 1 || kSteps % 2 == 0, "the two S^T register sets alternate within a tile");
  // Probability words per query block made one step early, under the P*V
  // MFMAs of the previous step (the part of a step that has no other VALU work).
  static constexpr int kEarly = SPATTN_EARLY;
  // With two or more steps per tile, the first K fragments of the block after
  // next are read ahead at the end of a step; with one step that block is two
  // tiles ahead and the fragments are read at the start of the step instead.
  static constexpr bool kPrefetch = kSteps >= 2;
  static constexpr int kCh = D / 8;                       // 16-byte chunks per K row
  static constexpr int kVCh = D / 8;                      // 16-byte chunks per V row
  static constexpr int kDC = D / 16;                      // k-steps of the Q.K MFMA
  static constexpr int kND = D / 32;                      // 32-row d-blocks of O^T
  static constexpr int kRowB = D * 2;                     // bytes per K row
  static constexpr int kVRowB = D * 2;                    // bytes per V row in LDS
  static constexpr int kTileB = kBN * kRowB;              // bytes per K tile
  static constexpr int kVTileB = kBN * kVRowB;            // bytes per V tile
  static constexpr int kLoads = kTileB / (kThreads * 16); // LDS-direct loads per lane per K tile
  static constexpr int kVLoads = kVTileB / (kThreads * 16);
  // K: tile t+1 read (and tile t too when a tile holds several steps),
  // t+2 .. t+1+kLead loading.  V: tile t read, t+1 .. t+kLead loading.  Slot
  // counts are rounded up to powers of two (slot indices become masks) when
  // that still fits the 160 KiB of LDS.
  static constexpr int kLead = SPATTN_LEAD;               // K/V tiles in flight ahead of the one in use
  static constexpr int kKNeed = kLead + (kSteps >= 2 ? 2 : 1);
  static constexpr int kVNeed = kLead + 1;
  static constexpr bool kPow2 = pow2_ceil(kKNeed) * kTileB + pow2_ceil(kVNeed) * kVTileB <= 160 * 1024;
  static constexpr int kKSlots = kPow2 ? pow2_ceil(kKNeed) : kKNeed;
  static constexpr int kVSlots = kPow2 ? pow2_ceil(kVNeed) : kVNeed;
  // K rows: chunk c of row r lives at c ^ (r mod kCh): the 32 rows an MFMA
  // operand read touches land on distinct chunk columns.
  static __device__ int swz_k(int r) { return r & (kCh - 1); }
  // V rows: the transposing read takes 4 rows x 32 bytes per 16 lanes; XOR
  // with 4*(r mod kVCh/4) moves those rows to different 64-byte bank groups.
  static __device__ int swz_v(int r) { return (r & (kVCh / 4 - 1)) << 2; }
};

__device__ inline float other_half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, nearest-even
  return __builtin_bit_cast(uint32_t, h);
}

// ---- K/V tile loads: LDS-direct buffer loads.  Wave w fills 1 KiB blocks
// w*kLoads .. w*kLoads+kLoads-1 of a 64-row tile; lane i of a load writes
// bytes [16i, 16i+16) of its block, so the per-lane source offsets (row, and
// the chunk that the XOR swizzle maps to that position) are fixed for the
// whole kernel and only the tile base (scalar) moves.
template <typename G, bool IS_V>
struct TileLoader {
  static constexpr int kLoads = IS_V ? G::kVLoads : G::kLoads;
  static constexpr int kRowB = IS_V ? G::kVRowB : G::kRowB;  // bytes of a tile row in LDS
  uint32_t voff[kLoads];  // byte offset of this lane's chunk from the tile's first row
  int rows[kLoads];       // tile row this lane loads

  __device__ void init(int wave, int lane, int64_t rowbytes) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int byte = (wave * kLoads + i) * 1024 + lane * 16;
      const int r = byte / kRowB;
      const int p = (byte % kRowB) >> 4;
      const int c = p ^ (IS_V ? G::swz_v(r) : G::swz_k(r));
      rows[i] = r;
      voff[i] = uint32_t(r * rowbytes + c * 16);
    }
  }
  // Buffer resource of a 64-row tile: base address, stride 0 (raw), 2 GiB range.
  static __device__ i32x4 rsrc(const char* base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFF), 0x7FFFFFFF, 0x00020000};
  }
  // One LDS-direct 16-byte load per lane.  Issued as inline asm so that the
  // compiler does not treat these in-flight LDS writes as aliasing every LDS
  // read that follows (it would wait for them with vmcnt(0) before the first
  // transposing read and serialise the tile pipeline).  The kernel waits for
  // them itself, with vmcnt, before the barrier that publishes a tile.
  static __device__ void issue(const i32x4& rs, char* lds_blk, uint32_t voffset) {
    // LDS address of this wave's 1 KiB block (wave-uniform; M0 needs an SGPR)
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds_blk)));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(rs)
                 : "memory", "m0");
  }
  // Full tile: every row < skv.
  __device__ void load(const uint16_t* hb, int tile, int64_t rowbytes, char* lds, int wave) const {
    const char* base = reinterpret_cast<const char*>(hb) + int64_t(tile) * G::kBN * rowbytes;
    const i32x4 rs = rsrc(base);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) issue(rs, lds + (wave * kLoads + i) * 1024, voff[i]);
  }
  // Full tile at byte address `addr` (wave-uniform).
  __device__ void load_at(uint64_t addr, char* lds, int wave) const {
    const i32x4 rs = rsrc(reinterpret_cast<const char*>(addr));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) issue(rs, lds + (wave * kLoads + i) * 1024, voff[i]);
  }
  // Tile whose first row is at `base` (wave-uniform); rows >= valid re-read
  // row valid-1 (see load_clamped).
  __device__ void load_base(const char* base, int valid, int64_t rowbytes, char* lds, int wave) const {
    const i32x4 rs = rsrc(base);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int over = rows[i] >= valid ? rows[i] - (valid - 1) : 0;
      issue(rs, lds + (wave * kLoads + i) * 1024, voff[i] - uint32_t(over * rowbytes));
    }
  }
  // Tile whose rows come from several shards: every lane finds the shard of
  // its own row and loads from a 64-bit address.
  __device__ void load_gather(const KvShards& kv, const void* const* ptr, int64_t hoff, int key0, int keyL,
                              int64_t rowbytes, char* lds, int wave) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int key = min(key0 + rows[i], keyL);
      int r = 0;
      for (int b = 1; b < kv.W; ++b) r += kv.start[b] <= key ? 1 : 0;
      const uint32_t chunk = voff[i] - uint32_t(rows[i] * rowbytes);
      const uint64_t addr = reinterpret_cast<uint64_t>(ptr[r]) + uint64_t(hoff) +
                            uint64_t(key - kv.start[r]) * uint64_t(rowbytes) + chunk;
      const uint32_t m0 =
          __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds + (wave * kLoads + i) * 1024)));
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0), "v"(addr) : "memory", "m0");
    }
  }
  // Last tile of a ragged sequence: rows >= skv re-read row skv-1 (finite data;
  // those keys are masked to -inf, so they carry zero weight).
  __device__ void load_clamped(const uint16_t* hb, int tile, int skv, int64_t rowbytes, char* lds,
                               int wave) const {
    const char* base = reinterpret_cast<const char*>(hb) + int64_t(tile) * G::kBN * rowbytes;
    const i32x4 rs = rsrc(base);
    const int valid = skv - tile * G::kBN;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int over = rows[i] >= valid ? rows[i] - (valid - 1) : 0;
      issue(rs, lds + (wave * kLoads + i) * 1024, voff[i] - uint32_t(over * rowbytes));
    }
  }
};

// S^T of 32 keys (rows r0 .. r0+31 of an LDS K tile) against the wave's 64
// queries.  MASKED: accumulated onto `init` (-inf on keys past the end of the
// sequence, else 0); otherwise onto the inline constant 0.
template <int D, bool MASKED, int QB = Geo<D>::QB>
__device__ inline void qk32(f32x16 (&s)[QB], const char* kb, int r0, const bf16x8 (&qf)[QB][Geo<D>::kDC],
                            const f32x16& init, int col, int hf) {
  using G = Geo<D>;
  const int r = r0 + col;
  const char* rowp = kb + r * G::kRowB;
  const int sw = G::swz_k(r);
#pragma unroll
  for (int cc = 0; cc < G::kDC; ++cc) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(rowp + (((2 * cc + hf) ^ sw) << 4));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (cc > 0)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][cc], s[qb], 0, 0, 0);
      else if (MASKED)
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][cc], init, 0, 0, 0);
      else
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][cc], f32x16{}, 0, 0, 0);
    }
  }
}

// Accumulator init for keys key0 .. key0+31: -inf where key >= skv, else 0.
__device__ inline f32x16 tail_init(int key0, int skv, int hf) {
  f32x16 m;
#pragma unroll
  for (int r = 0; r < 16; ++r) m[r] = (key0 + 8 * (r >> 2) + 4 * hf + (r & 3) >= skv) ? -INFINITY : 0.f;
  return m;
}

// Softmax state of the wave's 32*QB query columns (both wave halves hold the same values).
template <int QB>
struct SoftState {
  float m_run[QB];  // reference maximum (log2 units) the probabilities are taken against
  float l_run[QB];  // this lane's partial sum of bf16 probabilities
};

// max(a, b, c) in one instruction (the compiler would otherwise build a
// max/max/max3 tree).  Operands are finite floats or -inf.
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Maximum of a 32-key block per query column (raw scores; the lane's 16
// keys, then the other wave half), in log2 units.
template <int QB>
__device__ inline void block_max(const f32x16 (&s)[QB], float (&mt)[QB], float c) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float m = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = max3(m, s[qb][r], s[qb][r + 1]);
    mt[qb] = other_half_max(m) * c;
  }
}

// Probabilities of a 32-key block as packed bf16 pairs: pw[qb][u][e] holds
// keys (8u + 2e, 8u + 2e + 1) of the lane's accumulator order; pw[qb][u][0..3]
// is the B operand of P*V MFMA u.  (Kept as plain 32-bit words: element
// extraction from a vector type under __builtin_bit_cast was miscompiled.)
template <int QB>
using PW = uint32_t[QB][2][4];

template <typename G, int QB = G::QB>
__device__ inline void rescale_o(f32x16 (&o)[G::kND][QB], const float (&alpha)[QB]) {
#pragma unroll
  for (int db = 0; db < G::kND; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha[qb];
}

// One 32-key step, issued in a fixed order: every MFMA is followed by its
// share of the VALU work and a scheduling fence, so the SIMD's in-order issue
// alternates matrix and vector instructions (an MFMA occupies the matrix pipe
// for 8 passes while the following VALU instructions issue), and LDS operand
// reads are issued two MFMA pairs ahead of their use.
//
// On entry `cur` holds S^T of the step's keys and `st` the reference maximum.
// Part A: MFMAs compute S^T of the next 32 keys into `nxt` (HAS_NEXT) while the
//         VALU turns `cur` into bf16 probabilities (fma, exp2, cvt) and adds
//         their row sums (v_dot2); then the block check (see above).
// Part B: MFMAs accumulate P*V while the VALU makes the first kEarly
//         probability words of `nxt` (HAS_NEXT), so that both parts carry
//         about the same vector work.  Those words and their row sums enter
//         the next step in `pbn` / `ln`; if that step's check raises the
//         reference, all of its words are made again.
template <int D>
__device__ inline bf16x8 k_frag(const char* kb, int r0, int cc, int col, int hf) {
  using G = Geo<D>;
  const int r = r0 + col;
  return *reinterpret_cast<const bf16x8*>(kb + r * G::kRowB + (((2 * cc + hf) ^ G::swz_k(r)) << 4));
}

// Work items spread evenly over the issue slots of a part: slot i of M runs
// items [i*N/M, (i+1)*N/M) of N.
template <int N, int M, typename F>
__device__ inline void slot_items(int i, F&& f) {
#pragma unroll
  for (int w = 0; w < N; ++w)
    if (w * M / N == i) f(w);
}

// Probability word pr of query block pq: exp2(c*s - m) of scores 2pr, 2pr+1,
// rounded to bf16 and packed, its two values added to the row sum ls.
template <int QB>
__device__ __attribute__((always_inline)) inline void prob_word(const f32x16 (&s)[QB], const SoftState<QB>& st,
                                                               float c, int pq, int pr, PW<QB>& pb,
                                                               float (&ls)[QB]) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[pq][2 * pr], c, -st.m_run[pq]));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[pq][2 * pr + 1], c, -st.m_run[pq]));
  const uint32_t word = pack_bf16x2(p0, p1);
  pb[pq][pr >> 2][pr & 3] = word;
  ls[pq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), ones, ls[pq], false);
}

template <typename G, bool HAS_NEXT, bool MASK_NEXT, bool PRE_NEXT, int QB = G::QB>
__device__ __attribute__((always_inline)) inline void step32(f32x16 (&cur)[QB], f32x16 (&nxt)[QB], SoftState<QB>& st,
                              PW<QB>& pb, PW<QB>& pbn, float (&lc)[QB], float (&ln)[QB],
                              f32x16 (&acc)[G::kND][QB], const bf16x8 (&qf)[QB][G::kDC],
                              const char* kb_next, int rk_next, const f32x16& init_next, const char* vb, int rv,
                              float c, int lane, int col, int hf, bf16x8 (&kpre)[kRA], const char* kb_after,
                              int rk_after) {
  constexpr int D = G::kD;
  constexpr int kA = QB * G::kDC;      // MFMA slots of part A: S^T of the next block
  constexpr int kB = 2 * QB * G::kND;  // MFMA slots of part B: P*V
  constexpr int kNV = 2 * G::kND;      // V^T fragments (MFMA pairs u, db) per step
  constexpr int kE = G::kEarly;        // words per query block made during the previous step's part B
  constexpr int kEOff = SPATTN_EOFF;   // part B slots before the first early word (S^T of the next block settles)
  static_assert(kA >= 2 * kRA && kB >= 2 * kRA, "prefetch slots");
  __builtin_amdgcn_sched_barrier(0);

  // V^T fragment reads (issued from the end of part A on)
  const int g16 = lane >> 4, j16 = lane & 15;
  auto vread = [&](int k) {  // V^T fragment of MFMA pair k = u * kND + db
    const int u = k / G::kND, db = k % G::kND;
    const int ra = rv + 16 * u + 4 * hf + (j16 >> 2);
    const int dcol = db * 32 + 16 * (g16 & 1) + 4 * (j16 & 3);
    const int ch = dcol >> 3, inb = (dcol & 7) * 2;
    const char* p0 = vb + ra * G::kVRowB + ((ch ^ G::swz_v(ra)) << 4) + inb;
    const char* p1 = vb + (ra + 8) * G::kVRowB + ((ch ^ G::swz_v(ra + 8)) << 4) + inb;
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 vf[kNV];

  // ---- part A: MFMA slot i computes (cc = i / QB, qb = i % QB) of S^T(next);
  // the VALU produces the remaining bf16 probability words of `cur` and
  // completes the block's row sums.
  float ls[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) ls[qb] = lc[qb];
  const int rk = rk_next + col;
  const char* krow = kb_next + rk * G::kRowB;
  const int ksw = G::swz_k(rk);
  auto kread = [&](int cc) {
    return *reinterpret_cast<const bf16x8*>(krow + (((2 * cc + hf) ^ ksw) << 4));
  };
  bf16x8 kf[G::kDC];
  if (HAS_NEXT) {
#pragma unroll
    for (int r = 0; r < kRA; ++r) kf[r] = G::kPrefetch ? kpre[r] : kread(r);
  }
#pragma unroll
  for (int i = 0; i < kA; ++i) {
    const int cc = i / QB, qb = i % QB;
    if (HAS_NEXT) {
      if (qb == 0 && cc + kRA < G::kDC) kf[cc + kRA] = kread(cc + kRA);
      if (cc > 0)
        nxt[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cc], qf[qb][cc], nxt[qb], 0, 0, 0);
      else if (MASK_NEXT)
        nxt[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cc], qf[qb][cc], init_next, 0, 0, 0);
      else
        nxt[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[cc], qf[qb][cc], f32x16{}, 0, 0, 0);
    }
    slot_items<(8 - kE) * QB, kA>(i, [&](int w) {  // the late words: query block w/(8-kE), pair kE + w%(8-kE)
      prob_word(cur, st, c, w / (8 - kE), kE + w % (8 - kE), pb, ls);
    });
#pragma unroll
    for (int r = 0; r < kRA; ++r)
      if (i == kA - 2 * kRA + r) vf[r] = vread(r);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the row sums in part A: an empty asm consuming them stops IR passes
  // from sinking the v_dot2 chain past the fences.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(ls[qb]));

  // ---- check before the block enters P*V: every probability is at most
  // 2^kTau unless some lane's sum over its 16 keys exceeds 2^kTau (an
  // overflow to inf included).  Rarely, when it does, the block's maximum is
  // taken, the reference of the columns whose maximum exceeds it by more than
  // kTau is raised (the others keep it, alpha = 1 exactly, so no row depends
  // on the other rows of the wave), O and l are rescaled and the block's
  // words redone from the scores, which are still in registers.
  {
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) need |= ls[qb] > kCheck;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      float mt[QB], alpha[QB];
      block_max(cur, mt, c);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = mt[qb] > st.m_run[qb] + kTau ? mt[qb] : st.m_run[qb];
        alpha[qb] = __builtin_amdgcn_exp2f(st.m_run[qb] - m_new);
        st.m_run[qb] = m_new;
        st.l_run[qb] *= alpha[qb];
        ls[qb] = 0.f;
      }
      rescale_o<G>(acc, alpha);
#pragma unroll
      for (int w = 0; w < 8 * QB; ++w) prob_word(cur, st, c, w >> 3, w & 7, pb, ls);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) st.l_run[qb] += ls[qb];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- part B: MFMA slot i accumulates pair k = i / QB (u, db) for qb = i % QB,
  // while the VALU makes the early words of the next block (its scores are
  // complete: part A's MFMAs have been issued) under the reference that the
  // check above has settled.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) ln[qb] = 0.f;
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const int k = i / QB, qb = i % QB;
    const int u = k / G::kND, db = k % G::kND;
    if (qb == 0 && k + kRA < kNV) vf[k + kRA] = vread(k + kRA);
    acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        vf[k], __builtin_bit_cast(bf16x8, u32x4{pb[qb][u][0], pb[qb][u][1], pb[qb][u][2], pb[qb][u][3]}),
        acc[db][qb], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < kRA; ++r)
      if (PRE_NEXT && i == kB - 2 * kRA + r) kpre[r] = k_frag<D>(kb_after, rk_after, r, col, hf);
    if (HAS_NEXT && i >= kEOff)
      slot_items<kE * QB, kB - kEOff>(i - kEOff, [&](int w) { prob_word(nxt, st, c, w / kE, w % kE, pbn, ln); });
    __builtin_amdgcn_sched_barrier(0);
  }
  if (HAS_NEXT && kE > 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(ln[qb]));
  }
}

// f(integral_constant<int, I>) for I = 0, 1, ...: a loop whose index is a
// compile-time constant (the steps of a tile use it as a template argument).
template <int... Is, typename Fn>
__device__ __attribute__((always_inline)) inline void for_each_index(std::integer_sequence<int, Is...>, Fn&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// s_waitcnt immediate: vmcnt(vm), expcnt untouched, lgkmcnt(0).
constexpr unsigned waitcnt_vm_lgkm0(unsigned vm) { return (vm & 0xFu) | ((vm >> 4) << 14) | (0x7u << 4); }

// Tile barrier: this wave's older LDS-direct loads (all but the newest
// PENDING) have landed and its LDS reads have completed, then all waves meet.
// A bare s_barrier is used (the workgroup fences of __syncthreads would also
// wait for the loads still meant to be in flight); the signal fences stop the
// compiler from moving LDS accesses across it.
template <unsigned PENDING>
__device__ inline void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(PENDING));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// K/V argument of the kernel: one gathered [skv, H, d] buffer each, or a
// table of per-rank shards (GV).
struct KvFlat {
  const uint16_t* k;
  const uint16_t* v;
};
template <bool GV>
using KvArg = typename std::conditional<GV, KvShards, KvFlat>::type;

// SPLIT: the keys are cut into nsplit ranges of whole tiles, one per
// work-group index; each work-group writes its float32 O normalised over its
// own keys and that range's LSE (opart [nsplit, sq, H, D], lse [nsplit, H, sq])
// for merge_kernel to combine.
template <int D, bool GV, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(const uint16_t* __restrict__ q, const KvArg<GV> kv,
                                                             uint16_t* __restrict__ o, float* __restrict__ lse,
                                                             int sq, int skv_all, int H, float c, int nqt,
                                                             int nsplit, float* __restrict__ opart) {
  using G = Geo<D>;
  constexpr int QB = G::QB, BM = G::BM, kBN = G::kBN, kSteps = G::kSteps;
  constexpr int kKSlots = G::kKSlots, kVSlots = G::kVSlots, kLead = G::kLead;
  static_assert(kKSlots * G::kTileB + kVSlots * G::kVTileB <= 160 * 1024, "K/V slots exceed the LDS");
  // K tile j lives in slot j mod kKSlots, V tile j in slot j mod kVSlots.
  __shared__ __attribute__((aligned(1024))) char smem[kKSlots * G::kTileB + kVSlots * G::kVTileB];
  char* const vbase = smem + kKSlots * G::kTileB;
  constexpr unsigned kBatch = G::kLoads + G::kVLoads;  // LDS-direct loads per wave per tile (K and V)

  // Head-major order: consecutive work-groups (spread over all XCDs) share a
  // head.
  const int L = blockIdx.x;
  int h, qt, sp = 0;
  if constexpr (SPLIT) {  // query tiles fastest, then key ranges, then heads
    qt = L % nqt;
    const int rest = L / nqt;
    sp = rest % nsplit;
    h = rest / nsplit;
  } else {
    h = L / nqt;
    qt = L - h * nqt;
  }
  // This work-group's keys [k0, k0 + skv): all of them, or key range sp.
  int k0 = 0, skv = skv_all;
  if constexpr (SPLIT) {
    const int tiles = (skv_all + kBN - 1) / kBN;
    k0 = int(int64_t(tiles) * sp / nsplit) * kBN;
    skv = min(skv_all, int(int64_t(tiles) * (sp + 1) / nsplit) * kBN) - k0;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int hf = lane >> 5;
  const int64_t rowstride = int64_t(H) * D;
  const int64_t rowbytes = rowstride * 2;
  const uint16_t* kh = nullptr;
  const uint16_t* vh = nullptr;
  if constexpr (!GV) {
    kh = kv.k + int64_t(k0) * rowstride + int64_t(h) * D;
    vh = kv.v + int64_t(k0) * rowstride + int64_t(h) * D;
  }
  const int nT = (skv + kBN - 1) / kBN;
  const bool ragged = (skv % kBN) != 0;

  TileLoader<G, false> kl;
  TileLoader<G, true> vl;
  kl.init(wave, lane, rowbytes);
  vl.init(wave, lane, rowbytes);
  // Tile indices are never negative: unsigned remainders (a mask for a power
  // of two slot count) instead of the signed sequence the compiler must emit
  // wherever it cannot prove the index non-negative.
  auto kslot = [&](int j) { return smem + (unsigned(j) % unsigned(kKSlots)) * G::kTileB; };
  auto vslot = [&](int j) { return vbase + (unsigned(j) % unsigned(kVSlots)) * G::kVTileB; };
  // Tile indices past the end are clamped: those loads land in slots no live
  // tile uses and keep every batch the same size for the vmcnt accounting.
  // Sharded K/V: a cursor per stream (K, V) follows the shard that holds the
  // tiles being loaded (tiles are requested in increasing order).  A tile
  // inside one shard is loaded like a gathered one from that shard's base; a
  // tile across shard boundaries (at most W-1 per stream) takes the per-lane
  // path.
  struct Cursor {
    int r;           // shard holding the last tile's first key
    int s0, s1;      // its token range [s0, s1)
    const char* p;   // its base pointer, offset to the stream's columns of head h
    int64_t off;     // that byte offset inside a token row
  };
  const int64_t hoff = int64_t(h) * D * 2;  // byte offset of head h inside a token row
  Cursor kcur{0, 0, 0, nullptr, 0}, vcur{0, 0, 0, nullptr, 0};
  if constexpr (GV) {
    kcur = Cursor{0, 0, int(kv.start[1]), static_cast<const char*>(kv.k[0]) + hoff, hoff};
    vcur = Cursor{0, 0, int(kv.start[1]), static_cast<const char*>(kv.v[0]) + hoff, hoff};
  }
  auto load_sharded = [&](const auto& ld, const void* const* ptr, Cursor& cu, int tile, char* lds) {
    if constexpr (GV) {
      const int key0 = tile * kBN;
      const int keyL = min(key0 + kBN, skv) - 1;
      while (key0 >= cu.s1) {  // wave-uniform; empty shards are stepped over
        ++cu.r;
        cu.s0 = cu.s1;
        cu.s1 = int(kv.start[cu.r + 1]);
        cu.p = static_cast<const char*>(ptr[cu.r]) + cu.off;
      }
      if (keyL < cu.s1) {
        const char* base = cu.p + int64_t(key0 - cu.s0) * rowbytes;
        if (keyL - key0 + 1 == kBN) ld.load_at(reinterpret_cast<uint64_t>(base), lds, wave);
        else ld.load_base(base, keyL - key0 + 1, rowbytes, lds, wave);
      } else {
        ld.load_gather(kv, ptr, cu.off, key0, keyL, rowbytes, lds, wave);
      }
    }
  };
  auto load_k = [&](int j) {
    const int tile = min(j, nT - 1);
    if constexpr (GV) load_sharded(kl, kv.k, kcur, tile, kslot(j));
    else if (ragged && tile == nT - 1) kl.load_clamped(kh, tile, skv, rowbytes, kslot(j), wave);
    else kl.load(kh, tile, rowbytes, kslot(j), wave);
  };
  auto load_v = [&](int j) {
    const int tile = min(j, nT - 1);
    if constexpr (GV) load_sharded(vl, kv.v, vcur, tile, vslot(j));
    else if (ragged && tile == nT - 1) vl.load_clamped(vh, tile, skv, rowbytes, vslot(j), wave);
    else vl.load(vh, tile, rowbytes, vslot(j), wave);
  };
  // Batch j = {K tile j+1, V tile j}; tile t needs batch t.
  auto load_batch = [&](int j) {
    load_k(j + 1);
    load_v(j);
  };
  load_k(0);
#pragma unroll
  for (int j = 0; j < kLead; ++j) load_batch(j);

  // Q fragments (B operand of S^T = K Q^T): lane holds 8 d-values of one query.
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

  f32x16 acc[G::kND][QB];
#pragma unroll
  for (int db = 0; db < G::kND; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][qb][r] = 0.f;
  SoftState<QB> st;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) st.l_run[qb] = 0.f;
  const f32x16 zero = {};

  f32x16 sa[QB], sb[QB];  // S^T of the current / next 32 keys
  PW<QB> pa, pn;          // probability words of the current / next block
  float la[QB], ln[QB];   // row sums of the words made early

  tile_barrier<0>();
  if (nT == 1) qk32<D, true>(sa, kslot(0), 0, qf, tail_init(0, skv, hf), col, hf);
  else qk32<D, false>(sa, kslot(0), 0, qf, zero, col, hf);
  block_max(sa, st.m_run, c);  // the first block's maximum is the first reference (every column has a key)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    la[qb] = 0.f;
#pragma unroll
    for (int pr = 0; pr < G::kEarly; ++pr) prob_word(sa, st, c, qb, pr, pa, la);
  }
  // K fragments of the next step's part A are read ahead, at the end of the
  // previous part B (that K tile has been resident since an earlier barrier).
  bf16x8 kpre[kRA];
  if constexpr (G::kPrefetch) {
#pragma unroll
    for (int r = 0; r < kRA; ++r) kpre[r] = k_frag<D>(kslot(0), 32, r, col, hf);
  }
  // Tile t (kBN keys) = kSteps 32-key steps.  At its top batch t (K t+1, V t)
  // has landed, batches t+1 .. t+kLead-1 may still be in flight, and batch
  // t+kLead is issued into the slots that tile t-1 released.
  // The kSteps 32-key steps of tile t.  Step s holds S^T of block s of the
  // tile, computes S^T of the next block (the following block of this tile,
  // or block 0 of tile t+1) and reads ahead the first K fragments of the block
  // after that.  LAST: t is the last tile; NEXT_LAST: tile t+1 is.
  auto tile_steps = [&](int t, auto last_, auto next_last_) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_)::value;
    constexpr bool NEXT_LAST = decltype(next_last_)::value;
    const char* vb = vslot(t);
    char* kc = kslot(t);
    char* kn = kslot(t + 1);
    auto one = [&](auto s_) __attribute__((always_inline)) {
      constexpr int s = decltype(s_)::value;
      constexpr bool next_in = s + 1 < kSteps, after_in = s + 2 < kSteps;
      constexpr bool HAS_NEXT = next_in || !LAST;
      constexpr bool MASK_NEXT = next_in ? LAST : NEXT_LAST;
      constexpr bool PRE_NEXT = G::kPrefetch && (after_in || !LAST);
      const char* kb_next = next_in ? kc : kn;
      const char* kb_after = after_in ? kc : kn;
      const int rk_next = next_in ? 32 * (s + 1) : 0;
      const int rk_after = after_in ? 32 * (s + 2) : 32 * (s + 2 - kSteps);
      const f32x16 init = MASK_NEXT ? tail_init(t * kBN + 32 * (s + 1), skv, hf) : zero;
      if constexpr (s % 2 == 0)
        step32<G, HAS_NEXT, MASK_NEXT, PRE_NEXT>(sa, sb, st, pa, pn, la, ln, acc, qf, kb_next, rk_next, init, vb, 32 * s, c,
                                                 lane, col, hf, kpre, kb_after, rk_after);
      else
        step32<G, HAS_NEXT, MASK_NEXT, PRE_NEXT>(sb, sa, st, pn, pa, ln, la, acc, qf, kb_next, rk_next, init, vb, 32 * s, c,
                                                 lane, col, hf, kpre, kb_after, rk_after);
      if constexpr (kSteps == 1) {  // one step per tile: the next tile's S^T moves to the current set
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sa[qb] = sb[qb];
          if constexpr (G::kEarly > 0) {  // and so do the early words
            la[qb] = ln[qb];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int e = 0; e < 4; ++e) pa[qb][u][e] = pn[qb][u][e];
          }
        }
      }
    };
    for_each_index(std::make_integer_sequence<int, kSteps>{}, one);
  };
  using F = std::false_type;
  using T = std::true_type;

  // Steady part: the tiles loaded (K t+kLead+1, V t+kLead) are full and not
  // the last one, so their addresses simply advance by one tile per step.
  const uint64_t tb = uint64_t(kBN) * uint64_t(rowbytes);
  uint64_t kaddr = reinterpret_cast<uint64_t>(kh) + uint64_t(kLead + 1) * tb;
  uint64_t vaddr = reinterpret_cast<uint64_t>(vh) + uint64_t(kLead) * tb;
  int t = 0;
  // Sharded K/V: tiles below kcross (vcross) lie inside the stream's current
  // shard and advance from kaddr (vaddr) like gathered ones; a tile at or
  // past it goes through the cursor, which also resets the address and the
  // crossing point.  The steady loop runs between crossing points, so its
  // body holds no cursor test at all.
  int kcross = 0, vcross = 0;
  const int tsteady = nT - 2 - kLead;  // steady tiles: t < tsteady
  for (;;) {
    // Steady run: with sharded K/V it stops before the first tile whose loads
    // reach a crossing point (K tile t+kLead+1 >= kcross or V tile t+kLead >=
    // vcross), so its body is the gathered one.
    int tend = tsteady;
    if constexpr (GV) tend = min(tend, min(kcross - kLead - 1, vcross - kLead));
    for (; t < tend; ++t) {
      tile_barrier<kBatch * (kLead - 1)>();
      kl.load_at(kaddr, kslot(t + kLead + 1), wave);
      vl.load_at(vaddr, vslot(t + kLead), wave);
      kaddr += tb;
      vaddr += tb;
      tile_steps(t, F{}, F{});
    }
    if constexpr (!GV) {
      break;
    } else {
      if (t >= tsteady) break;
      // A crossing tile: the cursor loads it and resets the stream's address
      // and crossing point.
      tile_barrier<kBatch * (kLead - 1)>();
      const int jk = t + kLead + 1, jv = t + kLead;
      if (jk >= kcross) {
        load_sharded(kl, kv.k, kcur, jk, kslot(jk));
        kaddr = reinterpret_cast<uint64_t>(kcur.p) + uint64_t(int64_t(jk) * kBN - kcur.s0) * uint64_t(rowbytes);
        kcross = kcur.s1 / kBN;
      } else {
        kl.load_at(kaddr, kslot(jk), wave);
      }
      if (jv >= vcross) {
        load_sharded(vl, kv.v, vcur, jv, vslot(jv));
        vaddr = reinterpret_cast<uint64_t>(vcur.p) + uint64_t(int64_t(jv) * kBN - vcur.s0) * uint64_t(rowbytes);
        vcross = vcur.s1 / kBN;
      } else {
        vl.load_at(vaddr, vslot(jv), wave);
      }
      kaddr += tb;
      vaddr += tb;
      tile_steps(t, F{}, F{});
      ++t;
    }
  }
  for (; t < nT - 2; ++t) {  // the next tile is not the last one: no masking
    tile_barrier<kBatch * (kLead - 1)>();
    load_batch(t + kLead);
    tile_steps(t, F{}, F{});
  }
  if (t == nT - 2) {  // the next tile is the last one
    tile_barrier<kBatch * (kLead - 1)>();
    load_batch(t + kLead);
    tile_steps(t, F{}, T{});
    ++t;
  }
  tile_barrier<kBatch * (kLead - 1)>();  // last tile: no further loads are issued
  tile_steps(t, T{}, F{});
  // No LDS-direct load may still be landing once this work-group's LDS is
  // handed to the next one.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  // Epilogue: O = O^T / l, rows past sq are dropped.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(st.l_run[qb]);
    const float inv = 1.f / lt;
    const int row = qrow0 + qb * 32 + col;
    if (SPLIT && row < sq) {
      float* dst = opart + (int64_t(sp) * sq + row) * rowstride + int64_t(h) * D;
#pragma unroll
      for (int db = 0; db < G::kND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          *reinterpret_cast<f32x4*>(dst + d0) = f32x4{acc[db][qb][4 * g] * inv, acc[db][qb][4 * g + 1] * inv,
                                                      acc[db][qb][4 * g + 2] * inv, acc[db][qb][4 * g + 3] * inv};
        }
      if (hf == 0) lse[(int64_t(sp) * H + h) * sq + row] = (st.m_run[qb] + __log2f(lt)) * kLn2;
    } else if (row < sq) {
      uint16_t* dst = o + int64_t(row) * rowstride + int64_t(h) * D;
#pragma unroll
      for (int db = 0; db < G::kND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          u32x2 w;
          w[0] = pack_bf16x2(acc[db][qb][4 * g] * inv, acc[db][qb][4 * g + 1] * inv);
          w[1] = pack_bf16x2(acc[db][qb][4 * g + 2] * inv, acc[db][qb][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + d0) = w;
        }
      if (lse && hf == 0) lse[int64_t(h) * sq + row] = (st.m_run[qb] + __log2f(lt)) * kLn2;
    }
  }
}

template <int D, bool GV, bool SPLIT = false>
hipError_t launch_d(const void* q, const KvArg<GV>& kv, void* o, float* lse, int64_t sq, int64_t skv, int H,
                    float c, hipStream_t stream, int nsplit = 1, float* opart = nullptr) {
  const int64_t nqt = (sq + Geo<D>::BM - 1) / Geo<D>::BM;
  const int64_t grid = nqt * H * nsplit;  // the host has checked grid * kThreads <= kMaxItems
  if (grid > kMaxItems / kThreads) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_bf16_kernel<D, GV, SPLIT>), dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), kv, static_cast<uint16_t*>(o), lse, int(sq), int(skv), H, c,
                     int(nqt), nsplit, opart);
  return hipGetLastError();
}

// Combines the nsplit partial results of a split launch: with m = max_s lse_s
// and w_s = exp(lse_s - m), O = sum_s w_s O_s / sum_s w_s (rounded once to
// bf16) and LSE = m + log(sum_s w_s), all in float32.  One thread per 4
// output columns of one (row, head).  HBM-bound: reads the partials once.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ opart, const float* __restrict__ lpart,
                                                    uint16_t* __restrict__ o, float* __restrict__ lse, int nsplit,
                                                    int64_t sq, int H, int D) {
  const int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int per = D / 4;
  const int64_t rh = g / per;
  if (rh >= sq * H) return;
  const int c4 = int(g - rh * per);
  const int64_t row = rh / H;
  const int h = int(rh - row * H);
  // Eight ranges' loads in flight at a time (the LSEs for the maximum, then
  // the partial pieces); the sum keeps the order of the ranges.
  auto lse_of = [&](int s) { return lpart[(int64_t(s) * H + h) * sq + row]; };
  auto part = [&](int s) {
    return *reinterpret_cast<const f32x4*>(opart + (int64_t(s) * sq * H + rh) * D + 4 * c4);
  };
  float m = -INFINITY;
  {
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      float l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) l[i] = lse_of(s + i);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, l[i]);
    }
    for (; s < nsplit; ++s) m = fmaxf(m, lse_of(s));
  }
  float ws = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](int s, const f32x4& x) __attribute__((always_inline)) {
    const float w = expf(lse_of(s) - m);
    ws += w;
    acc += w * x;
  };
  {
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      f32x4 x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = part(s + i);
#pragma unroll
      for (int i = 0; i < 8; ++i) add(s + i, x[i]);
    }
    for (; s < nsplit; ++s) add(s, part(s));
  }
  const float inv = 1.f / ws;
  u32x2 w2;
  w2[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w2[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(o + rh * D + 4 * c4) = w2;
  if (lse && c4 == 0) lse[int64_t(h) * sq + row] = m + logf(ws);
}

hipError_t launch_merge(const float* opart, const float* lpart, void* o, float* lse, int nsplit, int64_t sq, int H,
                        int D, hipStream_t stream) {
  const int64_t threads = sq * H * (D / 4);
  const int64_t blocks = (threads + 255) / 256;  // checked with the attention grid before either launch
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, opart, lpart,
                     static_cast<uint16_t*>(o), lse, nsplit, sq, H, D);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq, int64_t skv,
                        int H, float c, int nsplit, float* opart, float* lpart, hipStream_t stream) {
  // Both grids are checked before the first launch, so a call that does not
  // fit enqueues nothing.
  if (attn_bf16_items(sq, H, D, nsplit) > kMaxItems || attn_merge_items(sq, H, D) > kMaxItems)
    return hipErrorInvalidConfiguration;
  const KvFlat kv{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v)};
  hipError_t e = launch_d<D, false, true>(q, kv, o, lpart, sq, skv, H, c, stream, nsplit, opart);
  if (e != hipSuccess) return e;
  return launch_merge(opart, lpart, o, lse, nsplit, sq, H, D, stream);
}

}  // namespace

int64_t attn_bf16_items(int64_t sq, int H, int d, int nsplit) {
  if (d == 512) return attn_d512_items(sq, H, nsplit);
  if (d == 128) return attn_d128_items(sq, H, nsplit);
  const int bm = Geo<64>::BM;
  const __int128 n = __int128((sq + bm - 1) / bm) * H * nsplit * kThreads;
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

int64_t attn_merge_items(int64_t sq, int H, int d) {
  if (d == 512) return attn_d512_merge_items(sq, H);
  const __int128 n = (__int128(sq) * H * (d / 4) + 255) / 256 * 256;
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                            int64_t skv, int H, int d, float scale, hipStream_t stream) {
  if (sq > (int64_t(1) << 31) - 1024) return hipErrorInvalidValue;
  const float c = scale * 1.4426950408889634f;
  const KvFlat kv{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v)};
  if (d == 64) return launch_d<64, false>(q, kv, o, lse, sq, skv, H, c, stream);
  if (d == 512) return launch_attn_d512(q, k, v, o, lse, sq, skv, H, c, 1, nullptr, stream);
  return launch_attn_d128(q, k, v, o, lse, sq, skv, H, c, 1, nullptr, stream);
}

hipError_t launch_attn_bf16_gv(const void* q, const KvShards& kv, void* o, float* lse, int64_t sq, int H, int d,
                               float scale, hipStream_t stream) {
  if (sq > (int64_t(1) << 31) - 1024) return hipErrorInvalidValue;
  const float c = scale * 1.4426950408889634f;
  const int64_t skv = kv.start[kv.W];
  if (d == 64) return launch_d<64, true>(q, kv, o, lse, sq, skv, H, c, stream);
  return launch_attn_d128_gv(q, kv, o, lse, sq, H, c, stream);
}

namespace {

// Partials of shard_attn_fwd_split_noalloc.  Its contents are never read
// before being written: every partial row and LSE the merge reads is written
// by the attention kernel of the same call first, so nothing is cleared.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    // The array's host-side name is only a handle: the device address of this
    // device's copy comes from the runtime, with the device current.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_attn_bf16_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                                  int64_t skv, int H, int d, float scale, int nsplit, float* opart, float* lpart,
                                  hipStream_t stream) {
  if (sq > (int64_t(1) << 31) - 1024) return hipErrorInvalidValue;
  const float c = scale * 1.4426950408889634f;
  if (d == 64) return launch_split<64>(q, k, v, o, lse, sq, skv, H, c, nsplit, opart, lpart, stream);
  // Both grids are checked before the first launch, so a call that does not
  // fit enqueues nothing.
  if (attn_bf16_items(sq, H, d, nsplit) > kMaxItems || attn_merge_items(sq, H, d) > kMaxItems)
    return hipErrorInvalidConfiguration;
  if (d == 512) {
    hipError_t e = launch_attn_d512(q, k, v, o, lpart, sq, skv, H, c, nsplit, opart, stream);
    if (e != hipSuccess) return e;
    return launch_merge_d512(opart, lpart, o, lse, nsplit, sq, H, stream);
  }
  hipError_t e = launch_attn_d128(q, k, v, o, lpart, sq, skv, H, c, nsplit, opart, stream);
  if (e != hipSuccess) return e;
  return launch_merge(opart, lpart, o, lse, nsplit, sq, H, d, stream);
}

}  // namespace spattn

// bf16 attention at head size 128 on gfx950: a rank's local queries against
// the full K/V, the gathered sequence or the per-rank shards, and the same
// with the keys cut into ranges (float32 partials and their log-sum-exp).
//
// Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", section 机制一: the
// local shard provides Q, K/V span the whole sequence, no mask.  The scale
// 1/sqrt(d) is passed in (page "NPU HunyuanImage-3.0模型推理优化实践",
// 消除FA中scale的冗余计算).  The plain definition is O = softmax(Q K^T s) V per
// head; this kernel computes it with an online softmax over 32-key steps.
//
// Layout of the work (MI355X / CDNA4):
//  * A work-group has eight waves, two on each SIMD (the hardware places waves
//    w and w + 4 of a work-group on one SIMD), and takes 512 query rows of one
//    head: 64 per wave, as two 32-column blocks of the MFMA, with their Q
//    fragments (64 registers) and O accumulators (128) in VGPRs for the whole
//    key loop.  At two waves per SIMD a wave has 256 registers in all; the
//    compiler splits the register file evenly between VGPRs and AGPRs as soon
//    as a kernel uses AGPRs, so every MFMA here is inline asm on VGPRs.  Calls
//    whose 512-row grid would leave CUs idle run 32 rows per wave (256 per
//    work-group) instead; a row's arithmetic is the same in both.
//  * Each 32-key step of a wave has an MFMA phase (P*V of the previous step,
//    then the scores S^T = K Q^T of this step: 32 MFMAs of 32x32x16) and a
//    softmax phase (VALU).  Waves 4..7 run half a step behind waves 0..3, with
//    a work-group barrier after every phase, so on each SIMD one wave's
//    softmax issues while the other wave's MFMAs run.  The row sums add float32
//    probabilities with plain adds: v_dot2 (the bf16 dot product) cannot issue
//    beside another wave's MFMAs, which serialised the two phases.
//  * K and V stream through LDS in 32-key tiles (8 KiB each), a tile set (K
//    and V of one step) per slot, four slots, two sets in flight.  Waves 0..3
//    issue every set's LDS-direct loads during their softmax phase, which has
//    slack; the MFMA phase issues none.  Within a 1 KiB block, K rows are
//    stored as 8 rows x 8 chunks (chunk-major) and V rows as 4 rows with the
//    chunks of one 32-column group together, so that every operand read of a
//    step is one per-lane base plus an immediate offset and the eight lanes
//    that the LDS serves together read 128 contiguous bytes.
//  * Scores are computed transposed, so one lane holds 16 keys of one query
//    column: the softmax is lane-local except for one v_permlane32_swap when a
//    maximum is taken.  The probabilities are packed to bf16 in place, into
//    the registers of the scores they came from, in the layout of the B
//    operand of O^T += V^T P^T; the V^T operand comes from the row-major V
//    tile through the transposing read ds_read_b64_tr_b16, in the same key
//    order.
//  * Online softmax in float32, base 2, the scale folded into log2(e).  The
//    reference is the first step's maximum and is raised only when a step
//    would hold a probability above 2^8: a lane's row sum above 2^8 (or not
//    finite) sends the wave, rarely, through a path that recomputes the step's
//    scores from the K tile still in LDS, raises the reference of the columns
//    whose maximum exceeds it by more than 8, rescales their O and row sums,
//    and makes their probabilities again.  Columns that keep their reference
//    keep every value bit for bit, so a row's result does not depend on the
//    other rows of its wave, on sq or on the row's position.
//  * Work-groups are ordered head-major, so all XCDs work on one head at a
//    time and its K+V stays in the Infinity Cache.
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace spattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
// 32-query MFMA blocks per wave: 2 (512 query rows per work-group), or 1
// (256 rows) for calls whose 512-row grid would leave CUs idle.
constexpr int kCUs = 256;                  // compute units of an MI355X
constexpr int kBN = 32;                    // keys per step (one K tile, one V tile)
constexpr int kTileB = kBN * kD * 2;       // bytes of a K or V tile
constexpr int kSetB = 2 * kTileB;          // a slot: K tile, then V tile
constexpr int kLead = 2;                   // tile sets in flight ahead of the one in use
constexpr int kSlots = kLead + 2;          // a slot is free again two steps after its last reader
constexpr int kDC = kD / 16;               // k-steps of the score MFMA
constexpr int kND = kD / 32;               // 32-row blocks of O^T
constexpr float kTau = 8.0f;               // reference raise threshold (log2 units)
constexpr float kCheck = 256.0f;           // 2^kTau
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kSlots * kSetB <= 160 * 1024, "LDS");

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, nearest-even
  return __builtin_bit_cast(uint32_t, h);
}
// v_permlane32_swap with both operands x returns, in an order that depends on
// the wave half, the lane's own x and that of lane l ^ 32.
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// s_waitcnt immediate: vmcnt(vm), expcnt untouched, lgkmcnt(0).
constexpr unsigned waitcnt_vm_lgkm0(unsigned vm) { return (vm & 0xFu) | ((vm >> 4) << 14) | (0x7u << 4); }

// This wave's LDS-direct loads but the newest PENDING have landed and its LDS
// reads have completed; then all waves meet.  The signal fences keep the
// compiler from moving LDS accesses across.
template <unsigned PENDING>
__device__ inline void barrier_wait() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(PENDING));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Buffer resource of a tile: base address, raw (stride 0), 2 GiB range.
__device__ inline i32x4 rsrc(const char* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFF), 0x7FFFFFFF, 0x00020000};
}
// One LDS-direct 16-byte load per lane: bytes [voffset, voffset + 16) above
// the resource's base into LDS m0 + 16 lane.  As inline asm, so that the
// compiler does not treat the in-flight LDS writes as aliasing the LDS reads
// that follow; the kernel waits for them itself (vmcnt) before the barrier
// that publishes a tile set.
__device__ inline void lds_load(const i32x4& rs, uint32_t m0, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs)
               : "memory", "m0");
}
// The same from a per-lane 64-bit address (a tile that spans shards).
__device__ inline void lds_load_at(uint32_t m0, uint64_t addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0), "v"(addr) : "memory", "m0");
}

// MFMAs as inline asm with VGPR operands.  The compiler's hazard checks do
// not see inside them: a dependent chain may issue back to back; the last
// score MFMA of a step is followed by 16 wait states before the VALU reads
// its result (a 32x32x16 bf16 MFMA needs 12); the VALU writes operands well
// before the MFMAs of the next phase read them.
__device__ inline void mfma_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ inline void mfma_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ inline void mfma_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7" : "+v"(d) : "v"(a), "v"(b));
}

// Maximum of a step's scores per query column (both wave halves), log2 units.
template <int QB>
__device__ inline void step_max(const f32x16 (&s)[QB], float (&mt)[QB], float c) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float m = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) m = max3(m, s[qb][r], s[qb][r + 1]);
    mt[qb] = halves_max(m) * c;
  }
}

// Probability word pr of query block qb: exp2(c s - m) of scores 2pr, 2pr+1,
// packed to bf16 in place at s[qb][8(pr>>2) + (pr&3)] (the words of 16-key
// half u then fill s[qb][8u .. 8u+3], the B operand of its P*V MFMA); the two
// float32 probabilities are added to the lane's row sum.
template <int QB>
__device__ __attribute__((always_inline)) inline void prob_word(f32x16 (&s)[QB], const float (&m)[QB], float c,
                                                               int qb, int pr, float (&ls)[QB]) {
  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][2 * pr], c, -m[qb]));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][2 * pr + 1], c, -m[qb]));
  s[qb][8 * (pr >> 2) + (pr & 3)] = __builtin_bit_cast(float, pack_bf16x2(p0, p1));
  ls[qb] = (ls[qb] + p0) + p1;
}

struct KvFlat {
  const uint16_t* k;
  const uint16_t* v;
};
template <bool GV>
using KvArg = typename std::conditional<GV, KvShards, KvFlat>::type;

// GV: K/V given as per-rank shards.  SPLIT: the keys are cut into nsplit
// ranges of whole 32-key tiles; the work-group of range sp writes its float32
// O normalised over its own keys (opart [nsplit, sq, H, 128]) and the range's
// LSE (lse [nsplit, H, sq]).
template <int QB, bool GV, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_d128_kernel(const uint16_t* __restrict__ q, const KvArg<GV> kv,
                                                             uint16_t* __restrict__ o, float* __restrict__ lse,
                                                             int sq, int skv_all, int H, float c, int nqt,
                                                             int nsplit, float* __restrict__ opart) {
  constexpr int BM = kWaves * 32 * QB;  // query rows per work-group
  __shared__ __attribute__((aligned(1024))) char smem[kSlots * kSetB];
  const uint32_t sbase = uint32_t(reinterpret_cast<uintptr_t>(smem));

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
  int k0 = 0, skv = skv_all;  // this work-group's keys [k0, k0 + skv)
  if constexpr (SPLIT) {
    const int tiles = (skv_all + kBN - 1) / kBN;  // the host keeps nsplit <= tiles: no range is empty
    k0 = int(int64_t(tiles) * sp / nsplit) * kBN;
    skv = min(skv_all, int(int64_t(tiles) * (sp + 1) / nsplit) * kBN) - k0;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool late = wave >= 4;  // runs half a step behind; issues no tile loads
  const int col = lane & 31, hf = lane >> 5;
  const int64_t rowstride = int64_t(H) * kD;
  const uint32_t rowbytes = uint32_t(rowstride * 2);  // the host keeps 64 token rows below 2 GiB
  const int64_t hoff = int64_t(h) * kD * 2;           // byte offset of head h in a token row
  const char* kh = nullptr;
  const char* vh = nullptr;
  if constexpr (!GV) {
    kh = reinterpret_cast<const char*>(kv.k) + int64_t(k0) * rowbytes + hoff;
    vh = reinterpret_cast<const char*>(kv.v) + int64_t(k0) * rowbytes + hoff;
  }
  const int nT = (skv + kBN - 1) / kBN;
  const bool ragged = (skv % kBN) != 0;

  // ---- tile loads (waves 0..3): wave w fills 1 KiB blocks w and w + 4 of the
  // K tile and of the V tile.  K block b holds rows 8R .. 8R+7 (R = b>>1),
  // chunks 8(b&1) .. +8 at 16-byte position ((chunk & 7) ^ (R & 1)) * 8 +
  // (row & 7): the 16 lanes that the LDS serves together (rows 8R .. 8R+15 of
  // one chunk) then cover all 64 banks once.  V block b holds rows 4b .. 4b+3,
  // chunk 4g + e of row a at position 16g + 8(e>>1) + 2a + (e&1).  Block w + 4
  // is block w sixteen rows down.
  const int rowK = 8 * (wave >> 1) + (lane & 7);
  const int rowV = 4 * wave + ((lane >> 1) & 3);
  const uint32_t voffK =
      uint32_t(rowK) * rowbytes + uint32_t(8 * (wave & 1) + ((lane >> 3) ^ ((wave >> 1) & 1))) * 16u;
  const uint32_t voffV =
      uint32_t(rowV) * rowbytes + uint32_t(4 * (lane >> 4) + 2 * ((lane >> 3) & 1) + (lane & 1)) * 16u;
  // Sharded K/V: a cursor on the shard that holds the last tile's first key
  // (tiles are loaded in increasing order; empty shards are stepped over),
  // with that shard's K and V bases for head h, read from the kernel
  // arguments only when the cursor moves.
  int cr = 0, cs0 = 0, cs1 = 0;
  const char* ck = nullptr;
  const char* cv = nullptr;
  if constexpr (GV) {
    cs1 = int(kv.start[1]);
    ck = static_cast<const char*>(kv.k[0]) + hoff;
    cv = static_cast<const char*>(kv.v[0]) + hoff;
  }
  // Tile set j = K and V tile j into slot j mod kSlots; indices past the last
  // tile reload it (those sets land in slots no live step reads, and every
  // step issues the same number of loads for the vmcnt accounting).
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int tile = min(j, nT - 1);
    const uint32_t slot = sbase + (unsigned(j) % unsigned(kSlots)) * kSetB;
    const uint32_t m0[4] = {slot + wave * 1024, slot + (wave + 4) * 1024, slot + kTileB + wave * 1024,
                            slot + kTileB + (wave + 4) * 1024};
    const int rows[4] = {rowK, rowK + 16, rowV, rowV + 16};
    uint32_t vo[4] = {voffK, voffK + 16 * rowbytes, voffV, voffV + 16 * rowbytes};
    const int key0 = tile * kBN;
    const int valid = min(skv - key0, kBN);
    if (valid < kBN) {  // the last tile of a ragged range: rows past it re-read row valid-1 (masked keys)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (rows[i] >= valid) vo[i] -= uint32_t(rows[i] - (valid - 1)) * rowbytes;
    }
    const char* kb = kh;
    const char* vb = vh;
    if constexpr (GV) {
      while (key0 >= cs1) {  // wave-uniform
        ++cr;
        cs0 = cs1;
        cs1 = int(kv.start[cr + 1]);
        ck = static_cast<const char*>(kv.k[cr]) + hoff;
        cv = static_cast<const char*>(kv.v[cr]) + hoff;
      }
      if (key0 + valid > cs1) {  // the tile spans shards: every lane finds its row's shard
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = min(rows[i], valid - 1);
          const int key = key0 + row;
          int r = cr;
          while (r + 1 < kv.W && kv.start[r + 1] <= key) ++r;
          const void* base = i < 2 ? kv.k[r] : kv.v[r];
          const uint64_t addr = reinterpret_cast<uint64_t>(base) + uint64_t(hoff) +
                                uint64_t(key - kv.start[r]) * uint64_t(rowbytes) + (vo[i] - uint32_t(row) * rowbytes);
          lds_load_at(m0[i], addr);
        }
        return;
      }
      kb = ck + int64_t(key0 - cs0) * rowbytes;
      vb = cv + int64_t(key0 - cs0) * rowbytes;
    } else {
      kb += int64_t(key0) * rowbytes;
      vb += int64_t(key0) * rowbytes;
    }
    const i32x4 rk = rsrc(kb), rv = rsrc(vb);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_load(i < 2 ? rk : rv, m0[i], vo[i]);
  };
  // The LDS-direct loads are issued before the Q loads below: the compiler
  // counts only its own loads when it waits for Q, so ours must be older.
  if (!late) {
#pragma unroll
    for (int j = 0; j < kLead; ++j) issue(j);
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds 8 channels of one
  // query per k-step; rows past sq read zeros and are never written.
  bf16x8 qf[QB][kDC];
  const int qrow0 = qt * BM + wave * 32 * QB;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + col;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + int64_t(row) * rowstride + int64_t(h) * kD + 8 * hf);
#pragma unroll
    for (int cc = 0; cc < kDC; ++cc) {
      u32x4 t = row < sq ? src[2 * cc] : u32x4{0, 0, 0, 0};
      qf[qb][cc] = __builtin_bit_cast(bf16x8, t);
    }
  }
  f32x16 acc[kND][QB];  // O^T: [32-row block of the head dimension][query block]
#pragma unroll
  for (int db = 0; db < kND; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][qb][r] = 0.f;
  float m_run[QB], l_run[QB];  // reference (log2 units; both halves), the lane's partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = 0.f;
    l_run[qb] = 0.f;
  }
  f32x16 s[QB];  // a step's scores; then its probability words (in place)

  // Per-lane LDS operand bases: K row `col`, chunk 2cc + hf (position bit 0
  // flipped in odd 8-row groups); V^T rows
  // 16u + 4hf + (j16 >> 2) (+8 for the second read), columns 32db + 16(g16&1)
  // + 4(j16&3).
  const char* const lds = smem;
  const uint32_t kl = uint32_t((col >> 3) * 2048 + (hf ^ ((col >> 3) & 1)) * 128 + (col & 7) * 16);
  const int g16 = lane >> 4, j16 = lane & 15;
  const uint32_t vl = uint32_t(hf * 1024 + 128 * (g16 & 1) + 32 * (j16 >> 2) + 8 * (j16 & 3));
  auto kread = [&](const char* kb, int cc) {
    return *reinterpret_cast<const bf16x8*>(kb + (cc >> 2) * 1024 + (cc & 3) * 256);
  };
  auto vread = [&](const char* vb, int kk) {  // V^T operand of MFMA pair kk = u * kND + db
    const int u = kk / kND, db = kk % kND;
    const char* p0 = vb + u * 4096 + db * 256;
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 2048));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T of step t into s; with `pre`, the first K operand is already in kf[0].
  // Keys at or past skv are masked to -inf when MASK.
  auto scores = [&](int t, bool mask, bf16x8 (&kf)[2], bool pre) __attribute__((always_inline)) {
    const char* kb = lds + (unsigned(t) % unsigned(kSlots)) * kSetB + kl;
    if (!pre) kf[0] = kread(kb, 0);
#pragma unroll
    for (int cc = 0; cc < kDC; ++cc) {
      if (cc + 1 < kDC) kf[(cc + 1) & 1] = kread(kb, cc + 1);
      const bf16x8 a = kf[cc & 1];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (cc == 0) mfma_first(s[qb], a, qf[qb][cc]);
        else if (cc + 1 < kDC || qb + 1 < QB) mfma_acc(s[qb], a, qf[qb][cc]);
        else mfma_last(s[qb], a, qf[qb][cc]);  // its wait states also cover the other block's last MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (mask) {
      const int key_last = skv - t * kBN;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * hf + (r & 3) >= key_last) s[qb][r] = -INFINITY;
    }
  };
  // O^T += V^T P^T of step t (the words in s); with pre_k, the last pair also
  // reads the first K operand of step t + 1.
  auto pv = [&](int t, bf16x8 (&kf)[2], bool pre_k) __attribute__((always_inline)) {
    const char* vb = lds + (unsigned(t) % unsigned(kSlots)) * kSetB + kTileB + vl;
    const char* kbn = lds + (unsigned(t + 1) % unsigned(kSlots)) * kSetB + kl;
    bf16x8 vf[2];
    vf[0] = vread(vb, 0);
#pragma unroll
    for (int kk = 0; kk < 2 * kND; ++kk) {
      const int u = kk / kND, db = kk % kND;
      if (kk + 1 < 2 * kND) vf[(kk + 1) & 1] = vread(vb, kk + 1);
      else if (pre_k) kf[0] = kread(kbn, 0);
      const bf16x8 a = vf[kk & 1];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const f32x4 w = u == 0 ? __builtin_shufflevector(s[qb], s[qb], 0, 1, 2, 3)
                               : __builtin_shufflevector(s[qb], s[qb], 8, 9, 10, 11);
        mfma_acc(acc[db][qb], a, __builtin_bit_cast(bf16x8, w));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Softmax of step t: probability words and row sums.  FIRST: the step's
  // maximum becomes the reference (every column has a key in the first step).
  auto softmax = [&](int t, bool first, bool mask) __attribute__((always_inline)) {
    if (first) step_max(s, m_run, c);
    float ls[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ls[qb] = 0.f;
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) prob_word(s, m_run, c, qb, pr, ls);
    }
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) need |= ls[qb] > kCheck;  // an overflow to inf included
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      bf16x8 kf[2];
      scores(t, mask, kf, false);  // the words replaced the scores: form them again
      float mt[QB], alpha[QB];
      step_max(s, mt, c);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = mt[qb] > m_run[qb] + kTau ? mt[qb] : m_run[qb];
        alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha[qb];
        ls[qb] = 0.f;
      }
#pragma unroll
      for (int db = 0; db < kND; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[db][qb] *= alpha[qb];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) prob_word(s, m_run, c, qb, pr, ls);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += ls[qb];
  };

  // ---- phases.  Phase p ends with barrier p.  Waves 0..3: phase 2t is the
  // MFMA phase of step t (P*V of step t-1, scores of step t), phase 2t+1 its
  // softmax, which first issues tile set t + kLead.  Waves 4..7: phase 0 is
  // empty, then MFMA phase of step t = phase 2t+1, softmax = phase 2t+2.
  // Tile set j is read in the MFMA phases of steps j (K) and j+1 (V) and in
  // the softmax of step j (the rare recompute): free after barrier 2j+3.  It
  // is issued after barrier 2j-4 into a slot last used by set j-4 (free after
  // barrier 2j-5), and waves 0..3 wait for it before barrier 2j-1, which
  // precedes its first reader.  Both groups pass 2nT + 1 barriers.
  bf16x8 kf[2];
  barrier_wait<4 * (kLead - 1)>();  // tile set 0 has landed
  if (late) barrier_wait<63>();
  auto bar_m = [&]() __attribute__((always_inline)) { barrier_wait<63>(); };
  auto bar_v = [&]() __attribute__((always_inline)) {
    if (late) barrier_wait<63>();
    else barrier_wait<4 * (kLead - 1)>();  // tile set t+1 has landed
  };
  auto mphase = [&](int t, bool mask, bool pre) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (t > 0) pv(t - 1, kf, true);
    scores(t, mask, kf, pre);
    __builtin_amdgcn_s_setprio(0);
    bar_m();
  };
  auto vphase = [&](int t, bool first, bool mask) __attribute__((always_inline)) {
    if (!late) issue(t + kLead);
    softmax(t, first, mask);
  };

  mphase(0, nT == 1 && ragged, false);
  vphase(0, true, nT == 1 && ragged);
  if (!(late && nT == 1)) bar_v();
  int t = 1;
  for (; t < nT - 1; ++t) {
    mphase(t, false, true);
    vphase(t, false, false);
    bar_v();
  }
  if (t == nT - 1) {
    mphase(t, ragged, true);
    vphase(t, false, ragged);
    if (!late) bar_v();
  }
  __builtin_amdgcn_s_setprio(1);
  pv(nT - 1, kf, false);
  __builtin_amdgcn_s_setprio(0);
  // 16 wait states before the VALU reads the last MFMA results; no
  // LDS-direct load may still be landing when the LDS is handed on.
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  // ---- epilogue: O = O^T / l, rows past sq are dropped
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const float inv = 1.f / lt;
    const int row = qrow0 + qb * 32 + col;
    if (row >= sq) continue;
    const float lv = (m_run[qb] + __log2f(lt)) * kLn2;
    if constexpr (SPLIT) {
      float* dst = opart + (int64_t(sp) * sq + row) * rowstride + int64_t(h) * kD;
#pragma unroll
      for (int db = 0; db < kND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          *reinterpret_cast<f32x4*>(dst + d0) = f32x4{acc[db][qb][4 * g] * inv, acc[db][qb][4 * g + 1] * inv,
                                                      acc[db][qb][4 * g + 2] * inv, acc[db][qb][4 * g + 3] * inv};
        }
      if (hf == 0) lse[(int64_t(sp) * H + h) * sq + row] = lv;
    } else {
      uint16_t* dst = o + int64_t(row) * rowstride + int64_t(h) * kD;
#pragma unroll
      for (int db = 0; db < kND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * hf;
          *reinterpret_cast<u32x2*>(dst + d0) =
              u32x2{pack_bf16x2(acc[db][qb][4 * g] * inv, acc[db][qb][4 * g + 1] * inv),
                    pack_bf16x2(acc[db][qb][4 * g + 2] * inv, acc[db][qb][4 * g + 3] * inv)};
        }
      if (lse && hf == 0) lse[int64_t(h) * sq + row] = lv;
    }
  }
}

// One 32-query block per wave when the 512-row grid would not give every CU
// a work-group; a row's arithmetic is the same either way.
int blocks_per_wave(int64_t sq, int H, int nsplit) {
  const int64_t wg2 = (sq + kWaves * 64 - 1) / (kWaves * 64) * H * nsplit;
  return wg2 < kCUs ? 1 : 2;
}

template <int QB, bool GV, bool SPLIT>
hipError_t launch_qb(const void* q, const KvArg<GV>& kv, void* o, float* lse, int64_t sq, int64_t skv, int H,
                     float c, int nsplit, float* opart, hipStream_t stream) {
  constexpr int BM = kWaves * 32 * QB;
  const int64_t nqt = (sq + BM - 1) / BM;
  const int64_t grid = nqt * H * nsplit;  // the host has checked grid * kThreads <= kMaxItems
  if (grid > kMaxItems / kThreads) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_d128_kernel<QB, GV, SPLIT>), dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), kv, static_cast<uint16_t*>(o), lse, int(sq), int(skv), H, c,
                     int(nqt), nsplit, opart);
  return hipGetLastError();
}

template <bool GV, bool SPLIT>
hipError_t launch(const void* q, const KvArg<GV>& kv, void* o, float* lse, int64_t sq, int64_t skv, int H, float c,
                  int nsplit, float* opart, hipStream_t stream) {
  if (sq < 1) return hipSuccess;
  if (blocks_per_wave(sq, H, nsplit) == 1)
    return launch_qb<1, GV, SPLIT>(q, kv, o, lse, sq, skv, H, c, nsplit, opart, stream);
  return launch_qb<2, GV, SPLIT>(q, kv, o, lse, sq, skv, H, c, nsplit, opart, stream);
}

}  // namespace

int64_t attn_d128_items(int64_t sq, int H, int nsplit) {
  const int64_t bm = kWaves * 32 * blocks_per_wave(sq, H, nsplit);
  const __int128 n = __int128((sq + bm - 1) / bm) * H * nsplit * kThreads;
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

hipError_t launch_attn_d128(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                            int64_t skv, int H, float c, int nsplit, float* opart, hipStream_t stream) {
  const KvFlat kv{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v)};
  if (opart) return launch<false, true>(q, kv, o, lse, sq, skv, H, c, nsplit, opart, stream);
  return launch<false, false>(q, kv, o, lse, sq, skv, H, c, 1, nullptr, stream);
}

hipError_t launch_attn_d128_gv(const void* q, const KvShards& kv, void* o, float* lse, int64_t sq, int H, float c,
                               hipStream_t stream) {
  return launch<true, false>(q, kv, o, lse, sq, kv.start[kv.W], H, c, 1, nullptr, stream);
}

}  // namespace spattn

// Attention at head size 512 (the VAE's single-head attention over C = 512
// channels) with every score formed once.
//
// Page "NPU HunyuanImage-3.0模型推理优化实践", section VAE并行优化: each process
// attends its block's queries to the keys and values of all blocks, one head
// over all channels, scale 1/sqrt(C).  The plain definition is
// O = softmax(Q K^T / sqrt(d)) V per head; this kernel computes it with an
// online softmax over 32-key tiles.
//
// Why a kernel of its own.  At head size 512 a wave cannot hold both the Q
// fragments of its 32 queries (128 registers) and the O accumulators of all
// 512 output columns (256 registers) next to the scores, the operands in
// flight and the softmax.  Instead, a work-group of 4 waves takes 128 queries:
//   * wave w forms the scores S^T = K Q^T of query block w (32 queries) over
//     the tile's 32 keys and their softmax, and writes the bf16 probabilities
//     (already in the B-operand layout of the P*V MFMA) to LDS;
//   * wave w accumulates output columns [128w, 128w + 128) for all four
//     query blocks, reading P from LDS and V^T from the tile.
// So every score is formed once, a lane holds 128 Q registers (VGPRs) and 256
// accumulators (4 blocks x 4 column tiles x 16, all the AGPRs), and each K
// operand read from LDS feeds one MFMA, each V^T operand four.  Per 32 keys
// and 128 queries: 256 MFMAs of 32x32x16 against 192 KiB of LDS operand reads
// (K 128, P 32, V 32) and 64 KiB of tile writes.
//
// Software pipeline, one barrier per tile.  Step t turns the scores of tile
// t (formed in step t-1) into probabilities while the matrix pipe runs two
// streams: the scores of tile t+1 and P*V of tile t-1 (whose probabilities
// are in LDS since the previous barrier).  The step is written out by hand,
// one score MFMA and one P*V MFMA at a time, each followed by the few loads,
// LDS reads and softmax instructions that can issue while it runs (in-order
// issue would otherwise hold them behind a burst of MFMAs, or the MFMAs behind
// a burst of tile loads).  The probabilities of tile t go to the second of two
// P buffers; then the one barrier.  K tile t+2 loads during step t into the
// slot of K tile t and V tile t into that of V tile t-2.  The first step's
// P*V of "tile -1" multiplies zero probabilities with finite values and the
// last step's scores of "tile nT" read a slot nobody writes then: both add
// nothing and keep the step free of branches (1.6% more MFMAs for 64 tiles).
// Row sums add the two bf16 halves of each probability word as float32 (the
// weights P*V uses, exactly; v_dot2 would wait for the wave's MFMAs).
//
// Softmax: float32, base 2 with the scale folded into log2(e).  The O
// accumulators are never rescaled (as C++ on AGPR values, a rescale would make
// the compiler keep VGPR copies of all 256 across the loop): each query's
// reference is its first tile's maximum plus 40, so probabilities start at or
// below 2^-40 (far above the underflow of any key within 86 of the maximum,
// all that can matter) and may then grow to 2^64 before the float32 sums come
// anywhere near overflow.  Only a score that tops its query's first-tile
// maximum by more than 104 (log2 units, about 72 nats) needs a larger
// reference: the work-group then restarts its keys with the raised reference.
// Each restart is caused by a later tile than the previous one, so there are
// at most as many restarts as tiles.
//
// K and V tiles stream through LDS with LDS-direct loads (no VGPR staging).
// LDS rows are padded (K 1040 bytes, V 1088) rather than
// swizzled, so every operand read is one per-lane base plus an immediate
// offset; the padding spreads the rows that one read touches over the banks.
#include <stdint.h>

#include "internal.h"

namespace spattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 512;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;            // query rows per work-group
constexpr int kBN = 32;                     // keys per tile
constexpr int kRowB = kD * 2;               // bytes per K / V row in global memory
constexpr int kKS = kRowB + 16;             // LDS stride of a K row
constexpr int kVS = kRowB + 64;             // LDS stride of a V row
constexpr int kDC = kD / 16;                // k-steps of the score MFMA
constexpr int kColsW = kD / kWaves;         // output columns per wave
constexpr int kCT = kColsW / 32;            // 32-column O^T tiles per wave and query block
constexpr int kRowsW = kBN / kWaves;        // tile rows each wave loads
constexpr int kKRA = 2;                     // K operands read ahead of their MFMA
constexpr float kOff = 40.0f;               // reference above a query's first-tile maximum (log2 units)
constexpr float kCheck = 18446744073709551616.0f;  // 2^64: a lane's sum of 16 probabilities above it restarts
constexpr float kLn2 = 0.69314718055994531f;

// LDS: two K slots, two V slots, the probabilities of the four query blocks,
// the restart flags of the current tile and the row sums (epilogue).
constexpr int kKSlotB = kBN * kKS;
constexpr int kVSlotB = kBN * kVS;
constexpr int kOffK = 0;
constexpr int kOffV = 2 * kKSlotB;
constexpr int kPB = kWaves * 2 * 64 * 16;             // probabilities of one tile: [block][u][lane] 16 bytes
constexpr int kOffP = kOffV + 2 * kVSlotB;             // two tiles' probabilities
constexpr int kOffF = kOffP + 2 * kPB;                 // int flag[tile & 1][block]
constexpr int kOffL = kOffF + 32;                      // float lsum[block][32]
constexpr int kSmem = kOffL + kWaves * 32 * 4;
static_assert(kSmem <= 160 * 1024, "LDS");

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, nearest-even
  return __builtin_bit_cast(uint32_t, h);
}
// v_permlane32_swap with both operands x returns, in some order that depends
// on the wave half, the lane's own x and that of lane l ^ 32: the sum and the
// maximum of the pair are the same in both halves.
__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// s_waitcnt immediate: vmcnt(vm), expcnt untouched, lgkmcnt(0).
constexpr unsigned waitcnt_vm_lgkm0(unsigned vm) { return (vm & 0xFu) | ((vm >> 4) << 14) | (0x7u << 4); }

// This wave's older LDS-direct loads (all but the newest PENDING) have landed
// and its LDS accesses have completed; then all waves meet.  The signal
// fences keep the compiler from moving LDS accesses across.
template <unsigned PENDING>
__device__ inline void barrier_wait() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(PENDING));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One LDS-direct 16-byte load per lane: bytes [16 lane, 16 lane + 16) of the
// global row at rsrc base + soffset into LDS row address m0 (both
// wave-uniform).  Inline asm keeps the compiler from treating the in-flight
// LDS writes as aliasing the LDS reads that follow; the kernel waits for them
// itself (vmcnt) before the barrier that publishes a tile.
__device__ inline void lds_load(const i32x4& rs, uint32_t m0, uint32_t soffset, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rs), "s"(soffset)
               : "memory", "m0");
}

// Buffer resource of a tile: base address, raw (stride 0), 2 GiB range.
__device__ inline i32x4 rsrc(const char* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFF), 0x7FFFFFFF, 0x00020000};
}

// Score MFMAs.  The O accumulators take all 256 AGPRs (the P*V MFMAs are
// compiler builtins in AGPR form), so the scores must stay in VGPRs: these
// three are written as inline asm with VGPR operands.  The compiler's hazard
// checks do not see inside them, so they carry their own: the chain's first
// MFMA starts from the inline constant 0 (no register written by another
// unit), dependent MFMAs of one chain may issue back to back, and the last is
// followed by 16 wait states before anything can read its result (a 32x32x16
// bf16 MFMA needs 12 before a VALU read).
__device__ inline f32x16 mfma_s_first(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ inline void mfma_s(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ inline void mfma_s_last(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7" : "+v"(d) : "v"(a), "v"(b));
}

// Maximum of the block per query column (both wave halves), in log2 units.
__device__ inline float col_max(const f32x16& s, float c) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
  return halves_max(m) * c;
}

// SPLIT: the keys are cut into nsplit ranges of whole tiles; work-group
// (range, query tile, head) writes its float32 O normalised over its own keys
// as one 128 x 512 block (opart: [nsplit, H, query tiles] blocks, the layout
// of the epilogue) and that range's LSE (lse [nsplit, H, sq]).
// Ranges vary fastest over the work-groups, so with 8 ranges the work-groups
// of one range share an XCD (and its L2) when blocks are dealt round-robin.
template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_d512_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             uint16_t* __restrict__ o, float* __restrict__ lse,
                                                             int sq, int skv_all, int H, float c, int nqt,
                                                             int nsplit, float* __restrict__ opart) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  const uint32_t sbase = uint32_t(reinterpret_cast<uintptr_t>(smem));

  const int L = blockIdx.x;
  int qt, h, sp = 0;
  if constexpr (SPLIT) {
    sp = L % nsplit;
    const int rest = L / nsplit;
    qt = rest % nqt;
    h = rest / nqt;
  } else {
    h = L / nqt;
    qt = L - h * nqt;
  }
  int k0 = 0, skv = skv_all;
  if constexpr (SPLIT) {
    const int tiles = (skv_all + kBN - 1) / kBN;
    k0 = int(int64_t(tiles) * sp / nsplit) * kBN;
    skv = min(skv_all, int(int64_t(tiles) * (sp + 1) / nsplit) * kBN) - k0;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;
  const int64_t rowstride = int64_t(H) * kD;
  const uint32_t rowbytes = uint32_t(rowstride * 2);  // the host keeps 32 rows below 2 GiB
  const char* kh = reinterpret_cast<const char*>(k + int64_t(k0) * rowstride + int64_t(h) * kD);
  const char* vh = reinterpret_cast<const char*>(v + int64_t(k0) * rowstride + int64_t(h) * kD);
  const int nT = (skv + kBN - 1) / kBN;
  const int64_t tb = int64_t(kBN) * rowbytes;
  const uint32_t lane16 = uint32_t(lane) * 16;

  auto kslot = [&](int j) { return sbase + kOffK + (unsigned(j) & 1u) * kKSlotB; };
  auto vslot = [&](int j) { return sbase + kOffV + (unsigned(j) & 1u) * kVSlotB; };
  // This wave's rows [8w, 8w + 8) of K tile j or V tile j; rows past the
  // range re-read its last row (finite data for keys that are masked).
  auto load_rows = [&](const char* base, int j, uint32_t slot, int stride) __attribute__((always_inline)) {
    const i32x4 rs = rsrc(base + int64_t(j) * tb);
    const int valid = min(skv - j * kBN, kBN);
#pragma unroll
    for (int jj = 0; jj < kRowsW; ++jj) {
      const int r = wave * kRowsW + jj;
      lds_load(rs, slot + r * stride, uint32_t(r < valid ? r : valid - 1) * rowbytes, lane16);
    }
  };
  // Row jj of this wave's part of K tile j / V tile j.
  auto load_row = [&](const char* base, int j, uint32_t slot, int stride, int jj) __attribute__((always_inline)) {
    const i32x4 rs = rsrc(base + int64_t(j) * tb);
    const int valid = min(skv - j * kBN, kBN);
    const int r = wave * kRowsW + jj;
    lds_load(rs, slot + r * stride, uint32_t(r < valid ? r : valid - 1) * rowbytes, lane16);
  };
  load_rows(kh, 0, kslot(0), kKS);

  // Q fragments of this wave's query block (B operand of S^T = K Q^T): lane
  // holds 8 channels of query `col` per k-step.  Rows past sq repeat row
  // sq-1: their columns are computed and never written to o (a split launch
  // writes them into its partial block, which the merge skips).
  bf16x8 qf[kDC];
  {
    const int row = min(qt * kBM + wave * 32 + col, sq - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(q + int64_t(row) * rowstride + int64_t(h) * kD + 8 * hf);
#pragma unroll
    for (int cc = 0; cc < kDC; ++cc) qf[cc] = __builtin_bit_cast(bf16x8, src[2 * cc]);
  }

  // O^T accumulators: [query block][column tile of this wave].  Every value
  // they take is an MFMA result (zero included), so they stay in AGPRs.
  const bf16x8 zb = {};
  f32x16 acc[kWaves][kCT];
#pragma unroll
  for (int b = 0; b < kWaves; ++b)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) acc[b][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zb, zb, f32x16{}, 0, 0, 0);
  float m_run = -INFINITY;  // this wave's query block: reference (log2 units), the same in both halves
  float l_run = 0.f;        // the lane's partial row sum

  const char* lds = reinterpret_cast<const char*>(smem);
  // Per-lane operand bases: K row `col`, chunk hf (+32 bytes per k-step);
  // V^T rows 4hf + j16/4 (+16 rows per MFMA u, +8 for the second half) and
  // channels 128w + 16(g16 & 1) + 4(j16 & 3) (+32 per column tile).
  const int g16 = lane >> 4, j16 = lane & 15;
  const uint32_t koff = uint32_t(col * kKS + hf * 16);
  const uint32_t voff = uint32_t((4 * hf + (j16 >> 2)) * kVS + (wave * kColsW + 16 * (g16 & 1) + 4 * (j16 & 3)) * 2);
  auto pread = [&](int t, int b, int u) {
    return *reinterpret_cast<const bf16x8*>(smem + kOffP + (unsigned(t) & 1u) * kPB + ((b * 2 + u) * 64 + lane) * 16);
  };
  // V^T operand of MFMA u, column tile ct of tile t: channels [32 ct, 32 ct + 32)
  // of this wave x the 16 keys of u, in the key order of the probability words.
  auto vread = [&](int t, int u, int ct) {
    const char* p0 = lds + (vslot(t) - sbase) + voff + u * 16 * kVS + ct * 64;
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * kVS));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // O^T[cols of this wave][queries of block b] += V^T P^T, MFMA group g (16-key
  // half u = g / kCT, column tile ct = g % kCT) of tile t; pf holds P(u).
  auto pv_group = [&](int t, int g, bf16x8 (&pf)[kWaves]) __attribute__((always_inline)) {
    const int u = g / kCT, ct = g % kCT;
    if (ct == 0) {
#pragma unroll
      for (int b = 0; b < kWaves; ++b) pf[b] = pread(t, b, u);
    }
    const bf16x8 vc = vread(t, u, ct);
#pragma unroll
    for (int b = 0; b < kWaves; ++b)
      acc[b][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, pf[b], acc[b][ct], 0, 0, 0);
  };
  constexpr int kGroups = 2 * kCT;  // MFMA groups of a tile's P*V

  // Scores S^T of this wave's block over the 32 keys of tile j, in kGroups
  // slices of 4 MFMAs; the K operands are read kKRA MFMAs ahead.
  auto kbase = [&](int j) { return lds + (kslot(j) - sbase) + koff; };
  auto kread = [&](const char* kb, int cc) { return *reinterpret_cast<const bf16x8*>(kb + 32 * cc); };
  auto s_slice = [&](f32x16& d, const char* kb, bf16x8 (&kf)[kKRA], int g) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cc = 4 * g + i;
      const bf16x8 a = kf[cc % kKRA];
      if (cc + kKRA < kDC) kf[cc % kKRA] = kread(kb, cc + kKRA);
      if (cc == 0) d = mfma_s_first(a, qf[0]);
      else if (cc + 1 < kDC) mfma_s(d, a, qf[cc]);
      else mfma_s_last(d, a, qf[cc]);
    }
  };
  auto scores_alone = [&](f32x16& d, int j) __attribute__((always_inline)) {
    const char* kb = kbase(j);
    bf16x8 kf[kKRA];
#pragma unroll
    for (int i = 0; i < kKRA; ++i) kf[i] = kread(kb, i);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      s_slice(d, kb, kf, g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The first step's P*V of "tile -1" multiplies zero probabilities (this
  // wave's block in the second P buffer) with finite values (V tile 0 loaded
  // into the second V slot): it adds exact zeros.
  auto zero_p1 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<u32x4*>(smem + kOffP + kPB + ((wave * 2 + u) * 64 + lane) * 16) = u32x4{0u, 0u, 0u, 0u};
  };
  // Prologue: K tiles 0 and 1, the scores of tile 0.
  if (nT > 1) load_rows(kh, 1, kslot(1), kKS);
  load_rows(vh, 0, vslot(1), kVS);
  zero_p1();
  barrier_wait<0>();  // K tiles 0 and 1 and V tile 0 have landed (each wave loads 8 rows of each); zeros visible
  f32x16 s;
  scores_alone(s, 0);

  // Step t: the softmax of tile t (its scores are in s) under two MFMA
  // streams, the scores of tile t+1 and P*V of tile t-1, a slice of each per
  // pair of probability words; then the probabilities of tile t and the raise
  // flag to LDS and one barrier.  K tile t+2 loads into the slot of K tile t
  // (read during step t-1) and V tile t into that of V tile t-2 (read during
  // step t-1); both land before the barrier.
  for (int t = 0; t < nT; ++t) {
    {
      const int key_last = skv - t * kBN;  // keys at or past this index are masked
      if (key_last < kBN) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * hf + (r & 3) >= key_last) s[r] = -INFINITY;
      }
    }
    if (t == 0) m_run = fmaxf(m_run, col_max(s, c) + kOff);  // every column has a key in the first tile
    uint32_t w[2][4];
    float ls = 0.f, mx = -INFINITY;
    f32x16 sn;
    __builtin_amdgcn_sched_barrier(0);
    {
      const char* kb = kbase(t + 1);
      const int jk = min(t + 2, nT - 1);  // past the last tile: the last again, into a slot nobody reads
      bf16x8 kf[kKRA], pf[kWaves];
#pragma unroll
      for (int i = 0; i < kKRA; ++i) kf[i] = kread(kb, i);
#pragma unroll
      for (int b = 0; b < kWaves; ++b) pf[b] = pread(t - 1, b, 0);
      bf16x8 vcur = vread(t - 1, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int ct = g % kCT;
        const int gn = g + 1, un = gn / kCT, ctn = gn % kCT;
        bf16x8 vnext = vcur;
        auto smf = [&](int i) __attribute__((always_inline)) {
          const int cc = 4 * g + i;
          const bf16x8 a = kf[cc % kKRA];
          if (cc + kKRA < kDC) kf[cc % kKRA] = kread(kb, cc + kKRA);
          if (cc == 0) sn = mfma_s_first(a, qf[0]);
          else if (cc + 1 < kDC) mfma_s(sn, a, qf[cc]);
          else mfma_s_last(sn, a, qf[cc]);
        };
        auto pvf = [&](int b) __attribute__((always_inline)) {
          acc[b][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, pf[b], acc[b][ct], 0, 0, 0);
          if (gn < kGroups && ctn == 0) pf[b] = pread(t - 1, b, un);
        };
        const int pr = g;
        float p0, p1;
        uint32_t wd;
        smf(0);
        load_row(vh, t, vslot(t), kVS, g);
        __builtin_amdgcn_sched_barrier(0);
        pvf(0);
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[2 * pr], s[2 * pr + 1]));
        p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * pr], c, -m_run));
        __builtin_amdgcn_sched_barrier(0);
        smf(1);
        load_row(kh, jk, kslot(t + 2), kKS, g);
        __builtin_amdgcn_sched_barrier(0);
        pvf(1);
        p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * pr + 1], c, -m_run));
        __builtin_amdgcn_sched_barrier(0);
        smf(2);
        if (gn < kGroups) vnext = vread(t - 1, un, ctn);
        __builtin_amdgcn_sched_barrier(0);
        pvf(2);
        wd = pack_bf16x2(p0, p1);
        w[pr >> 2][pr & 3] = wd;
        __builtin_amdgcn_sched_barrier(0);
        smf(3);
        __builtin_amdgcn_sched_barrier(0);
        pvf(3);
        ls = (ls + __uint_as_float(wd << 16)) + __uint_as_float(wd & 0xFFFF0000u);
        __builtin_amdgcn_sched_barrier(0);
        vcur = vnext;
      }
    }
    asm volatile("" : "+v"(ls));
    const bool over = __builtin_amdgcn_ballot_w64(ls > kCheck) != 0;
    if (over) m_run = fmaxf(m_run, halves_max(mx) * c + kOff);
    l_run += ls;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<u32x4*>(smem + kOffP + (unsigned(t) & 1u) * kPB + ((wave * 2 + u) * 64 + lane) * 16) =
          u32x4{w[u][0], w[u][1], w[u][2], w[u][3]};
    if (lane == 0) *reinterpret_cast<int*>(smem + kOffF + (unsigned(t) & 1u) * 16 + wave * 4) = over ? 1 : 0;
    barrier_wait<0>();  // tile t's probabilities and flags visible; K tile t+2 and V tile t have landed

    // ---- restart (rare): some query's reference was raised; every wave
    // starts over from the first tile (the raised references carry over)
    {
      const i32x4 fl = *reinterpret_cast<const i32x4*>(smem + kOffF + (unsigned(t) & 1u) * 16);
      if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]) != 0) {
#pragma unroll
        for (int b = 0; b < kWaves; ++b)
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct)
            acc[b][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zb, zb, f32x16{}, 0, 0, 0);
        l_run = 0.f;
        zero_p1();
        load_rows(kh, 0, kslot(0), kKS);
        if (nT > 1) load_rows(kh, 1, kslot(1), kKS);
        barrier_wait<0>();  // K tiles 0 and 1 have landed and every wave has read the flags
        scores_alone(s, 0);
        t = -1;
        continue;
      }
    }
    s = sn;
  }
  // ---- P*V of the last tile
  {
    bf16x8 pf[kWaves];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      pv_group(nT - 1, g, pf);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: row sums of every block through LDS, O = O^T / l
  const float l_tot = halves_sum(l_run);
  if (hf == 0) *reinterpret_cast<float*>(smem + kOffL + (wave * 32 + col) * 4) = l_tot;
  {
    const int row = qt * kBM + wave * 32 + col;
    if (hf == 0 && row < sq) {
      const float lv = (m_run + __log2f(l_tot)) * kLn2;
      if (SPLIT) lse[(int64_t(sp) * H + h) * sq + row] = lv;
      else if (lse) lse[int64_t(h) * sq + row] = lv;
    }
  }
  barrier_wait<0>();
  if constexpr (SPLIT) {
    // Partial block of this work-group, in the order of the accumulators:
    // [wave][query block][column tile][row group][lane] x 16 bytes, so every
    // store is one contiguous KiB.  Rows past sq are written too (finite: they
    // repeat row sq-1) and the merge skips them.
    float* const blk = opart + ((int64_t(sp) * H + h) * nqt + qt) * int64_t(kBM * kD);
#pragma unroll
    for (int b = 0; b < kWaves; ++b) {
      const float inv = 1.f / *reinterpret_cast<const float*>(smem + kOffL + (b * 32 + col) * 4);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[b][ct];
          *reinterpret_cast<f32x4*>(blk + ((((wave * kWaves + b) * kCT + ct) * 4 + g) * 64 + lane) * 4) =
              f32x4{a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
        }
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < kWaves; ++b) {
      const int row = qt * kBM + b * 32 + col;
      const float inv = 1.f / *reinterpret_cast<const float*>(smem + kOffL + (b * 32 + col) * 4);
      if (row >= sq) continue;
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const int cb = wave * kColsW + ct * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = cb + 8 * g + 4 * hf;
          const f32x16& a = acc[b][ct];
          uint16_t* dst = o + int64_t(row) * rowstride + int64_t(h) * kD + d0;
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(a[4 * g] * inv, a[4 * g + 1] * inv),
                                                 pack_bf16x2(a[4 * g + 2] * inv, a[4 * g + 3] * inv)};
        }
      }
    }
  }
}

// Merge of the key ranges of a split launch (the partial blocks above): with
// m = max_s lse_s and w_s = exp(lse_s - m), O = sum_s w_s O_s / sum_s w_s
// (rounded once to bf16) and LSE = m + log(sum_s w_s), in float32.  One
// thread per 16-byte piece of a block, the same place in every range's block;
// the weights and the order of the sum are those of the row-major merge of the
// other head sizes.  HBM-bound: reads the partials once, eight ranges' loads in
// flight at a time (the LSEs for the maximum, then the partial pieces).
__global__ __launch_bounds__(256) void merge_d512_kernel(const float* __restrict__ opart,
                                                         const float* __restrict__ lpart, uint16_t* __restrict__ o,
                                                         float* __restrict__ lse, int nsplit, int sq, int H,
                                                         int nqt) {
  constexpr int kPieces = kBM * kD / 4;  // 16-byte pieces of one block
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t blkid = gid / kPieces;  // h * nqt + qt
  if (blkid >= int64_t(H) * nqt) return;
  const int c = int(gid - blkid * kPieces);
  const int h = int(blkid / nqt), qt = int(blkid - int64_t(h) * nqt);
  const int ln = c & 63, g = (c >> 6) & 3, ct = (c >> 8) & (kCT - 1), b = (c >> 10) & (kWaves - 1), w = c >> 12;
  const int row = qt * kBM + b * 32 + (ln & 31);
  if (row >= sq) return;
  const int ch = w * kColsW + ct * 32 + 8 * g + 4 * (ln >> 5);
  float m = -INFINITY;
  {
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      float l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) l[i] = lpart[(int64_t(s + i) * H + h) * sq + row];
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, l[i]);
    }
    for (; s < nsplit; ++s) m = fmaxf(m, lpart[(int64_t(s) * H + h) * sq + row]);
  }
  float ws = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto part = [&](int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(opart + ((int64_t(s) * H + h) * nqt + qt) * int64_t(kBM * kD) +
                                           int64_t(c) * 4);
  };
  auto add = [&](int s, const f32x4& x) __attribute__((always_inline)) {
    const float wgt = expf(lpart[(int64_t(s) * H + h) * sq + row] - m);
    ws += wgt;
    acc += wgt * x;
  };
  int s = 0;
  for (; s + 8 <= nsplit; s += 8) {
    f32x4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = part(s + i);
#pragma unroll
    for (int i = 0; i < 8; ++i) add(s + i, x[i]);
  }
  for (; s < nsplit; ++s) add(s, part(s));
  const float inv = 1.f / ws;
  *reinterpret_cast<u32x2*>(o + (int64_t(row) * H + h) * kD + ch) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (lse && ch == 0) lse[int64_t(h) * sq + row] = m + logf(ws);
}

}  // namespace

int64_t attn_d512_items(int64_t sq, int H, int nsplit) {
  const __int128 n = __int128((sq + kBM - 1) / kBM) * H * nsplit * kThreads;
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

int64_t attn_d512_merge_items(int64_t sq, int H) {
  const __int128 n = __int128((sq + kBM - 1) / kBM) * H * (kBM * kD / 4);
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

hipError_t launch_merge_d512(const float* opart, const float* lpart, void* o, float* lse, int nsplit, int64_t sq,
                             int H, hipStream_t stream) {
  const int64_t nqt = (sq + kBM - 1) / kBM;
  const int64_t blocks = nqt * H * (kBM * kD / 4) / 256;  // the host has checked the items against kMaxItems
  hipLaunchKernelGGL(merge_d512_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, opart, lpart,
                     static_cast<uint16_t*>(o), lse, nsplit, int(sq), H, int(nqt));
  return hipGetLastError();
}

hipError_t launch_attn_d512(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                            int64_t skv, int H, float c, int nsplit, float* opart, hipStream_t stream) {
  if (sq < 1) return hipSuccess;
  if (int64_t(H) * kRowB * kBN >= (int64_t(1) << 31)) return hipErrorInvalidValue;  // 32-bit row offsets
  const int64_t nqt = (sq + kBM - 1) / kBM;
  const int64_t grid = nqt * H * nsplit;  // the host has checked grid * kThreads <= kMaxItems
  if (grid > kMaxItems / kThreads) return hipErrorInvalidConfiguration;
  if (opart)
    hipLaunchKernelGGL(attn_d512_kernel<true>, dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, int(sq), int(skv), H, c,
                       int(nqt), nsplit, opart);
  else
    hipLaunchKernelGGL(attn_d512_kernel<false>, dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, int(sq), int(skv), H, c,
                       int(nqt), 1, opart);
  return hipGetLastError();
}

}  // namespace spattn

// Rotary position embedding of one rank's local slice at absolute positions.
//
// Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", section 机制一: the
// RoPE frequency table is sliced with the rank's token range, so token t of
// the slice rotates at position pos0 + t.  Page "NPU HunyuanImage-3.0模型推理优化
// 实践", section 消除旋转位置编码冗余cast算子: the rotation applies to q and k.
//
// Each thread owns PG consecutive frequency pairs of one token: it derives the
// angles p * theta^(-2j/d) and their cos/sin once in float64 (positions reach
// 3.7e5 here, where a float32 angle would be off by up to 0.03 rad) and then
// walks all H heads of that token, so the float64 work is shared by H rows.
// The rotation itself is float32; the result is rounded to the storage type
// (nearest-even).  HBM-bound: each element is read once and written once.
#include <hip/hip_bf16.h>

#include "internal.h"

namespace spattn {
namespace {

constexpr int kThreads = 256;

__device__ inline float ld(const float* p) { return *p; }
__device__ inline float ld(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }

__device__ inline uint16_t to_bf16(float f) {
  __hip_bfloat16 b = __float2bfloat16(f);  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}
__device__ inline void st(float* p, float f) { *p = f; }
__device__ inline void st(uint16_t* p, float f) { *p = to_bf16(f); }

// cos/sin of the PG pairs j0 .. j0+PG-1 of token t.
// Multi-axis form: the d/2 pairs are split into consecutive groups of n0, n1
// and d/2-n0-n1 pairs (axes 0, 1, 2); pair j' of axis a rotates by
// pos[t][a] * theta^(-2 j' / (2 n_a)).  With pos == nullptr the single axis
// position pos0 + t is used and the caller passes n0 = d/2, n1 = 0 (plain 1-D
// RoPE, where this is p * theta^(-2j/d)).
template <int PG>
__device__ inline void pair_angles(int64_t t, int j0, int half, int64_t pos0, const int64_t* __restrict__ pos,
                                   int n0, int n1, double log2theta, float (&cs)[PG], float (&sn)[PG]) {
#pragma unroll
  for (int u = 0; u < PG; ++u) {
    const int j = j0 + u;
    const int a = j < n0 ? 0 : (j < n0 + n1 ? 1 : 2);
    const int jl = j - (a == 0 ? 0 : (a == 1 ? n0 : n0 + n1));      // index inside the axis group
    const int da = 2 * (a == 0 ? n0 : (a == 1 ? n1 : half - n0 - n1));  // 2 * pairs of the axis
    const double p = pos ? double(pos[t * 3 + a]) : double(pos0 + t);
    const double inv = exp2(-double(2 * jl) / double(da) * log2theta);
    double sv, cv;
    sincos(p * inv, &sv, &cv);
    cs[u] = float(cv);
    sn[u] = float(sv);
  }
}

// Element offsets inside a head row of the two members of pair j.
template <bool INTERLEAVED>
__device__ inline int first_of(int j, int half) { return INTERLEAVED ? 2 * j : j; }
template <bool INTERLEAVED>
__device__ inline int second_of(int j, int half) { return INTERLEAVED ? 2 * j + 1 : j + half; }

// PG pairs per thread; element loads/stores are PG (or 2*PG) contiguous values
// and the compiler merges them into vector accesses when aligned.
template <typename T, int PG, bool INTERLEAVED>
__global__ __launch_bounds__(kThreads) void rope_kernel(const T* x, T* y, int64_t s, int H, int d, int64_t pos0,
                                                        const int64_t* __restrict__ pos, int n0, int n1,
                                                        double log2theta) {
  const int half = d >> 1;
  const int groups = half / PG;
  const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t t = g / groups;
  if (t >= s) return;
  const int j0 = int(g - t * groups) * PG;

  float cs[PG], sn[PG];
  pair_angles<PG>(t, j0, half, pos0, pos, n0, n1, log2theta, cs, sn);

  // Heads are processed in batches of HB: all loads of a batch are issued
  // before its stores.  x and y are either the same buffer or disjoint, and
  // every element is read and written by this thread only, so reading ahead
  // of the stores is safe in place too (the compiler cannot prove it, so the
  // batching is explicit).
  constexpr int HB = 8;
  for (int h0 = 0; h0 < H; h0 += HB) {
    float a[HB][PG], b[HB][PG];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (h0 + hh >= H) break;
      const int64_t row = (t * H + h0 + hh) * int64_t(d);
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        if (INTERLEAVED) {
          a[hh][u] = ld(x + row + 2 * (j0 + u));
          b[hh][u] = ld(x + row + 2 * (j0 + u) + 1);
        } else {
          a[hh][u] = ld(x + row + j0 + u);
          b[hh][u] = ld(x + row + half + j0 + u);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (h0 + hh >= H) break;
      const int64_t row = (t * H + h0 + hh) * int64_t(d);
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        const float ya = a[hh][u] * cs[u] - b[hh][u] * sn[u];
        const float yb = b[hh][u] * cs[u] + a[hh][u] * sn[u];
        if (INTERLEAVED) {
          st(y + row + 2 * (j0 + u), ya);
          st(y + row + 2 * (j0 + u) + 1, yb);
        } else {
          st(y + row + j0 + u, ya);
          st(y + row + half + j0 + u, yb);
        }
      }
    }
  }
}

// v + (v of the partner lane selected by the DPP control CTRL).
template <int CTRL>
__device__ inline float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sums over aligned groups of L lanes (L a power of two <= 64), N values at
// once.  Each stage adds the value of a partner lane from the other half of
// the current subgroup: quad permutations [1,0,3,2] and [2,3,0,1], then the
// mirror inside 8 lanes and inside 16 lanes (after the earlier stages every
// lane of a subgroup holds the subgroup's sum, so any partner in the other
// half serves), then xor 16 and 32 across rows.  Partners add the same two
// values, so every lane of a group ends with identical bits.
template <int N>
__device__ inline void group_sums(float (&v)[N], int L) {
  if (L > 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0xB1>(v[i]);
  }
  if (L > 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x4E>(v[i]);
  }
  if (L > 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x141>(v[i]);
  }
  if (L > 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x140>(v[i]);
  }
  for (int m = 16; m < L; m <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], m);
  }
}

// Per-head RMSNorm followed by the rotation (page "NPU HunyuanImage-3.0模型推理
// 优化实践", sections 计算分解 and RmsNorm算子优化: q and k heads are
// normalised over the head dimension, scaled by a learned weight, then
// rotated).  Token t's head row is spread over L = 2^lanes_log2 consecutive
// lanes of one wave (L >= d/2/PG, lanes beyond d/2/PG hold zeros and store
// nothing); each lane squares and sums its 2*PG elements, group_sums adds
// them across the L lanes so that every lane holds the same row sum, then
//   y = rotate(x * gamma / sqrt(sum(x^2) / d + eps))
// in float32, rounded once to the storage type.  One read and one write per
// element, like rope_kernel.
template <typename T, int PG, bool INTERLEAVED>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(const T* x, T* y, int64_t s, int H, int d,
                                                                int lanes_log2, const float* __restrict__ gamma,
                                                                float eps, int64_t pos0,
                                                                const int64_t* __restrict__ pos, int n0, int n1,
                                                                double log2theta) {
  const int half = d >> 1;
  const int groups = half / PG;
  const int L = 1 << lanes_log2;
  const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t t = g >> lanes_log2;
  if (t >= s) return;  // whole L-lane groups leave together, so the butterflies below stay inside live groups
  const int jg = int(g & (L - 1));
  const bool act = jg < groups;
  const int j0 = (act ? jg : 0) * PG;

  float cs[PG], sn[PG], ga[PG], gb[PG];
  pair_angles<PG>(t, j0, half, pos0, pos, n0, n1, log2theta, cs, sn);
#pragma unroll
  for (int u = 0; u < PG; ++u) {
    ga[u] = gamma[first_of<INTERLEAVED>(j0 + u, half)];
    gb[u] = gamma[second_of<INTERLEAVED>(j0 + u, half)];
  }
  const float fd = float(d);

  // Heads in batches of HB with all loads of a batch before its stores; safe
  // in place for the same reason as in rope_kernel.
  constexpr int HB = 8;
  for (int h0 = 0; h0 < H; h0 += HB) {
    float a[HB][PG], b[HB][PG], ss[HB];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) ss[hh] = 0.f;
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      // a last batch past head H-1 re-reads head H-1 and stores nothing for
      // it, and idle lanes read pair 0 and drop it: every load stays
      // unconditional, so the loads vectorise and need no branch
      const int64_t row = (t * H + min(h0 + hh, H - 1)) * int64_t(d);
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        const float va = ld(x + row + first_of<INTERLEAVED>(j0 + u, half));
        const float vb = ld(x + row + second_of<INTERLEAVED>(j0 + u, half));
        a[hh][u] = act ? va : 0.f;
        b[hh][u] = act ? vb : 0.f;
        ss[hh] += a[hh][u] * a[hh][u] + b[hh][u] * b[hh][u];
      }
    }
    group_sums(ss, L);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (!act || h0 + hh >= H) break;
      const int64_t row = (t * H + h0 + hh) * int64_t(d);
      const float r = 1.0f / sqrtf(ss[hh] / fd + eps);
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        const float na = a[hh][u] * r * ga[u];
        const float nb = b[hh][u] * r * gb[u];
        st(y + row + first_of<INTERLEAVED>(j0 + u, half), na * cs[u] - nb * sn[u]);
        st(y + row + second_of<INTERLEAVED>(j0 + u, half), nb * cs[u] + na * sn[u]);
      }
    }
  }
}

template <typename T, int PG, bool IL>
hipError_t launch_norm_typed(const void* x, void* y, int64_t s, int H, int d, const float* gamma, float eps,
                             int64_t pos0, const int64_t* pos, int n0, int n1, double l2t, hipStream_t stream) {
  const int groups = (d / 2) / PG;
  int lg = 0;
  while ((1 << lg) < groups) ++lg;
  const int64_t threads = s << lg;
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > kMaxGrid) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((qk_norm_rope_kernel<T, PG, IL>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const T*>(x), static_cast<T*>(y), s, H, d, lg, gamma, eps, pos0, pos, n0,
                     n1, l2t);
  return hipGetLastError();
}

template <typename T, bool IL>
hipError_t launch_norm_pg(const void* x, void* y, int64_t s, int H, int d, const float* gamma, float eps,
                          int64_t pos0, const int64_t* pos, int n0, int n1, double l2t, hipStream_t stream) {
  switch (norm_pairs_per_lane(d)) {
    case 4: return launch_norm_typed<T, 4, IL>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    case 8: return launch_norm_typed<T, 8, IL>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    case 2: return launch_norm_typed<T, 2, IL>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    case 1: return launch_norm_typed<T, 1, IL>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int PG, bool IL>
hipError_t launch_typed(const void* x, void* y, int64_t s, int H, int d, int64_t pos0, const int64_t* pos, int n0,
                        int n1, double l2t, hipStream_t stream) {
  const int64_t threads = s * ((d / 2) / PG);
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > kMaxGrid) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((rope_kernel<T, PG, IL>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const T*>(x), static_cast<T*>(y), s, H, d, pos0, pos, n0, n1, l2t);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const void* x, void* y, int64_t s, int H, int d, int64_t pos0, const int64_t* pos, int n0,
                        int n1, double l2t, int style, hipStream_t stream) {
  const bool wide = ((d / 2) % 4) == 0;
  if (style == 1)
    return wide ? launch_typed<T, 4, true>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream)
                : launch_typed<T, 1, true>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream);
  return wide ? launch_typed<T, 4, false>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream)
              : launch_typed<T, 1, false>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream);
}

}  // namespace

hipError_t launch_rope(int dtype, const void* x, void* y, int64_t s, int H, int d, int64_t pos0,
                       double theta, int style, hipStream_t stream) {
  const double l2t = log2(theta);
  if (dtype == 0) return launch_dtype<float>(x, y, s, H, d, pos0, nullptr, d / 2, 0, l2t, style, stream);
  return launch_dtype<uint16_t>(x, y, s, H, d, pos0, nullptr, d / 2, 0, l2t, style, stream);
}

hipError_t launch_rope_mx(int dtype, const void* x, void* y, int64_t s, int H, int d, const int64_t* pos,
                          const int* sections, double theta, int style, hipStream_t stream) {
  const double l2t = log2(theta);
  if (dtype == 0)
    return launch_dtype<float>(x, y, s, H, d, 0, pos, sections[0], sections[1], l2t, style, stream);
  return launch_dtype<uint16_t>(x, y, s, H, d, 0, pos, sections[0], sections[1], l2t, style, stream);
}

int norm_pairs_per_lane(int d) {
  const int half = d / 2;
  if (half % 4 == 0 && half / 4 <= 64) return 4;
  if (half % 8 == 0 && half / 8 <= 64) return 8;
  if (half % 2 == 0 && half / 2 <= 64) return 2;
  if (half <= 64) return 1;
  return 0;
}

hipError_t launch_qk_norm_rope(int dtype, const void* x, void* y, int64_t s, int H, int d, const float* gamma,
                               float eps, int64_t pos0, const int64_t* pos, const int* sections, double theta,
                               int style, hipStream_t stream) {
  const double l2t = log2(theta);
  const int n0 = pos ? sections[0] : d / 2, n1 = pos ? sections[1] : 0;
  if (dtype == 0)
    return style == 1 ? launch_norm_pg<float, true>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream)
                      : launch_norm_pg<float, false>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
  return style == 1 ? launch_norm_pg<uint16_t, true>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream)
                    : launch_norm_pg<uint16_t, false>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
}

}  // namespace spattn

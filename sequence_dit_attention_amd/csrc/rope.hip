// Rotary position embedding of one rank's local slice at absolute positions,
// and the per-head RMSNorm fused in front of it.
//
// Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", section 机制一: the
// RoPE frequency table is sliced with the rank's token range, so token t of
// the slice rotates at position pos0 + t.  Page "NPU HunyuanImage-3.0模型推理优化
// 实践", section 消除旋转位置编码冗余cast算子: the rotation applies to q and k;
// sections 计算分解 and RmsNorm算子优化: q and k heads are normalised over the
// head dimension, scaled by a learned weight, then rotated.
//
// Angles p * theta^(-2j/d) and their range reduction are float64 (positions
// reach 3.7e5 here, where a float32 angle would be off by up to 0.03 rad);
// cos/sin are rounded to float32, the norm and the rotation are float32 and
// the result is rounded once to the storage type (nearest-even).  HBM-bound:
// each element is read once and written once.
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
__device__ inline float widen(float v) { return v; }
__device__ inline float widen(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ inline float narrow(float f, float*) { return f; }
__device__ inline uint16_t narrow(float f, uint16_t*) { return to_bf16(f); }

// N consecutive elements as one vector access, non-temporal (every element is
// touched once).  Written out explicitly: element-wise bf16 accesses are not
// merged by the compiler and run at two thirds of the vector rate.
template <typename T, int N>
struct Vec {
  typedef T type __attribute__((ext_vector_type(N)));
};
template <typename T>
struct Vec<T, 1> {
  typedef T type;
};
template <int N, typename T>
__device__ inline void ldv(const T* p, float (&o)[N]) {
  typedef typename Vec<T, N>::type V;
  const V v = __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  if constexpr (N == 1) {
    o[0] = widen(v);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = widen(T(v[i]));
  }
}
template <int N, typename T>
__device__ inline void stv(T* p, const float (&f)[N]) {
  typedef typename Vec<T, N>::type V;
  V v;
  if constexpr (N == 1) {
    v = narrow(f[0], p);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = narrow(f[i], p);
  }
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

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

// The rotation of pair (x1, x2), each output rounded once from an explicit
// fused multiply-add: the same bits whichever kernel or access width computes
// it (left to the compiler, the contraction of a*c - b*s varies with the
// shape of the surrounding code).
__device__ inline float rot_first(float x1, float x2, float c, float s) { return fmaf(x1, c, -(x2 * s)); }
__device__ inline float rot_second(float x1, float x2, float c, float s) { return fmaf(x2, c, x1 * s); }

// Element offsets inside a head row of the two members of pair j.
template <bool INTERLEAVED>
__device__ inline int first_of(int j, int half) { return INTERLEAVED ? 2 * j : j; }
template <bool INTERLEAVED>
__device__ inline int second_of(int j, int half) { return INTERLEAVED ? 2 * j + 1 : j + half; }

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

// One wave per token.  Its 64 lanes form R = 64 / L row slots of L lanes
// (L = 2^lanes_log2 >= d/2/PG); slot r handles heads r, r + R, r + 2R, ... of
// the token, so each load instruction of the wave covers R consecutive head
// rows, and lane jg of a slot owns pairs jg*PG .. jg*PG+PG-1 (lanes past
// d/2/PG read pair 0 and store nothing).  A lane's PG first and PG second
// pair members are contiguous (2*PG for the interleaved pairing), so they move
// as vectors.  With d/2 <= 64 each lane derives the cos/sin of one pair and
// the wave shares them by lane shuffles: every angle of a token is computed
// once.  NORM: each lane squares and sums its 2*PG elements, group_sums adds
// them across the row's L lanes, and y = rotate(x * gamma / sqrt(sum / d + eps)).
// Heads are processed in batches of HB iterations with all loads of a batch
// before its stores: in place is allowed, and each element is read and
// written by one lane only.
template <typename T, int PG, bool IL, bool NORM>
__global__ __launch_bounds__(kThreads) void rope_rows_kernel(const T* x, T* y, int64_t s, int H, int d,
                                                             int lanes_log2, const float* __restrict__ gamma,
                                                             float eps, int64_t pos0,
                                                             const int64_t* __restrict__ pos, int n0, int n1,
                                                             double log2theta) {
  const int half = d >> 1;
  const int groups = half / PG;
  const int L = 1 << lanes_log2, R = 64 >> lanes_log2;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  if (t >= s) return;  // whole waves leave together
  const int slot = lane >> lanes_log2, jg = lane & (L - 1);
  const bool act = jg < groups;
  const int j0 = (act ? jg : 0) * PG;

  float cs[PG], sn[PG];
  if (half <= 64) {
    float c1[1], s1[1];
    pair_angles<1>(t, lane < half ? lane : 0, half, pos0, pos, n0, n1, log2theta, c1, s1);
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      cs[u] = __shfl(c1[0], j0 + u);
      sn[u] = __shfl(s1[0], j0 + u);
    }
  } else {
    pair_angles<PG>(t, j0, half, pos0, pos, n0, n1, log2theta, cs, sn);
  }
  float ga[PG], gb[PG];
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < PG; ++u) {
      ga[u] = gamma[first_of<IL>(j0 + u, half)];
      gb[u] = gamma[second_of<IL>(j0 + u, half)];
    }
  }
  const float fd = float(d);
  const int nk = (H + R - 1) / R;  // head iterations of a slot
  constexpr int HB = 6;            // iterations per batch (24 heads of 128: one batch)
  for (int k0 = 0; k0 < nk; k0 += HB) {
    float a[HB][PG], b[HB][PG], ss[HB];
#pragma unroll
    for (int kk = 0; kk < HB; ++kk) ss[kk] = 0.f;
#pragma unroll
    for (int kk = 0; kk < HB; ++kk) {
      if (k0 + kk >= nk) break;
      // a slot past head H-1 re-reads head H-1 and stores nothing
      const T* row = x + (t * H + min((k0 + kk) * R + slot, H - 1)) * int64_t(d);
      if constexpr (IL && PG == 1) {  // one pair: two element accesses, element alignment suffices
        float va[1], vb[1];
        ldv<1>(row + 2 * j0, va);
        ldv<1>(row + 2 * j0 + 1, vb);
        a[kk][0] = act ? va[0] : 0.f;
        b[kk][0] = act ? vb[0] : 0.f;
      } else if constexpr (IL) {
        float v[2 * PG];
        ldv<2 * PG>(row + 2 * j0, v);
#pragma unroll
        for (int u = 0; u < PG; ++u) {
          a[kk][u] = act ? v[2 * u] : 0.f;
          b[kk][u] = act ? v[2 * u + 1] : 0.f;
        }
      } else {
        float va[PG], vb[PG];
        ldv<PG>(row + j0, va);
        ldv<PG>(row + half + j0, vb);
#pragma unroll
        for (int u = 0; u < PG; ++u) {
          a[kk][u] = act ? va[u] : 0.f;
          b[kk][u] = act ? vb[u] : 0.f;
        }
      }
      if constexpr (NORM) {
#pragma unroll
        for (int u = 0; u < PG; ++u) ss[kk] = fmaf(b[kk][u], b[kk][u], fmaf(a[kk][u], a[kk][u], ss[kk]));
      }
    }
    if constexpr (NORM) group_sums(ss, L);
#pragma unroll
    for (int kk = 0; kk < HB; ++kk) {
      if (k0 + kk >= nk) break;
      const int h = (k0 + kk) * R + slot;
      if (!act || h >= H) continue;
      T* row = y + (t * H + h) * int64_t(d);
      float r = 1.f;
      if constexpr (NORM) r = 1.0f / sqrtf(ss[kk] / fd + eps);
      float ya[PG], yb[PG];
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        const float na = NORM ? a[kk][u] * r * ga[u] : a[kk][u];
        const float nb = NORM ? b[kk][u] * r * gb[u] : b[kk][u];
        ya[u] = rot_first(na, nb, cs[u], sn[u]);
        yb[u] = rot_second(na, nb, cs[u], sn[u]);
      }
      if constexpr (IL && PG == 1) {
        stv<1>(row + 2 * j0, ya);
        stv<1>(row + 2 * j0 + 1, yb);
      } else if constexpr (IL) {
        float v[2 * PG];
#pragma unroll
        for (int u = 0; u < PG; ++u) {
          v[2 * u] = ya[u];
          v[2 * u + 1] = yb[u];
        }
        stv<2 * PG>(row + 2 * j0, v);
      } else {
        stv<PG>(row + j0, ya);
        stv<PG>(row + half + j0, yb);
      }
    }
  }
}

// General shapes (a head row that does not fit one wave in groups of 1, 2, 4
// or 8 pairs, or buffers not aligned for the vector accesses): each thread
// owns PG consecutive pairs of one token and walks all H heads of that token,
// element by element.  Same arithmetic as rope_rows_kernel without NORM.
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

  constexpr int HB = 8;
  for (int h0 = 0; h0 < H; h0 += HB) {
    float a[HB][PG], b[HB][PG];
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (h0 + hh >= H) break;
      const int64_t row = (t * H + h0 + hh) * int64_t(d);
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        a[hh][u] = ld(x + row + first_of<INTERLEAVED>(j0 + u, half));
        b[hh][u] = ld(x + row + second_of<INTERLEAVED>(j0 + u, half));
      }
    }
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      if (h0 + hh >= H) break;
      const int64_t row = (t * H + h0 + hh) * int64_t(d);
#pragma unroll
      for (int u = 0; u < PG; ++u) {
        st(y + row + first_of<INTERLEAVED>(j0 + u, half), rot_first(a[hh][u], b[hh][u], cs[u], sn[u]));
        st(y + row + second_of<INTERLEAVED>(j0 + u, half), rot_second(a[hh][u], b[hh][u], cs[u], sn[u]));
      }
    }
  }
}

template <typename T, int PG, bool IL, bool NORM>
hipError_t launch_rows(const void* x, void* y, int64_t s, int H, int d, const float* gamma, float eps, int64_t pos0,
                       const int64_t* pos, int n0, int n1, double l2t, hipStream_t stream) {
  const int groups = (d / 2) / PG;
  int lg = 0;
  while ((1 << lg) < groups) ++lg;
  const int64_t blocks = (s + kThreads / 64 - 1) / (kThreads / 64);  // one wave per token
  if (blocks > kMaxItems / kThreads) return hipErrorInvalidConfiguration;  // checked by the host already
  hipLaunchKernelGGL((rope_rows_kernel<T, PG, IL, NORM>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const T*>(x), static_cast<T*>(y), s, H, d, lg, gamma, eps, pos0, pos, n0,
                     n1, l2t);
  return hipGetLastError();
}

template <typename T, bool IL, bool NORM>
hipError_t launch_rows_pg(int pg, const void* x, void* y, int64_t s, int H, int d, const float* gamma, float eps,
                          int64_t pos0, const int64_t* pos, int n0, int n1, double l2t, hipStream_t stream) {
  switch (pg) {
    case 4: return launch_rows<T, 4, IL, NORM>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    case 8: return launch_rows<T, 8, IL, NORM>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    case 2: return launch_rows<T, 2, IL, NORM>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    case 1: return launch_rows<T, 1, IL, NORM>(x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int PG, bool IL>
hipError_t launch_general(const void* x, void* y, int64_t s, int H, int d, int64_t pos0, const int64_t* pos, int n0,
                          int n1, double l2t, hipStream_t stream) {
  const int64_t threads = s * ((d / 2) / PG);
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > kMaxItems / kThreads) return hipErrorInvalidConfiguration;  // checked by the host already
  hipLaunchKernelGGL((rope_kernel<T, PG, IL>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const T*>(x), static_cast<T*>(y), s, H, d, pos0, pos, n0, n1, l2t);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_t(const void* x, void* y, int64_t s, int H, int d, int64_t pos0, const int64_t* pos, int n0,
                         int n1, double l2t, int style, hipStream_t stream) {
  const int pg = rows_pairs_per_lane(d, style, int(sizeof(T)), x, y);
  if (pg) {
    if (style == 1)
      return launch_rows_pg<T, true, false>(pg, x, y, s, H, d, nullptr, 0.f, pos0, pos, n0, n1, l2t, stream);
    return launch_rows_pg<T, false, false>(pg, x, y, s, H, d, nullptr, 0.f, pos0, pos, n0, n1, l2t, stream);
  }
  const bool wide = ((d / 2) % 4) == 0;
  if (style == 1)
    return wide ? launch_general<T, 4, true>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream)
                : launch_general<T, 1, true>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream);
  return wide ? launch_general<T, 4, false>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream)
              : launch_general<T, 1, false>(x, y, s, H, d, pos0, pos, n0, n1, l2t, stream);
}

}  // namespace

int rows_pairs_per_lane(int d, int style, int eb, const void* x, const void* y) {
  const int half = d / 2;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y);
  for (int pg : {4, 8, 2, 1}) {
    if (half % pg != 0 || half / pg > 64) continue;
    const uintptr_t vec = uintptr_t(pg) * (style == 1 && pg > 1 ? 2 : 1) * eb;  // bytes of one vector access
    if (addr % vec == 0) return pg;
  }
  return 0;
}

int64_t rope_items(int eb, int64_t s, int d, int style, const void* x, const void* y, bool norm) {
  const int pg = rows_pairs_per_lane(d, style, eb, x, y);
  __int128 n;
  if (pg || norm) {
    n = __int128((s + kThreads / 64 - 1) / (kThreads / 64)) * kThreads;  // one wave per token
  } else {
    const int per = (d / 2) / (((d / 2) % 4) == 0 ? 4 : 1);  // threads per token of the element-wise kernel
    n = (__int128(s) * per + kThreads - 1) / kThreads * kThreads;
  }
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

hipError_t launch_rope(int dtype, const void* x, void* y, int64_t s, int H, int d, int64_t pos0,
                       double theta, int style, hipStream_t stream) {
  const double l2t = log2(theta);
  if (dtype == 0) return launch_rope_t<float>(x, y, s, H, d, pos0, nullptr, d / 2, 0, l2t, style, stream);
  return launch_rope_t<uint16_t>(x, y, s, H, d, pos0, nullptr, d / 2, 0, l2t, style, stream);
}

hipError_t launch_rope_mx(int dtype, const void* x, void* y, int64_t s, int H, int d, const int64_t* pos,
                          const int* sections, double theta, int style, hipStream_t stream) {
  const double l2t = log2(theta);
  if (dtype == 0)
    return launch_rope_t<float>(x, y, s, H, d, 0, pos, sections[0], sections[1], l2t, style, stream);
  return launch_rope_t<uint16_t>(x, y, s, H, d, 0, pos, sections[0], sections[1], l2t, style, stream);
}

hipError_t launch_qk_norm_rope(int dtype, const void* x, void* y, int64_t s, int H, int d, const float* gamma,
                               float eps, int64_t pos0, const int64_t* pos, const int* sections, double theta,
                               int style, hipStream_t stream) {
  const double l2t = log2(theta);
  const int n0 = pos ? sections[0] : d / 2, n1 = pos ? sections[1] : 0;
  const int pg = rows_pairs_per_lane(d, style, dtype == 0 ? 4 : 2, x, y);
  if (dtype == 0) {
    if (style == 1)
      return launch_rows_pg<float, true, true>(pg, x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
    return launch_rows_pg<float, false, true>(pg, x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
  }
  if (style == 1)
    return launch_rows_pg<uint16_t, true, true>(pg, x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
  return launch_rows_pg<uint16_t, false, true>(pg, x, y, s, H, d, gamma, eps, pos0, pos, n0, n1, l2t, stream);
}

}  // namespace spattn

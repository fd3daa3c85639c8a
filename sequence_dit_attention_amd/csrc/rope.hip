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

// PG pairs per thread; element loads/stores are PG (or 2*PG) contiguous values
// and the compiler merges them into vector accesses when aligned.
// Multi-axis form: the d/2 pairs are split into consecutive groups of n0, n1
// and d/2-n0-n1 pairs (axes 0, 1, 2); pair j' of axis a rotates by
// pos[t][a] * theta^(-2 j' / (2 n_a)).  With pos == nullptr the single axis
// position pos0 + t is used and the caller passes n0 = d/2, n1 = 0 (plain 1-D
// RoPE, the same arithmetic as before).
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

}  // namespace spattn

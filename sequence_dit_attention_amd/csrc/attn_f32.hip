// Float32 attention of local queries against the full K/V (no mask).
//
// Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", section 机制一: Q
// from the rank's shard, K/V over the whole sequence.  This is the small,
// float32 path: one lane per (query row, head), K/V tiles of 32 keys staged in
// LDS and read as broadcasts, and the usual online softmax (running max,
// rescaled running sum and accumulator) in float32, base 2 with the scale
// folded into log2(e).
#include "internal.h"

#include <type_traits>

namespace spattn {
namespace {

constexpr int kRows = 64;  // query rows (lanes) per work-group: one wave
constexpr int kBN = 32;    // keys per LDS tile

// K/V argument: gathered [skv, H, d] buffers, or per-rank shards (GV).
struct KvFlatF32 {
  const float* k;
  const float* v;
};
template <bool GV>
using KvArgF32 = typename std::conditional<GV, KvShards, KvFlatF32>::type;

template <int D, bool GV>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(const float* __restrict__ q, const KvArgF32<GV> kv,
                                                         float* __restrict__ o, float* __restrict__ lse,
                                                         int64_t sq, int64_t skv, int H,
                                                         float c /* scale * log2(e) */, int64_t nqt) {
  __shared__ float ks[kBN][D];
  __shared__ float vs[kBN][D];
  const int64_t wg = blockIdx.x;
  const int h = int(wg / nqt);
  const int64_t i = (wg % nqt) * kRows + threadIdx.x;
  const bool live = i < sq;

  float qr[D], acc[D];
  const float* qp = q + (i * H + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qr[e] = live ? qp[e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int64_t j0 = 0; j0 < skv; j0 += kBN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kBN * D; idx += kRows) {
      const int r = idx / D, e = idx % D;
      const int64_t j = j0 + r;
      float kx = 0.f, vx = 0.f;
      if (j < skv) {
        if constexpr (GV) {  // shard s holds tokens [start[s], start[s+1])
          int s = 0;
          for (int b = 1; b < kv.W; ++b) s += kv.start[b] <= j ? 1 : 0;
          const int64_t off = ((j - kv.start[s]) * H + h) * D + e;
          kx = static_cast<const float*>(kv.k[s])[off];
          vx = static_cast<const float*>(kv.v[s])[off];
        } else {
          kx = kv.k[(j * H + h) * D + e];
          vx = kv.v[(j * H + h) * D + e];
        }
      }
      ks[r][e] = kx;
      vs[r][e] = vx;
    }
    __syncthreads();
    float sc[kBN];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < kBN; ++r) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qr[e], ks[r][e], dot);
      sc[r] = (j0 + r < skv) ? dot * c : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < kBN; ++r) {
      sc[r] = exp2f(sc[r] - mn);
      rs += sc[r];
    }
    l = l * alpha + rs;
    m = mn;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      float a = acc[e] * alpha;
#pragma unroll
      for (int r = 0; r < kBN; ++r) a = fmaf(sc[r], vs[r][e], a);
      acc[e] = a;
    }
  }
  if (!live) return;
  const float inv = 1.f / l;
  float* op = o + (i * H + h) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
  if (lse) lse[int64_t(h) * sq + i] = (m + log2f(l)) * 0.69314718055994531f;
}

template <bool GV>
hipError_t launch_any(const float* q, const KvArgF32<GV>& kv, float* o, float* lse, int64_t sq, int64_t skv,
                      int H, int d, float scale, hipStream_t stream) {
  const int64_t nqt = (sq + kRows - 1) / kRows;
  const int64_t grid = nqt * H;  // the host has checked grid * kRows <= kMaxItems
  if (grid > kMaxItems / kRows) return hipErrorInvalidConfiguration;
  const float c = scale * 1.4426950408889634f;
  if (d == 64)
    hipLaunchKernelGGL((attn_f32_kernel<64, GV>), dim3(unsigned(grid)), dim3(kRows), 0, stream, q, kv, o, lse, sq,
                       skv, H, c, nqt);
  else
    hipLaunchKernelGGL((attn_f32_kernel<128, GV>), dim3(unsigned(grid)), dim3(kRows), 0, stream, q, kv, o, lse,
                       sq, skv, H, c, nqt);
  return hipGetLastError();
}

}  // namespace

int64_t attn_f32_items(int64_t sq, int H) {
  const __int128 n = __int128((sq + kRows - 1) / kRows) * H * kRows;
  return n > INT64_MAX ? INT64_MAX : int64_t(n);
}

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int64_t sq, int64_t skv, int H, int d, float scale, hipStream_t stream) {
  return launch_any<false>(q, KvFlatF32{k, v}, o, lse, sq, skv, H, d, scale, stream);
}

hipError_t launch_attn_f32_gv(const float* q, const KvShards& kv, float* o, float* lse, int64_t sq, int H, int d,
                              float scale, hipStream_t stream) {
  return launch_any<true>(q, kv, o, lse, sq, kv.start[kv.W], H, d, scale, stream);
}

}  // namespace spattn

// Launchers shared between the host C ABI (capi.cpp) and the gfx950 kernels.
// Arguments reaching these functions have been validated by capi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spattn {

// One contiguous copy per (outer slice, segment):
//   bytes [0, nbytes) of src + o*src_stride  ->  dst + o*dst_stride, o in [0, outer)
struct CopySeg {
  const char* src;
  char* dst;
  int64_t nbytes;
  int64_t src_stride;
  int64_t dst_stride;
  int64_t outer = -1;  // outer steps of this segment; -1: the launch's `outer`
};

// Enqueue the copies of `n` segments (any n >= 0) on `stream`: segment i
// copies nbytes from src + o*src_stride to dst + o*dst_stride for each outer
// step o below its own outer count (or the call's `outer`).
hipError_t launch_segcopy(const CopySeg* segs, int n, int64_t outer, hipStream_t stream);

// RoPE of x[s, H, d] into y (may alias x).  dtype: 0 f32, 1 bf16.  style: 0 half, 1 interleaved.
hipError_t launch_rope(int dtype, const void* x, void* y, int64_t s, int H, int d,
                       int64_t pos0, double theta, int style, hipStream_t stream);

// Multi-axis RoPE with explicit positions pos[s][3] (device) and pairs per axis sections[3] (host).
hipError_t launch_rope_mx(int dtype, const void* x, void* y, int64_t s, int H, int d, const int64_t* pos,
                          const int* sections, double theta, int style, hipStream_t stream);

// Pairs per lane of the one-wave-per-token RoPE kernels for head size d,
// pairing style (0 half, 1 interleaved), element bytes eb and the buffers x, y
// (their addresses must suit the vector accesses); 0 if the head row does not
// fit one wave in groups of 1, 2, 4 or 8 pairs with aligned accesses.
int rows_pairs_per_lane(int d, int style, int eb, const void* x, const void* y);
hipError_t launch_qk_norm_rope(int dtype, const void* x, void* y, int64_t s, int H, int d, const float* gamma,
                               float eps, int64_t pos0, const int64_t* pos, const int* sections, double theta,
                               int style, hipStream_t stream);

// Attention of q[sq, H, d] against k, v[skv, H, d].
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t sq, int64_t skv, int H, int d, float scale, hipStream_t stream);
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int64_t sq, int64_t skv, int H, int d, float scale, hipStream_t stream);

// K/V given as W per-rank shards instead of one gathered buffer: shard r
// holds tokens [start[r], start[r+1]) of the sequence as a contiguous
// [start[r+1] - start[r], H, d] tensor (k[r], v[r] may be null when empty).
constexpr int kMaxShards = 16;
struct KvShards {
  const void* k[kMaxShards];
  const void* v[kMaxShards];
  int64_t start[kMaxShards + 1];
  int W;
};

// Attention against sharded K/V (same results as the gathered call on the
// concatenation of the shards).
// Split-key attention: nsplit launches' worth of key ranges in one launch
// writing float32 partials (opart: split_rows(sq, d) x H x d floats per range,
// lpart [nsplit, H, sq]), then a merge into o (bf16) and lse (may be null).
hipError_t launch_attn_bf16_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                                  int64_t skv, int H, int d, float scale, int nsplit, float* opart, float* lpart,
                                  hipStream_t stream);
hipError_t launch_attn_bf16_gv(const void* q, const KvShards& kv, void* o, float* lse, int64_t sq, int H, int d,
                               float scale, hipStream_t stream);
hipError_t launch_attn_f32_gv(const float* q, const KvShards& kv, float* o, float* lse, int64_t sq, int H, int d,
                              float scale, hipStream_t stream);

// Head size 512 (bf16, its own kernel: every score formed once).  c is the
// softmax scale times log2(e).  opart == nullptr: writes o and lse (may be
// null); otherwise the keys are cut into nsplit ranges and the call writes
// float32 partials, one 128-query x 512 block per (range, head, query tile)
// in the order of the kernel's accumulators, and their LSE into lse
// ([nsplit, H, sq]); launch_merge_d512 combines them.
hipError_t launch_attn_d512(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                            int64_t skv, int H, float c, int nsplit, float* opart, hipStream_t stream);
hipError_t launch_merge_d512(const float* opart, const float* lpart, void* o, float* lse, int nsplit, int64_t sq,
                             int H, hipStream_t stream);
int64_t attn_d512_items(int64_t sq, int H, int nsplit);
int64_t attn_d512_merge_items(int64_t sq, int H);

// Rows of float32 partials per (range, head) that a split launch writes: sq,
// or for head size 512 sq rounded up to whole 128-query tiles.
inline int64_t split_rows(int64_t sq, int d) { return d == 512 ? (sq + 127) / 128 * 128 : sq; }

// Head size 128 (bf16, eight waves per work-group, two per SIMD).  c is the
// softmax scale times log2(e).  opart == nullptr: writes o and lse (may be
// null); otherwise key ranges, float32 partials opart [nsplit, sq, H, 128] and
// their LSE into lse ([nsplit, H, sq]).
hipError_t launch_attn_d128(const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                            int64_t skv, int H, float c, int nsplit, float* opart, hipStream_t stream);
hipError_t launch_attn_d128_gv(const void* q, const KvShards& kv, void* o, float* lse, int64_t sq, int H, float c,
                               hipStream_t stream);
int64_t attn_d128_items(int64_t sq, int H, int nsplit);

// Device scratch of the split attention's allocation-free entry point: one
// file-scope array per device (kScratchBytes, 256-byte aligned), held until
// the process ends.  scratch_address() gives the current device's copy; the
// address is looked up once per device and kept.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
hipError_t scratch_address(void** out);

// A HIP launch's grid size is a 32-bit count of work-items per dimension.
// The host checks every launch of a call against it before enqueuing any.
constexpr int64_t kMaxItems = (int64_t(1) << 32) - 1;

// Work-items (grid dimension x) of each launch a call makes, for that check;
// saturate at INT64_MAX instead of overflowing.
int64_t attn_bf16_items(int64_t sq, int H, int d, int nsplit);  // the attention kernel
int64_t attn_merge_items(int64_t sq, int H, int d);              // merge of a split launch
int64_t attn_f32_items(int64_t sq, int H);
int64_t rope_items(int eb, int64_t s, int d, int style, const void* x, const void* y, bool norm);
// Largest work-item count of any one batch launch_segcopy would make.
int64_t segcopy_max_items(const CopySeg* segs, int n);

}  // namespace spattn

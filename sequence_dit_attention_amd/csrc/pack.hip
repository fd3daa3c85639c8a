// AllGatherV data movement on one GPU: a batch of contiguous copies.
//
// varlen_pack writes every rank's shard into its block of the flat receive
// buffer and varlen_unpack narrows/views/concatenates the blocks back into a
// sequence-major tensor (page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...",
// section 后端 A).  Both reduce to a list of (src, dst, nbytes) copies, one per
// (outer slice, rank).  The copy is HBM-bound: each work-group moves one
// fixed 4 KiB chunk of one segment, one 16-byte non-temporal load and store
// per lane.  Many small work-groups keep more requests in flight across the
// chip than few large ones (on MI355X a 4.5 GB copy runs at about 6.5 TB/s
// with 4 KiB chunks against 5.2 TB/s with 32 KiB chunks).
#include "internal.h"

namespace spattn {
namespace {

constexpr int kThreads = 256;
constexpr int kVecs = 1;                                      // 16-byte vectors per lane
constexpr int64_t kChunk = int64_t(kThreads) * kVecs * 16;    // bytes per work-group
constexpr int kMaxSegs = 32;                                  // segments per launch
constexpr int64_t kMaxGridY = 65535;

struct SegArgs {
  const char* src[kMaxSegs];
  char* dst[kMaxSegs];
  int64_t nbytes[kMaxSegs];
  int64_t src_stride[kMaxSegs];
  int64_t dst_stride[kMaxSegs];
  int64_t outer[kMaxSegs];          // outer steps of each segment
  int64_t first_blk[kMaxSegs + 1];  // work-group prefix of each segment within one outer slice
  int nseg;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void segcopy_kernel(SegArgs a, int64_t o_base) {
  const int64_t blk = blockIdx.x;
  int s = 0;
  while (s + 1 < a.nseg && a.first_blk[s + 1] <= blk) ++s;
  const int64_t o = o_base + blockIdx.y;
  if (o >= a.outer[s]) return;  // a segment with fewer outer steps than the launch
  const int64_t off = (blk - a.first_blk[s]) * kChunk;
  const int64_t left = a.nbytes[s] - off;  // int64 throughout: a segment may exceed 2^31 bytes
  const int64_t n = left < kChunk ? left : kChunk;
  const char* src = a.src[s] + o * a.src_stride[s] + off;
  char* dst = a.dst[s] + o * a.dst_stride[s] + off;
  const int tid = threadIdx.x;

  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | uintptr_t(n)) & 15) == 0) {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    const int nv = static_cast<int>(n >> 4);
    if (nv == kThreads * kVecs) {  // full chunk: all loads in flight, then all stores
      u32x4 r[kVecs];
#pragma unroll
      for (int i = 0; i < kVecs; ++i) r[i] = __builtin_nontemporal_load(s4 + tid + i * kThreads);
#pragma unroll
      for (int i = 0; i < kVecs; ++i) __builtin_nontemporal_store(r[i], d4 + tid + i * kThreads);
    } else {
      for (int i = tid; i < nv; i += kThreads) d4[i] = s4[i];
    }
  } else if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | uintptr_t(n)) & 3) == 0) {
    const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src);
    uint32_t* d1 = reinterpret_cast<uint32_t*>(dst);
    const int nw = static_cast<int>(n >> 2);
    for (int i = tid; i < nw; i += kThreads) d1[i] = s1[i];
  } else {  // elements are 2 or 4 bytes, so 2-byte alignment always holds
    const uint16_t* s1 = reinterpret_cast<const uint16_t*>(src);
    uint16_t* d1 = reinterpret_cast<uint16_t*>(dst);
    const int nh = static_cast<int>(n >> 1);
    for (int i = tid; i < nh; i += kThreads) d1[i] = s1[i];
  }
}

}  // namespace

namespace {

// Fills one launch's batch with the non-empty segments from segs[i] on (at
// most kMaxSegs of them); returns the index of the first segment left over.
int next_batch(const CopySeg* segs, int n, int i, int64_t outer, SegArgs& a, int64_t& blocks, int64_t& outer_max) {
  a = SegArgs{};
  a.nseg = 0;
  blocks = 0;
  outer_max = 0;
  for (; i < n && a.nseg < kMaxSegs; ++i) {
    if (segs[i].nbytes <= 0) continue;
    const int j = a.nseg++;
    a.src[j] = segs[i].src;
    a.dst[j] = segs[i].dst;
    a.nbytes[j] = segs[i].nbytes;
    a.src_stride[j] = segs[i].src_stride;
    a.dst_stride[j] = segs[i].dst_stride;
    a.outer[j] = segs[i].outer >= 0 ? segs[i].outer : outer;
    if (a.outer[j] > outer_max) outer_max = a.outer[j];
    a.first_blk[j] = blocks;
    blocks += (segs[i].nbytes + kChunk - 1) / kChunk;
  }
  a.first_blk[a.nseg] = blocks;
  return i;
}

}  // namespace

int64_t segcopy_max_items(const CopySeg* segs, int n) {
  int64_t most = 0;
  for (int i = 0; i < n;) {
    SegArgs a;
    int64_t blocks, outer_max;
    i = next_batch(segs, n, i, 0, a, blocks, outer_max);
    const int64_t items = blocks * int64_t(kThreads);  // blocks <= total bytes / 4 KiB + 32: no overflow
    if (items > most) most = items;
  }
  return most;
}

hipError_t launch_segcopy(const CopySeg* segs, int n, int64_t outer, hipStream_t stream) {
  int i = 0;  // next segment to place; empty ones are skipped, so a batch may span more than kMaxSegs entries
  while (i < n) {
    SegArgs a;
    int64_t blocks, outer_max;
    i = next_batch(segs, n, i, outer, a, blocks, outer_max);
    if (a.nseg == 0) continue;
    // Grid x covers one outer slice (the host has checked blocks * kThreads
    // against the 32-bit grid limit); grid y walks the outer slices in
    // launches of at most 65,535.
    for (int64_t o = 0; o < outer_max; o += kMaxGridY) {
      const int64_t rest = outer_max - o;
      const unsigned gy = static_cast<unsigned>(rest < kMaxGridY ? rest : kMaxGridY);
      hipLaunchKernelGGL(segcopy_kernel, dim3(static_cast<unsigned>(blocks), gy), dim3(kThreads), 0,
                         stream, a, o);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace spattn

// Host side of libspattn.so: argument validation, error state and launches.
// Every check runs before anything is enqueued; on failure nothing runs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "../../include/spattn.h"
#include "internal.h"

using spattn::CopySeg;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SP_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

int elem_bytes(int32_t dtype) {
  if (dtype == SP_F32) return 4;
  if (dtype == SP_BF16) return 2;
  return 0;
}

// Byte ranges [lo, hi) on the device address space.
bool ranges_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (abytes <= 0 || bbytes <= 0) return false;
  auto a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

// Checks that the element blocks [displs[r], displs[r] + sizes[r]) with sizes > 0 are disjoint.
bool blocks_disjoint(int32_t W, const int64_t* displs, const std::vector<int64_t>& sizes) {
  std::vector<std::pair<int64_t, int64_t>> iv;
  iv.reserve(W);
  for (int32_t r = 0; r < W; ++r)
    if (sizes[r] > 0) iv.emplace_back(displs[r], displs[r] + sizes[r]);
  std::sort(iv.begin(), iv.end());
  for (size_t i = 1; i < iv.size(); ++i)
    if (iv[i].first < iv[i - 1].second) return false;
  return true;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Launch grids are 32-bit counts of work-items: a call whose launch would
// exceed that is refused before anything is enqueued.
int grid_check(const char* fn, int64_t items) {
  if (items > spattn::kMaxItems)
    return fail(SP_ERANGE, "%s: a launch would need %lld work-items, more than the 2^32-1 a HIP grid holds", fn,
                static_cast<long long>(items));
  return SP_OK;
}

int launch_copies(const std::vector<CopySeg>& segs, int64_t outer, void* stream) {
  if (segs.empty()) return ok();
  if (int rc = grid_check("copy", spattn::segcopy_max_items(segs.data(), static_cast<int>(segs.size())))) return rc;
  (void)hipGetLastError();  // launches below report their own status
  hipError_t e = spattn::launch_segcopy(segs.data(), static_cast<int>(segs.size()), outer,
                                        as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "segmented copy launch");
  return ok();
}

}  // namespace

namespace {

// Checks shared by both attention entry points; fills the byte sizes of q/o,
// of all K (or V) tokens, and of lse.
int check_attn(const char* fn, int32_t dtype, int64_t sq, int64_t skv, int32_t H, int32_t d, float scale,
               bool allow512, int64_t* qb, int64_t* kb, int64_t* lb) {
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (sq < 0 || skv < 1 || H < 1) return fail(SP_EINVAL, "%s: need sq >= 0, skv >= 1, H >= 1", fn);
  const bool d512 = allow512 && dtype == SP_BF16 && d == 512;
  if (d != 64 && d != 128 && !d512)
    return fail(SP_EUNSUPPORTED, "%s: head size %d not supported (64, 128%s)", fn, d,
                allow512 ? "; 512 with bf16" : "");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(SP_EINVAL, "%s: scale must be finite and > 0", fn);
  int64_t qn, kn;
  if (!mul_ok(sq, int64_t(H) * d, &qn) || !mul_ok(skv, int64_t(H) * d, &kn) || !mul_ok(qn, eb, qb) ||
      !mul_ok(kn, eb, kb) || !mul_ok(sq, int64_t(H) * 4, lb))
    return fail(SP_ERANGE, "%s: size overflows int64", fn);
  if (int rc = grid_check(fn, dtype == SP_BF16 ? spattn::attn_bf16_items(sq, H, d, 1) : spattn::attn_f32_items(sq, H)))
    return rc;
  if (skv > (int64_t(1) << 31) - 256) return fail(SP_ERANGE, "%s: skv must be < 2^31", fn);
  if (sq > (int64_t(1) << 31) - 256) return fail(SP_ERANGE, "%s: sq must be < 2^31", fn);
  // The kernels address a 64-token K/V tile with 32-bit byte offsets.
  if (int64_t(H) * d * 4 * 64 > (int64_t(1) << 31) - 1)
    return fail(SP_ERANGE, "%s: H*d too large (64 tokens of K must span < 2 GiB)", fn);
  return SP_OK;
}

// The bf16 kernels move Q, K and V in 16-byte vectors and O in 8-byte ones;
// the float32 kernel uses element accesses.  lse is float32.
int check_attn_align(const char* fn, int32_t dtype, std::initializer_list<const void*> tensors, const float* lse) {
  const uintptr_t need = dtype == SP_BF16 ? 16 : 4;
  for (const void* p : tensors)
    if (reinterpret_cast<uintptr_t>(p) % need)
      return fail(SP_EINVAL, "%s: q, k, v, o (and every shard) must be %d-byte aligned for this dtype", fn, int(need));
  if (reinterpret_cast<uintptr_t>(lse) % 4) return fail(SP_EINVAL, "%s: lse must be 4-byte aligned", fn);
  return SP_OK;
}

}  // namespace

extern "C" {

int sp_abi_version(void) { return SPATTN_ABI_VERSION; }

const char* sp_last_error(void) { return g_err; }

int sp_shard_bounds(int64_t S, int32_t W, int32_t r, int64_t* start, int64_t* end) {
  if (!start || !end) return fail(SP_EINVAL, "sp_shard_bounds: null output pointer");
  if (W < 1) return fail(SP_EINVAL, "sp_shard_bounds: W must be >= 1 (got %d)", W);
  if (r < 0 || r >= W) return fail(SP_EINVAL, "sp_shard_bounds: rank %d outside [0, %d)", r, W);
  if (S < 0) return fail(SP_EINVAL, "sp_shard_bounds: S must be >= 0 (got %lld)", (long long)S);
  __int128 s = S;
  *start = static_cast<int64_t>((s * r) / W);
  *end = static_cast<int64_t>((s * (r + 1)) / W);
  return ok();
}

int sp_allgatherv_layout(int64_t S, int32_t W, int64_t outer, int64_t inner, int64_t* counts,
                         int64_t* displs) {
  if (!counts || !displs) return fail(SP_EINVAL, "sp_allgatherv_layout: null output array");
  if (W < 1) return fail(SP_EINVAL, "sp_allgatherv_layout: W must be >= 1 (got %d)", W);
  if (S < 0 || outer < 0 || inner < 0)
    return fail(SP_EINVAL, "sp_allgatherv_layout: S, outer and inner must be >= 0");
  int64_t tot;
  if (!mul_ok(outer, S, &tot) || !mul_ok(tot, inner, &tot))
    return fail(SP_ERANGE, "sp_allgatherv_layout: outer*S*inner overflows int64");
  int64_t off = 0;
  for (int32_t r = 0; r < W; ++r) {
    __int128 s = S;
    int64_t a = static_cast<int64_t>((s * r) / W), b = static_cast<int64_t>((s * (r + 1)) / W);
    counts[r] = outer * (b - a) * inner;  // <= tot, no overflow
    displs[r] = off;
    off += counts[r];
  }
  return ok();
}

int sp_allgatherv_layout_lens(int32_t W, const int64_t* seq_lens, int64_t outer, int64_t inner, int64_t* counts,
                              int64_t* displs) {
  const char* fn = "sp_allgatherv_layout_lens";
  if (!seq_lens || !counts || !displs) return fail(SP_EINVAL, "%s: null host array", fn);
  if (W < 1) return fail(SP_EINVAL, "%s: W must be >= 1 (got %d)", fn, W);
  if (outer < 0 || inner < 0) return fail(SP_EINVAL, "%s: outer and inner must be >= 0", fn);
  // Validate everything before writing an output.
  int64_t off = 0;
  for (int32_t r = 0; r < W; ++r) {
    if (seq_lens[r] < 0) return fail(SP_EINVAL, "%s: seq_lens[%d] < 0", fn, r);
    int64_t n;
    if (!mul_ok(outer, seq_lens[r], &n) || !mul_ok(n, inner, &n) || !add_ok(off, n, &off))
      return fail(SP_ERANGE, "%s: outer*sum(seq_lens)*inner overflows int64", fn);
  }
  off = 0;
  for (int32_t r = 0; r < W; ++r) {
    counts[r] = outer * seq_lens[r] * inner;  // checked above
    displs[r] = off;
    off += counts[r];
  }
  return ok();
}

int varlen_pack(int32_t dtype, int32_t W, const void* const* send, const int64_t* counts,
                const int64_t* displs, void* flat, int64_t flat_elems, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "varlen_pack: unknown dtype %d", dtype);
  if (W < 1) return fail(SP_EINVAL, "varlen_pack: W must be >= 1 (got %d)", W);
  if (!send || !counts || !displs) return fail(SP_EINVAL, "varlen_pack: null host array");
  if (flat_elems < 0) return fail(SP_EINVAL, "varlen_pack: flat_elems < 0");
  int64_t flat_bytes;
  if (!mul_ok(flat_elems, eb, &flat_bytes)) return fail(SP_ERANGE, "varlen_pack: flat size overflows");
  std::vector<int64_t> sizes(W);
  std::vector<CopySeg> segs;
  for (int32_t r = 0; r < W; ++r) {
    const int64_t c = counts[r], dsp = displs[r];
    if (c < 0 || dsp < 0)
      return fail(SP_EINVAL, "varlen_pack: rank %d has a negative count or displacement", r);
    if (c > flat_elems || dsp > flat_elems - c)
      return fail(SP_ERANGE, "varlen_pack: rank %d block [%lld, %lld) exceeds flat_elems %lld", r,
                  (long long)dsp, (long long)dsp + (long long)c, (long long)flat_elems);
    sizes[r] = c;
    if (c == 0) continue;
    if (!send[r]) return fail(SP_EINVAL, "varlen_pack: rank %d send pointer is null", r);
    if (!flat) return fail(SP_EINVAL, "varlen_pack: flat is null");
    if (ranges_overlap(send[r], c * eb, flat, flat_bytes))
      return fail(SP_EOVERLAP, "varlen_pack: rank %d send buffer overlaps flat", r);
    segs.push_back(CopySeg{static_cast<const char*>(send[r]), static_cast<char*>(flat) + dsp * eb,
                           c * eb, 0, 0});
  }
  if (!blocks_disjoint(W, displs, sizes))
    return fail(SP_EOVERLAP, "varlen_pack: destination blocks overlap");
  return launch_copies(segs, 1, stream);
}

int varlen_unpack(int32_t dtype, int32_t W, const void* flat, int64_t flat_elems,
                  const int64_t* displs, const int64_t* seq_lens, int64_t outer, int64_t inner,
                  void* out, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "varlen_unpack: unknown dtype %d", dtype);
  if (W < 1) return fail(SP_EINVAL, "varlen_unpack: W must be >= 1 (got %d)", W);
  if (!displs || !seq_lens) return fail(SP_EINVAL, "varlen_unpack: null host array");
  if (flat_elems < 0 || outer < 0 || inner < 0)
    return fail(SP_EINVAL, "varlen_unpack: negative flat_elems, outer or inner");
  int64_t flat_bytes;
  if (!mul_ok(flat_elems, eb, &flat_bytes)) return fail(SP_ERANGE, "varlen_unpack: flat size overflows");
  int64_t S = 0;
  std::vector<int64_t> sizes(W);
  for (int32_t r = 0; r < W; ++r) {
    const int64_t s = seq_lens[r], dsp = displs[r];
    if (s < 0 || dsp < 0)
      return fail(SP_EINVAL, "varlen_unpack: rank %d has a negative length or displacement", r);
    int64_t n;
    if (!add_ok(S, s, &S) || !mul_ok(outer, s, &n) || !mul_ok(n, inner, &n))
      return fail(SP_ERANGE, "varlen_unpack: sizes overflow int64");
    if (n > flat_elems || dsp > flat_elems - n)
      return fail(SP_ERANGE, "varlen_unpack: rank %d block [%lld, %lld) exceeds flat_elems %lld", r,
                  (long long)dsp, (long long)dsp + (long long)n, (long long)flat_elems);
    sizes[r] = n;
  }
  int64_t out_elems, out_bytes;
  if (!mul_ok(outer, S, &out_elems) || !mul_ok(out_elems, inner, &out_elems) ||
      !mul_ok(out_elems, eb, &out_bytes))
    return fail(SP_ERANGE, "varlen_unpack: output size overflows int64");
  if (!blocks_disjoint(W, displs, sizes))
    return fail(SP_EOVERLAP, "varlen_unpack: source blocks overlap");
  if (out_elems == 0) return ok();
  if (!flat || !out) return fail(SP_EINVAL, "varlen_unpack: null device pointer");
  if (ranges_overlap(out, out_bytes, flat, flat_bytes))
    return fail(SP_EOVERLAP, "varlen_unpack: out overlaps flat");
  std::vector<CopySeg> segs;
  int64_t a = 0;
  for (int32_t r = 0; r < W; ++r) {
    const int64_t s = seq_lens[r];
    if (s > 0 && inner > 0)
      segs.push_back(CopySeg{static_cast<const char*>(flat) + displs[r] * eb,
                             static_cast<char*>(out) + a * inner * eb, s * inner * eb,
                             s * inner * eb, S * inner * eb});
    a += s;
  }
  return launch_copies(segs, outer, stream);
}

int rope_apply(int32_t dtype, const void* x, void* y, int64_t s, int32_t H, int32_t d,
               int64_t pos0, double theta, int32_t style, void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "rope_apply: unknown dtype %d", dtype);
  if (style != SP_ROPE_HALF && style != SP_ROPE_INTERLEAVED)
    return fail(SP_EINVAL, "rope_apply: unknown style %d", style);
  if (s < 0 || H < 1) return fail(SP_EINVAL, "rope_apply: need s >= 0 and H >= 1");
  if (d < 2 || d > 1024 || (d & 1)) return fail(SP_EINVAL, "rope_apply: d must be even, 2..1024 (got %d)", d);
  if (!(std::isfinite(theta) && theta > 0.0)) return fail(SP_EINVAL, "rope_apply: theta must be finite and > 0");
  const int64_t lim = int64_t(1) << 53;
  if (pos0 <= -lim || pos0 >= lim || s >= lim || pos0 + s >= lim)
    return fail(SP_EINVAL, "rope_apply: positions must stay within +-2^53");
  int64_t n, bytes;
  if (!mul_ok(s, int64_t(H) * d, &n) || !mul_ok(n, eb, &bytes))
    return fail(SP_ERANGE, "rope_apply: size overflows int64");
  if (n == 0) return ok();
  if (!x || !y) return fail(SP_EINVAL, "rope_apply: null device pointer");
  if (x != y && ranges_overlap(x, bytes, y, bytes))
    return fail(SP_EOVERLAP, "rope_apply: x and y overlap without being equal");
  if (int rc = grid_check("rope_apply", spattn::rope_items(eb, s, d, style, x, y, false))) return rc;
  (void)hipGetLastError();
  hipError_t e = spattn::launch_rope(dtype, x, y, s, H, d, pos0, theta, style, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return ok();
}

int rope_apply_mx(int32_t dtype, const void* x, void* y, int64_t s, int32_t H, int32_t d, const int64_t* pos,
                  const int32_t* sections, double theta, int32_t style, void* stream) {
  const char* fn = "rope_apply_mx";
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (style != SP_ROPE_HALF && style != SP_ROPE_INTERLEAVED) return fail(SP_EINVAL, "%s: unknown style %d", fn, style);
  if (s < 0 || H < 1) return fail(SP_EINVAL, "%s: need s >= 0 and H >= 1", fn);
  if (d < 2 || d > 1024 || (d & 1)) return fail(SP_EINVAL, "%s: d must be even, 2..1024 (got %d)", fn, d);
  if (!(std::isfinite(theta) && theta > 0.0)) return fail(SP_EINVAL, "%s: theta must be finite and > 0", fn);
  if (!sections) return fail(SP_EINVAL, "%s: null sections", fn);
  if (sections[0] < 0 || sections[1] < 0 || sections[2] < 0 || sections[0] + sections[1] + sections[2] != d / 2)
    return fail(SP_EINVAL, "%s: sections must be >= 0 and add up to d/2 = %d pairs", fn, d / 2);
  int64_t n, bytes, pbytes;
  if (!mul_ok(s, int64_t(H) * d, &n) || !mul_ok(n, eb, &bytes) || !mul_ok(s, 3 * 8, &pbytes))
    return fail(SP_ERANGE, "%s: size overflows int64", fn);
  if (n == 0) return ok();
  if (!x || !y || !pos) return fail(SP_EINVAL, "%s: null device pointer", fn);
  if (x != y && ranges_overlap(x, bytes, y, bytes)) return fail(SP_EOVERLAP, "%s: x and y overlap without being equal", fn);
  if (ranges_overlap(pos, pbytes, y, bytes)) return fail(SP_EOVERLAP, "%s: positions overlap y", fn);
  const int sec[3] = {sections[0], sections[1], sections[2]};
  if (int rc = grid_check(fn, spattn::rope_items(eb, s, d, style, x, y, false))) return rc;
  (void)hipGetLastError();
  hipError_t e = spattn::launch_rope_mx(dtype, x, y, s, H, d, pos, sec, theta, style, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return ok();
}

int sp_tile_bounds(int64_t Hh, int64_t Ww, int32_t pr, int32_t pc, int32_t p, int64_t* out) {
  const char* fn = "sp_tile_bounds";
  if (!out) return fail(SP_EINVAL, "%s: null output", fn);
  if (pr < 1 || pc < 1) return fail(SP_EINVAL, "%s: need pr, pc >= 1", fn);
  if (int64_t(pr) * pc > (int64_t(1) << 31) - 1) return fail(SP_ERANGE, "%s: pr*pc too large", fn);
  if (p < 0 || int64_t(p) >= int64_t(pr) * pc) return fail(SP_EINVAL, "%s: block %d outside [0, pr*pc)", fn, p);
  if (Hh < 0 || Ww < 0) return fail(SP_EINVAL, "%s: negative grid size", fn);
  const int32_t i = p / pc, j = p % pc;
  const __int128 h = Hh, w = Ww;
  out[0] = static_cast<int64_t>((h * i) / pr);
  out[1] = static_cast<int64_t>((h * (i + 1)) / pr);
  out[2] = static_cast<int64_t>((w * j) / pc);
  out[3] = static_cast<int64_t>((w * (j + 1)) / pc);
  return ok();
}

namespace {

// Copies between channels-last rasters [Hh, Ww, C] and their pr*pc blocks
// laid out one after another in block order (each block row-major), for n
// (raster, flat) pairs of one shape.  One segment per (pair, block) with one
// outer step per pixel row of the block, all in one batch of copies.
constexpr int32_t kMaxTilePairs = 16;

int tile_copy(const char* fn, bool to_flat, int32_t dtype, int32_t npair, const void* const* rasters, int64_t Hh,
              int64_t Ww, int64_t C, int32_t pr, int32_t pc, const void* const* flats, int64_t flat_elems,
              void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (npair < 1 || npair > kMaxTilePairs) return fail(SP_EINVAL, "%s: need 1 <= n <= %d", fn, kMaxTilePairs);
  if (!rasters || !flats) return fail(SP_EINVAL, "%s: null pointer table", fn);
  if (pr < 1 || pc < 1 || int64_t(pr) * pc > 65536) return fail(SP_EINVAL, "%s: need 1 <= pr*pc <= 65536", fn);
  if (Hh < 0 || Ww < 0 || C < 0 || flat_elems < 0) return fail(SP_EINVAL, "%s: negative size", fn);
  int64_t n, bytes;
  if (!mul_ok(Hh, Ww, &n) || !mul_ok(n, C, &n) || !mul_ok(n, eb, &bytes))
    return fail(SP_ERANGE, "%s: size overflows int64", fn);
  if (flat_elems < n) return fail(SP_ERANGE, "%s: flat holds %lld elements, the blocks need %lld", fn,
                                  (long long)flat_elems, (long long)n);
  if (n == 0) return ok();
  for (int32_t a = 0; a < npair; ++a) {
    if (!rasters[a] || !flats[a]) return fail(SP_EINVAL, "%s: null device pointer", fn);
    // The written buffers (flats when packing, rasters when unpacking) must
    // not overlap any buffer of the call.
    const void* wa = to_flat ? flats[a] : rasters[a];
    for (int32_t b = 0; b < npair; ++b) {
      if (ranges_overlap(wa, bytes, to_flat ? rasters[b] : flats[b], bytes))
        return fail(SP_EOVERLAP, "%s: raster and flat overlap", fn);
      if (b != a && ranges_overlap(wa, bytes, to_flat ? flats[b] : rasters[b], bytes))
        return fail(SP_EOVERLAP, "%s: two output buffers overlap", fn);
    }
  }
  const int64_t rowpitch = Ww * C * eb;  // bytes per raster row
  std::vector<CopySeg> segs;
  for (int32_t a = 0; a < npair; ++a) {
    int64_t off = 0;  // element offset of the current block in flat
    for (int32_t i = 0; i < pr; ++i) {
      const __int128 h = Hh, w = Ww;
      const int64_t r0 = static_cast<int64_t>((h * i) / pr), r1 = static_cast<int64_t>((h * (i + 1)) / pr);
      for (int32_t j = 0; j < pc; ++j) {
        const int64_t c0 = static_cast<int64_t>((w * j) / pc), c1 = static_cast<int64_t>((w * (j + 1)) / pc);
        const int64_t bw = (c1 - c0) * C * eb;  // bytes per block row
        char* fl = static_cast<char*>(const_cast<void*>(flats[a])) + off * eb;
        char* ra = static_cast<char*>(const_cast<void*>(rasters[a])) + r0 * rowpitch + c0 * C * eb;
        if (to_flat) segs.push_back(CopySeg{ra, fl, bw, rowpitch, bw, r1 - r0});
        else segs.push_back(CopySeg{fl, ra, bw, bw, rowpitch, r1 - r0});
        off += (r1 - r0) * (c1 - c0) * C;
      }
    }
  }
  // one segment per (pair, block), each with its own number of pixel rows
  return launch_copies(segs, 0, stream);
}

}  // namespace

int tile_pack(int32_t dtype, const void* raster, int64_t Hh, int64_t Ww, int64_t C, int32_t pr, int32_t pc,
              void* flat, int64_t flat_elems, void* stream) {
  const void* fl = flat;
  return tile_copy("tile_pack", true, dtype, 1, &raster, Hh, Ww, C, pr, pc, &fl, flat_elems, stream);
}

int tile_pack_n(int32_t dtype, int32_t n, const void* const* rasters, int64_t Hh, int64_t Ww, int64_t C, int32_t pr,
                int32_t pc, void* const* flats, int64_t flat_elems, void* stream) {
  return tile_copy("tile_pack_n", true, dtype, n, rasters, Hh, Ww, C, pr, pc,
                   const_cast<const void* const*>(flats), flat_elems, stream);
}

int tile_unpack(int32_t dtype, const void* flat, int64_t flat_elems, int64_t Hh, int64_t Ww, int64_t C, int32_t pr,
                int32_t pc, void* raster, void* stream) {
  const void* ra = raster;
  return tile_copy("tile_unpack", false, dtype, 1, &ra, Hh, Ww, C, pr, pc, &flat, flat_elems, stream);
}

int qk_norm_rope(int32_t dtype, const void* x, void* y, int64_t s, int32_t H, int32_t d, const float* gamma,
                 double eps, int64_t pos0, const int64_t* pos, const int32_t* sections, double theta, int32_t style,
                 void* stream) {
  const char* fn = "qk_norm_rope";
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(SP_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (style != SP_ROPE_HALF && style != SP_ROPE_INTERLEAVED) return fail(SP_EINVAL, "%s: unknown style %d", fn, style);
  if (s < 0 || H < 1) return fail(SP_EINVAL, "%s: need s >= 0 and H >= 1", fn);
  if (d < 2 || d > 1024 || (d & 1)) return fail(SP_EINVAL, "%s: d must be even, 2..1024 (got %d)", fn, d);
  if (!(std::isfinite(theta) && theta > 0.0)) return fail(SP_EINVAL, "%s: theta must be finite and > 0", fn);
  if (!(std::isfinite(eps) && eps >= 0.0 && eps <= 3.0e38)) return fail(SP_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (pos) {
    if (!sections) return fail(SP_EINVAL, "%s: null sections with explicit positions", fn);
    if (sections[0] < 0 || sections[1] < 0 || sections[2] < 0 || sections[0] + sections[1] + sections[2] != d / 2)
      return fail(SP_EINVAL, "%s: sections must be >= 0 and add up to d/2 = %d pairs", fn, d / 2);
  } else {
    const int64_t lim = int64_t(1) << 53;
    if (pos0 <= -lim || pos0 >= lim || s >= lim || pos0 + s >= lim)
      return fail(SP_EINVAL, "%s: positions must stay within +-2^53", fn);
  }
  int64_t n, bytes, pbytes;
  if (!mul_ok(s, int64_t(H) * d, &n) || !mul_ok(n, eb, &bytes) || !mul_ok(s, 3 * 8, &pbytes))
    return fail(SP_ERANGE, "%s: size overflows int64", fn);
  if (n == 0) return ok();
  if (!x || !y || !gamma) return fail(SP_EINVAL, "%s: null device pointer", fn);
  if (x != y && ranges_overlap(x, bytes, y, bytes)) return fail(SP_EOVERLAP, "%s: x and y overlap without being equal", fn);
  if (ranges_overlap(gamma, int64_t(d) * 4, y, bytes)) return fail(SP_EOVERLAP, "%s: gamma overlaps y", fn);
  if (pos && ranges_overlap(pos, pbytes, y, bytes)) return fail(SP_EOVERLAP, "%s: positions overlap y", fn);
  if (!spattn::rows_pairs_per_lane(d, style, eb, x, y))
    return fail(SP_EUNSUPPORTED,
                "%s: d = %d with these buffers: a head row must split into at most 64 lanes of 1, 2, 4 or 8 pairs "
                "with x and y aligned to that many elements", fn, d);
  const int sec[3] = {pos ? sections[0] : d / 2, pos ? sections[1] : 0, pos ? sections[2] : 0};
  if (int rc = grid_check(fn, spattn::rope_items(eb, s, d, style, x, y, true))) return rc;
  (void)hipGetLastError();
  hipError_t e = spattn::launch_qk_norm_rope(dtype, x, y, s, H, d, gamma, static_cast<float>(eps), pos0, pos, sec,
                                             theta, style, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "qk_norm_rope launch");
  return ok();
}

int sp_av_positions(int64_t T, int64_t Hh, int64_t Ww, int64_t n_audio, int64_t a, int64_t b, int64_t* out) {
  const char* fn = "sp_av_positions";
  if (T < 0 || Hh < 0 || Ww < 0 || n_audio < 0) return fail(SP_EINVAL, "%s: negative grid size", fn);
  int64_t hw, V, S;
  if (!mul_ok(Hh, Ww, &hw) || !mul_ok(T, hw, &V) || !add_ok(V, n_audio, &S))
    return fail(SP_ERANGE, "%s: grid size overflows int64", fn);
  if (a < 0 || a > b || b > S) return fail(SP_EINVAL, "%s: token range [%lld, %lld) outside [0, %lld)", fn,
                                           static_cast<long long>(a), static_cast<long long>(b),
                                           static_cast<long long>(S));
  if (b > a && !out) return fail(SP_EINVAL, "%s: null output", fn);
  for (int64_t i = a; i < b; ++i) {
    int64_t* o = out + (i - a) * 3;
    if (i < V) {
      o[0] = i / hw;
      o[1] = (i / Ww) % Hh;
      o[2] = i % Ww;
    } else {
      o[0] = i - V;
      o[1] = 0;
      o[2] = 0;
    }
  }
  return ok();
}


int shard_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t sq, int64_t skv, int32_t H, int32_t d, float scale, void* stream) {
  int64_t qb, kb, lb;
  if (int rc = check_attn("shard_attn_fwd", dtype, sq, skv, H, d, scale, true, &qb, &kb, &lb)) return rc;
  if (sq == 0) return ok();
  if (!q || !k || !v || !o) return fail(SP_EINVAL, "shard_attn_fwd: null device pointer");
  if (int rc = check_attn_align("shard_attn_fwd", dtype, {q, k, v, o}, lse)) return rc;
  if (ranges_overlap(o, qb, q, qb) || ranges_overlap(o, qb, k, kb) || ranges_overlap(o, qb, v, kb))
    return fail(SP_EOVERLAP, "shard_attn_fwd: o overlaps an input");
  if (lse && (ranges_overlap(lse, lb, q, qb) || ranges_overlap(lse, lb, k, kb) ||
              ranges_overlap(lse, lb, v, kb) || ranges_overlap(lse, lb, o, qb)))
    return fail(SP_EOVERLAP, "shard_attn_fwd: lse overlaps another buffer");
  (void)hipGetLastError();
  hipError_t e;
  if (dtype == SP_BF16)
    e = spattn::launch_attn_bf16(q, k, v, o, lse, sq, skv, H, d, scale, as_stream(stream));
  else
    e = spattn::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                static_cast<const float*>(v), static_cast<float*>(o), lse, sq, skv, H,
                                d, scale, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

int64_t sp_attn_split_workspace(int64_t sq, int32_t H, int32_t d, int32_t nsplit) {
  if (sq < 0 || H < 1 || d < 1 || nsplit < 1) return fail(SP_EINVAL, "sp_attn_split_workspace: bad arguments");
  int64_t on, ob, ln, lbytes;
  if (sq > (int64_t(1) << 60)) return fail(SP_ERANGE, "sp_attn_split_workspace: size overflows int64");
  if (!mul_ok(spattn::split_rows(sq, d), int64_t(H) * d, &on) || !mul_ok(on, int64_t(nsplit) * 4, &ob) ||
      !mul_ok(sq, int64_t(H), &ln) ||
      !mul_ok(ln, int64_t(nsplit) * 4, &lbytes) || ob > (int64_t(1) << 60) || lbytes > (int64_t(1) << 60))
    return fail(SP_ERANGE, "sp_attn_split_workspace: size overflows int64");
  ok();
  return ((ob + 255) / 256) * 256 + lbytes;
}

namespace {

// Validation shared by the split entry points, everything but the
// workspace: fills the byte sizes of q/o, K (or V) and lse and the workspace
// the call needs.  *skip is set when sq == 0 (nothing to enqueue).
int check_split(const char* fn, int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                int64_t sq, int64_t skv, int32_t H, int32_t d, float scale, int32_t nsplit, int64_t* qb,
                int64_t* kb, int64_t* lb, int64_t* need, bool* skip) {
  *skip = false;
  if (int rc = check_attn(fn, dtype, sq, skv, H, d, scale, true, qb, kb, lb)) return rc;
  if (dtype != SP_BF16) return fail(SP_EUNSUPPORTED, "%s: bf16 only", fn);
  if (nsplit < 1 || nsplit > 1024 || nsplit > (skv + 63) / 64)
    return fail(SP_EINVAL, "%s: nsplit must be in [1, min(1024, ceil(skv / 64))] (got %d)", fn, nsplit);
  *need = sp_attn_split_workspace(sq, H, d, nsplit);
  if (*need < 0) return static_cast<int>(*need);
  if (sq == 0) {
    *skip = true;
    return SP_OK;
  }
  if (!q || !k || !v || !o) return fail(SP_EINVAL, "%s: null device pointer", fn);
  if (int rc = check_attn_align(fn, dtype, {q, k, v, o}, lse)) return rc;
  if (int rc = grid_check(fn, spattn::attn_bf16_items(sq, H, d, nsplit))) return rc;
  if (int rc = grid_check(fn, spattn::attn_merge_items(sq, H, d))) return rc;
  if (ranges_overlap(o, *qb, q, *qb) || ranges_overlap(o, *qb, k, *kb) || ranges_overlap(o, *qb, v, *kb))
    return fail(SP_EOVERLAP, "%s: o overlaps an input", fn);
  if (lse && (ranges_overlap(lse, *lb, q, *qb) || ranges_overlap(lse, *lb, k, *kb) ||
              ranges_overlap(lse, *lb, v, *kb) || ranges_overlap(lse, *lb, o, *qb)))
    return fail(SP_EOVERLAP, "%s: lse overlaps another buffer", fn);
  return SP_OK;
}

// Partial outputs at the start of the workspace, partial LSEs after them
// (at the next 256-byte boundary).
int launch_split_in(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse, int64_t sq,
                    int64_t skv, int32_t H, int32_t d, float scale, int32_t nsplit, void* workspace, void* stream) {
  const int64_t ob = spattn::split_rows(sq, d) * H * d * int64_t(nsplit) * 4;  // checked by the size query
  float* opart = static_cast<float*>(workspace);
  float* lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((ob + 255) / 256) * 256);
  (void)hipGetLastError();
  hipError_t e = spattn::launch_attn_bf16_split(q, k, v, o, lse, sq, skv, H, d, scale, nsplit, opart, lpart,
                                                as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // namespace

int shard_attn_fwd_split(int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t sq, int64_t skv, int32_t H, int32_t d, float scale, int32_t nsplit,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  const char* fn = "shard_attn_fwd_split";
  int64_t qb, kb, lb, need;
  bool skip;
  if (int rc = check_split(fn, dtype, q, k, v, o, lse, sq, skv, H, d, scale, nsplit, &qb, &kb, &lb, &need, &skip))
    return rc;
  if (skip) return ok();
  if (!workspace) return fail(SP_EINVAL, "%s: null workspace", fn);
  if (workspace_bytes < need)
    return fail(SP_ERANGE, "%s: workspace holds %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                (long long)need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(SP_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (ranges_overlap(workspace, need, q, qb) || ranges_overlap(workspace, need, k, kb) ||
      ranges_overlap(workspace, need, v, kb) || ranges_overlap(workspace, need, o, qb) ||
      (lse && ranges_overlap(workspace, need, lse, lb)))
    return fail(SP_EOVERLAP, "%s: workspace overlaps another buffer", fn);
  return launch_split_in(fn, q, k, v, o, lse, sq, skv, H, d, scale, nsplit, workspace, stream);
}

int shard_attn_fwd_split_noalloc(int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                                 int64_t sq, int64_t skv, int32_t H, int32_t d, float scale, int32_t nsplit,
                                 void* stream) {
  const char* fn = "shard_attn_fwd_split_noalloc";
  int64_t qb, kb, lb, need;
  bool skip;
  if (int rc = check_split(fn, dtype, q, k, v, o, lse, sq, skv, H, d, scale, nsplit, &qb, &kb, &lb, &need, &skip))
    return rc;
  if (skip) return ok();
  if (need > spattn::kScratchBytes)
    return fail(SP_ERANGE, "%s: the call needs %lld bytes of partials, more than the %lld-byte device scratch", fn,
                (long long)need, (long long)spattn::kScratchBytes);
  void* scratch = nullptr;
  if (hipError_t e = spattn::scratch_address(&scratch)) return hip_fail(e, "scratch address");
  return launch_split_in(fn, q, k, v, o, lse, sq, skv, H, d, scale, nsplit, scratch, stream);
}

int shard_attn_fwd_gv(int32_t dtype, const void* q, int32_t W, const void* const* k_shards,
                      const void* const* v_shards, const int64_t* seq_lens, void* o, float* lse, int64_t sq,
                      int32_t H, int32_t d, float scale, void* stream) {
  const char* fn = "shard_attn_fwd_gv";
  if (W < 1) return fail(SP_EINVAL, "%s: W must be >= 1", fn);
  if (W > spattn::kMaxShards) return fail(SP_EUNSUPPORTED, "%s: at most %d shards", fn, spattn::kMaxShards);
  if (!k_shards || !v_shards || !seq_lens) return fail(SP_EINVAL, "%s: null host array", fn);
  spattn::KvShards kv{};
  kv.W = W;
  kv.start[0] = 0;
  for (int32_t r = 0; r < W; ++r) {
    if (seq_lens[r] < 0) return fail(SP_EINVAL, "%s: seq_lens[%d] < 0", fn, r);
    if (!add_ok(kv.start[r], seq_lens[r], &kv.start[r + 1])) return fail(SP_ERANGE, "%s: sum of seq_lens overflows", fn);
    kv.k[r] = k_shards[r];
    kv.v[r] = v_shards[r];
  }
  const int64_t skv = kv.start[W];
  int64_t qb, kb, lb;
  if (int rc = check_attn(fn, dtype, sq, skv, H, d, scale, false, &qb, &kb, &lb)) return rc;
  if (sq == 0) return ok();
  if (!q || !o) return fail(SP_EINVAL, "%s: null device pointer", fn);
  if (int rc = check_attn_align(fn, dtype, {q, o}, lse)) return rc;
  for (int32_t r = 0; r < W; ++r)
    if (seq_lens[r] > 0)
      if (int rc = check_attn_align(fn, dtype, {kv.k[r], kv.v[r]}, nullptr)) return rc;
  const int64_t tok_bytes = int64_t(H) * d * elem_bytes(dtype);
  if (ranges_overlap(o, qb, q, qb)) return fail(SP_EOVERLAP, "%s: o overlaps q", fn);
  if (lse && (ranges_overlap(lse, lb, q, qb) || ranges_overlap(lse, lb, o, qb)))
    return fail(SP_EOVERLAP, "%s: lse overlaps another buffer", fn);
  for (int32_t r = 0; r < W; ++r) {
    const int64_t nb = seq_lens[r] * tok_bytes;  // <= kb, no overflow
    if (nb == 0) continue;
    if (!kv.k[r] || !kv.v[r]) return fail(SP_EINVAL, "%s: null shard %d with %lld tokens", fn, r,
                                          static_cast<long long>(seq_lens[r]));
    if (ranges_overlap(o, qb, kv.k[r], nb) || ranges_overlap(o, qb, kv.v[r], nb))
      return fail(SP_EOVERLAP, "%s: o overlaps shard %d", fn, r);
    if (lse && (ranges_overlap(lse, lb, kv.k[r], nb) || ranges_overlap(lse, lb, kv.v[r], nb)))
      return fail(SP_EOVERLAP, "%s: lse overlaps shard %d", fn, r);
  }
  (void)hipGetLastError();
  hipError_t e;
  if (dtype == SP_BF16)
    e = spattn::launch_attn_bf16_gv(q, kv, o, lse, sq, H, d, scale, as_stream(stream));
  else
    e = spattn::launch_attn_f32_gv(static_cast<const float*>(q), kv, static_cast<float*>(o), lse, sq, H, d, scale,
                                   as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

}  // extern "C"

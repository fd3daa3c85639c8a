/*
 * spattn.h -- C ABI of libspattn.so: one rank's share of packed-token
 * sequence-parallel DiT self-attention on AMD Instinct MI355X (gfx950).
 *
 * The method (page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU 中 DiT 序列并行与
 * peer-copy 双后端机制", sections 机制一 and 机制二/后端 A): a packed audio+video
 * token sequence of S tokens is split over W ranks; each rank rotates its
 * local slice with RoPE, the ranks' K/V shards are reassembled into the full
 * sequence with AllGatherV semantics (per-rank element counts and
 * displacements into one flat buffer, then narrow/view/concat), attention runs
 * with the rank's local queries against the full K/V, and the per-rank outputs
 * are concatenated back along the sequence.  Page "NPU HunyuanImage-3.0模型推理
 * 优化实践" adds the per-head norm in front of the rotation (section 计算分解)
 * and the VAE's spatial block split (section VAE并行优化), whose attention
 * gathers the K/V of all blocks the same way.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, contiguous and token-major: [tokens, H, d] (batch 1);
 *    a VAE feature map is channels-last [Hh, Ww, C], i.e. Hh*Ww tokens of one
 *    head of C channels.
 *  - Element types: SP_F32 (IEEE binary32) or SP_BF16 (bfloat16 bit patterns).
 *  - Counts, displacements and lengths are in ELEMENTS, as in AllGatherV.
 *  - Device pointers are HIP device memory of the current device; host arrays
 *    are read during the call only.  The caller allocates and frees every
 *    buffer; the library keeps no pointer after a call returns and makes no
 *    device allocation (scratch memory, where a call needs it, is a
 *    caller-owned workspace argument).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously on it; nothing synchronises with the host.
 *    The caller synchronises the stream before reading results, as the
 *    page's collective path does (async on the current stream, then one
 *    synchronize()).  Faults during execution therefore surface at the
 *    caller's synchronisation.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    error nothing is enqueued, a negative status is returned and
 *    sp_last_error() describes the failure.  There is no fallback path.
 *    This includes the size of every launch a call would make: a HIP grid
 *    holds at most 2^32 - 1 work-items, and a call needing more returns
 *    SP_ERANGE.  SP_EHIP (the runtime refusing a launch that passed those
 *    checks) is the one status after which launches of the same call that
 *    came before the refused one may still run.
 */
#ifndef SPATTN_H
#define SPATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPATTN_ABI_VERSION 1

/* Status codes. */
enum {
  SP_OK = 0,
  SP_EINVAL = -1,        /* malformed argument (negative size, null pointer with data, bad enum) */
  SP_EUNSUPPORTED = -2,  /* well-formed but not implemented (head size, dtype) */
  SP_ERANGE = -3,        /* a block or index falls outside its buffer, or a size overflows int64 */
  SP_EOVERLAP = -4,      /* destination blocks overlap each other, or an output overlaps an input */
  SP_EHIP = -5           /* the HIP runtime refused a launch; message holds the HIP error */
};

/* Element types. */
enum { SP_F32 = 0, SP_BF16 = 1 };

/* RoPE pairings: (j, j + d/2) ("rotate_half") or (2j, 2j + 1). */
enum { SP_ROPE_HALF = 0, SP_ROPE_INTERLEAVED = 1 };

/* ABI version of the loaded library (SPATTN_ABI_VERSION). */
int sp_abi_version(void);

/* Message of the last failing call on this thread ("" if none).  The string
 * is owned by the library and valid until the next call on the same thread. */
const char* sp_last_error(void);

/*
 * sp_shard_bounds -- token range [*start, *end) of rank r.
 * Defined by section 机制一: rank r owns [S*r // W, S*(r+1) // W) (floor
 * division; computed exactly in 128-bit integers, so any S >= 0 is valid).
 * Shards differ in length by at most one token when W does not divide S; a
 * rank may own zero tokens when S < W.
 * Errors: SP_EINVAL if W < 1, r outside [0, W), S < 0 or a null output.
 * Host-only: touches no device.
 */
int sp_shard_bounds(int64_t S, int32_t W, int32_t r, int64_t* start, int64_t* end);

/*
 * sp_allgatherv_layout -- AllGatherV counts and displacements (elements).
 * Defined by section 后端 A (counts = element counts per rank,
 * displacements = target offsets in the flat receive buffer).  Rank r's
 * local tensor has shape [outer, s_r, inner]; counts[r] = outer*s_r*inner and
 * displs[r] = counts[0] + ... + counts[r-1] (rank order, no gaps).
 * counts and displs are host arrays of W entries written by the call.
 * Errors: SP_EINVAL (W < 1, negative outer/inner, null arrays),
 * SP_ERANGE (outer*S*inner overflows int64).  Host-only.
 */
int sp_allgatherv_layout(int64_t S, int32_t W, int64_t outer, int64_t inner,
                         int64_t* counts, int64_t* displs);

/*
 * sp_allgatherv_layout_lens -- AllGatherV counts and displacements for any
 * per-rank lengths along any concatenation axis (elements).
 * Defined by section 后端 A of the same page: exchange(rank, tensors,
 * cat_dims) gathers tensors that agree outside the concatenation axis, with
 * counts = element counts per rank and displacements = target offsets in the
 * flat receive buffer.  Rank r's tensor is viewed as [outer, seq_lens[r],
 * inner] (outer = product of the sizes before the concatenation axis, inner =
 * product after it); counts[r] = outer*seq_lens[r]*inner and displs[r] =
 * counts[0] + ... + counts[r-1] (rank order, no gaps).  With seq_lens from
 * sp_shard_bounds it equals sp_allgatherv_layout.
 *   seq_lens  host array of W lengths along the concatenation axis (>= 0)
 *   counts, displs  host arrays of W entries written by the call (untouched
 *                   on error)
 * Errors: SP_EINVAL (W < 1, a negative length, outer or inner, null arrays),
 * SP_ERANGE (outer*sum(seq_lens)*inner overflows int64).  Host-only.
 */
int sp_allgatherv_layout_lens(int32_t W, const int64_t* seq_lens, int64_t outer, int64_t inner,
                              int64_t* counts, int64_t* displs);

/*
 * varlen_pack -- the data movement of one AllGatherV into a flat buffer.
 * Defined by section 后端 A: for every rank r and 0 <= i < counts[r],
 * flat[displs[r] + i] = send[r][i].  Bits are copied unchanged; elements of
 * `flat` outside every block are left untouched.
 *   send    host array of W device pointers (rank r's shard, counts[r] elements)
 *   counts  host array of W element counts (>= 0)
 *   displs  host array of W element offsets into flat (>= 0), any order,
 *           gaps allowed (MPI AllGatherV semantics)
 *   flat    device buffer of flat_elems elements
 * Errors: SP_EINVAL (bad dtype, W < 1, negative count/displacement, null
 * pointer with a nonzero count), SP_ERANGE (a block past flat_elems),
 * SP_EOVERLAP (two blocks overlap, or a source overlaps flat), SP_EHIP.
 */
int varlen_pack(int32_t dtype, int32_t W, const void* const* send,
                const int64_t* counts, const int64_t* displs,
                void* flat, int64_t flat_elems, void* stream);

/*
 * varlen_unpack -- narrow -> view -> concat of an AllGatherV receive buffer.
 * Defined by section 后端 A: rank r's block of flat, starting at displs[r] and
 * holding outer*seq_lens[r]*inner elements, is viewed as
 * [outer, seq_lens[r], inner]; the views are concatenated along the sequence
 * axis into out = [outer, sum(seq_lens), inner]:
 *   out[o, a_r + t, k] = flat[displs[r] + (o*seq_lens[r] + t)*inner + k],
 *   a_r = seq_lens[0] + ... + seq_lens[r-1].
 * With outer == 1 every rank's block is one contiguous copy.
 *   flat      device buffer of flat_elems elements (read)
 *   displs, seq_lens  host arrays of W entries
 *   out       device buffer of outer*sum(seq_lens)*inner elements (written)
 * Errors: SP_EINVAL (bad dtype, W < 1, negative sizes, null pointers with
 * data), SP_ERANGE (a block past flat_elems, size overflow), SP_EOVERLAP
 * (blocks overlap each other, or out overlaps flat), SP_EHIP.
 */
int varlen_unpack(int32_t dtype, int32_t W, const void* flat, int64_t flat_elems,
                  const int64_t* displs, const int64_t* seq_lens,
                  int64_t outer, int64_t inner, void* out, void* stream);

/*
 * rope_apply -- rotary position embedding of a rank's local slice.
 * Section 机制一 slices the RoPE frequency table with the rank's token range,
 * so positions are absolute: token t of the slice sits at p = pos0 + t (pos0
 * is the rank's start from sp_shard_bounds).  Page "NPU HunyuanImage-3.0模型推理
 * 优化实践", section 消除旋转位置编码冗余cast算子, applies the rotation to query
 * and key states only (apply_rotary_pos_emb(q, k, cos, sin)); V is never
 * rotated.  For pair j in 0 .. d/2-1 with angle phi = p * theta^(-2j/d):
 *   y1 = x1 cos(phi) - x2 sin(phi),  y2 = x2 cos(phi) + x1 sin(phi),
 * pairs (x1, x2) = (x[j], x[j + d/2]) for SP_ROPE_HALF and (x[2j], x[2j+1])
 * for SP_ROPE_INTERLEAVED.  phi and its range reduction are float64, the
 * rotation float32, the result rounded to dtype (nearest-even).
 *   x, y  device [s, H, d] of dtype; y == x (in place) is allowed, any other
 *         overlap is not.
 * Errors: SP_EINVAL (bad dtype/style, s < 0, H < 1, d odd or > 1024,
 * theta not finite and > 0, |pos0| or |pos0 + s| >= 2^53, null pointers
 * with data), SP_EOVERLAP (partial overlap of x and y), SP_EHIP.
 */
int rope_apply(int32_t dtype, const void* x, void* y, int64_t s, int32_t H, int32_t d,
               int64_t pos0, double theta, int32_t style, void* stream);

/*
 * rope_apply_mx -- multi-axis rotary embedding with explicit positions.
 * Section 机制一 slices "the RoPE frequency table" with the rank's token
 * range without defining the table; for packed video tokens the table is
 * read here as the usual multi-axis form.  The d/2 pairs (paired as in
 * rope_apply) are split into consecutive groups of sections[0], sections[1]
 * and sections[2] pairs, one per axis; pair j' of axis a (0-based inside its
 * group) rotates by phi = pos[t][a] * theta^(-2 j' / (2 sections[a])).  With
 * sections = {d/2, 0, 0} and pos[t][0] = pos0 + t this is rope_apply
 * (same arithmetic, same bits).  Precision as rope_apply.
 *   x, y       device [s, H, d] of dtype; y == x allowed, other overlap not
 *   pos        device int64 [s, 3]: token t's position on each axis; values
 *              must satisfy |pos| < 2^53 (device data, not checked)
 *   sections   host array of 3 pair counts, each >= 0, summing to d/2
 * Errors: as rope_apply, plus SP_EINVAL (null or invalid sections, null pos
 * with s > 0) and SP_EOVERLAP (pos overlaps y).
 */
int rope_apply_mx(int32_t dtype, const void* x, void* y, int64_t s, int32_t H, int32_t d,
                  const int64_t* pos, const int32_t* sections, double theta, int32_t style, void* stream);

/*
 * sp_tile_bounds -- spatial block of process p in the VAE split (host).
 * Page "NPU HunyuanImage-3.0模型推理优化实践", section VAE并行优化: a large image
 * is cut along height and width into blocks, one per process.  Processes are
 * numbered row-major over a pr x pc block grid (p = i*pc + j); each axis is
 * cut like the token ranges of section 机制一:
 *   out = {Hh*i/pr, Hh*(i+1)/pr, Ww*j/pc, Ww*(j+1)/pc}   (floor, exact)
 * i.e. rows [out[0], out[1]) and columns [out[2], out[3]).
 * Errors: SP_EINVAL (pr or pc < 1, p outside [0, pr*pc), negative sizes, null
 * out), SP_ERANGE (pr*pc >= 2^31).  Host-only.
 */
int sp_tile_bounds(int64_t Hh, int64_t Ww, int32_t pr, int32_t pc, int32_t p, int64_t* out);

/*
 * tile_pack / tile_unpack -- between a raster and its blocks in process order.
 * Section VAE并行优化 splits the input over the processes by its spatial
 * dimensions and, at the end, gathers the blocks in two stages and puts each
 * back at its original position.  With the blocks of sp_tile_bounds laid out
 * one after another in process order, each row-major ([h_p, w_p, C]):
 *   tile_pack:   flat  <- blocks of raster   (the split; also the order of
 *                the AllGatherV receive buffer of the gathered K and V)
 *   tile_unpack: raster <- blocks of flat    (second stage of the gather)
 *   raster  device [Hh, Ww, C] of dtype, channels last
 *   flat    device, at least Hh*Ww*C elements; block p starts at element
 *           C * sum_{q<p} h_q*w_q
 * Bit-exact copies.  Errors: SP_EINVAL (bad dtype, pr*pc outside [1, 65536],
 * negative sizes, null pointers with data), SP_ERANGE (flat too small, size
 * overflow), SP_EOVERLAP (raster and flat overlap), SP_EHIP.
 */
int tile_pack(int32_t dtype, const void* raster, int64_t Hh, int64_t Ww, int64_t C, int32_t pr, int32_t pc,
              void* flat, int64_t flat_elems, void* stream);
int tile_unpack(int32_t dtype, const void* flat, int64_t flat_elems, int64_t Hh, int64_t Ww, int64_t C, int32_t pr,
                int32_t pc, void* raster, void* stream);

/*
 * tile_pack_n -- tile_pack of n rasters of one shape in one batch of copies.
 * Section VAE并行优化 gathers the K and V blocks of every process before the
 * attention; this packs both (or any n <= 16 tensors) with one launch instead
 * of one per tensor: flats[a] <- blocks of rasters[a], each exactly as
 * tile_pack.
 *   rasters, flats  host arrays of n device pointers (the caller keeps them;
 *                   read during the call only)
 *   flat_elems      capacity of every flats[a], in elements
 * Errors: those of tile_pack, plus SP_EINVAL (n outside [1, 16], null arrays)
 * and SP_EOVERLAP (a flat overlaps any raster or another flat).
 */
int tile_pack_n(int32_t dtype, int32_t n, const void* const* rasters, int64_t Hh, int64_t Ww, int64_t C, int32_t pr,
                int32_t pc, void* const* flats, int64_t flat_elems, void* stream);

/*
 * qk_norm_rope -- per-head RMSNorm of q or k fused with the rotary embedding.
 * Page "NPU HunyuanImage-3.0模型推理优化实践", section 计算分解: after the merged
 * QKV projection the query and key heads are normalised and then rotated
 * before attention; section RmsNorm算子优化: RMSNorm is LayerNorm without the
 * mean subtraction.  For each token t and head h, over the d features of the
 * head row:
 *   n = x * gamma / sqrt(sum(x^2) / d + eps),   y = rope(n)
 * where rope is rope_apply at positions pos0 + t when pos is NULL, else
 * rope_apply_mx with pos and sections.  Norm and rotation are float32 (the
 * angles float64, as in rope_apply); y is rounded once to dtype
 * (nearest-even).  With eps = 0 an all-zero row gives NaN, as the formula.
 *   x, y      device [s, H, d] of dtype; y == x allowed, other overlap not
 *   gamma     device float32 [d]: the learned weight, shared by all heads
 *   eps       added to the mean square; finite, >= 0 (applied in float32)
 *   pos0      first token's position when pos is NULL (ignored otherwise)
 *   pos       NULL, or device int64 [s, 3] as in rope_apply_mx
 *   sections  host array of 3 pair counts (only read when pos is not NULL)
 * Errors: as rope_apply / rope_apply_mx, plus SP_EINVAL (eps negative or not
 * finite, null gamma with data), SP_EUNSUPPORTED (a head row must split into
 * at most 64 lanes of g = 1, 2, 4 or 8 pairs with x and y aligned to g
 * elements, 2g for SP_ROPE_INTERLEAVED with g > 1: every even d up to 128
 * qualifies for any buffers, and every d up to 1024 with d/2 a multiple of 8
 * for 32-byte aligned ones, such as torch's allocations), SP_EOVERLAP (gamma
 * or pos overlaps y).
 */
int qk_norm_rope(int32_t dtype, const void* x, void* y, int64_t s, int32_t H, int32_t d, const float* gamma,
                 double eps, int64_t pos0, const int64_t* pos, const int32_t* sections, double theta, int32_t style,
                 void* stream);

/*
 * sp_av_positions -- axis positions of tokens [a, b) of a packed video+audio
 * sequence (host).  The packed sequence of section 机制一 holds the video
 * tokens of a T x Hh x Ww latent grid (frame-major, then row-major) followed
 * by n_audio audio tokens.  Video token i gets (i / (Hh*Ww), (i / Ww) % Hh,
 * i % Ww); audio token i gets (i - T*Hh*Ww, 0, 0), a 1-D position meant for
 * rope_apply_mx with sections {d/2, 0, 0}.
 *   out   host array of 3*(b-a) int64 values, written by the call
 * Errors: SP_EINVAL (negative sizes, a range outside [0, T*Hh*Ww + n_audio),
 * null out with b > a), SP_ERANGE (grid size overflows int64).  Host-only.
 */
int sp_av_positions(int64_t T, int64_t Hh, int64_t Ww, int64_t n_audio, int64_t a, int64_t b, int64_t* out);

/*
 * shard_attn_fwd -- attention of the rank's local queries against the full
 * gathered sequence.  Section 机制一: Q comes from the local shard while K/V
 * must cover the whole sequence.  Unmasked (bidirectional) softmax attention:
 *   O[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k[j,h,:]>) v[j,h,:]
 * for 0 <= i < sq, 0 <= j < skv.  The scale is computed once by the caller
 * (1/sqrt(d) in page "NPU HunyuanImage-3.0模型推理优化实践", section
 * 消除FA中scale的冗余计算) and passed in.
 *   q    device [sq, H, d];  k, v  device [skv, H, d];  o  device [sq, H, d]
 *   lse  NULL or device float32 [H, sq]: natural-log log-sum-exp of the
 *        scaled logits of each (head, query) row.
 * SP_BF16: bf16 operands, float32 accumulation and float32 online softmax,
 * probabilities rounded to bf16 for the P*V product, O rounded to bf16.
 * SP_F32: float32 throughout.  Each output row depends only on its own query
 * row and on K/V, in a fixed key order, so results are deterministic and a
 * row's result does not depend on sq or on where the row sits in q.
 * Head sizes 64 and 128; SP_BF16 also 512 (the single-head attention over
 * all channels of a VAE feature map, page "NPU HunyuanImage-3.0模型推理优化
 * 实践", section VAE并行优化, where K and V of all spatial blocks are
 * gathered).
 * Alignment: SP_BF16 moves Q, K and V in 16-byte vectors and O in 8-byte
 * ones, so q, k, v and o must be 16-byte aligned (SP_F32: 4-byte, the
 * element size); lse must be 4-byte aligned.  A token-row slice of a
 * torch allocation qualifies, since a bf16 row of H*d elements spans a
 * multiple of 128 bytes for d = 64, 128 and 512.
 * Errors: SP_EINVAL (bad dtype, sq < 0, skv < 1, H < 1, scale not finite or
 * <= 0, null pointers with data, a misaligned pointer), SP_EUNSUPPORTED
 * (other head sizes), SP_ERANGE (sq or skv of 2^31 - 256 or more, a grid
 * beyond 2^32 - 1 work-items, or 64 tokens of K spanning 2 GiB or more),
 * SP_EOVERLAP (o or lse overlaps an input or each other), SP_EHIP.
 * sq == 0 enqueues nothing.
 */
int shard_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                   void* o, float* lse, int64_t sq, int64_t skv, int32_t H, int32_t d,
                   float scale, void* stream);

/*
 * shard_attn_fwd_split -- shard_attn_fwd with the keys cut into nsplit ranges
 * that run as separate work-groups, for calls with too few query tiles to
 * fill the GPU (the single-head attention of the VAE block split, page "NPU
 * HunyuanImage-3.0模型推理优化实践", section VAE并行优化, has one head and a
 * few thousand queries per process).  Range s covers whole key tiles
 * [T*s/nsplit, T*(s+1)/nsplit) of the T tiles (32 keys each at head sizes
 * 128 and 512, 64 at head size 64); each range yields its own
 * normalised float32 output O_s and log-sum-exp L_s, and the results are
 * combined exactly as the softmax over the union of the ranges:
 *   O = sum_s exp(L_s - M) O_s / sum_s exp(L_s - M),  LSE = M + log sum_s exp(L_s - M)
 * with M = max_s L_s, in float32, O rounded once to bf16.  With nsplit = 1
 * the result is bit-identical to shard_attn_fwd.
 *   q, k, v, o, lse, sq, skv, H, d, scale, stream  as in shard_attn_fwd
 *                (SP_BF16 only; d 64, 128 or 512)
 *   nsplit      1 .. min(1024, ceil(skv / 64))
 *   workspace   device scratch of at least sp_attn_split_workspace(sq, H, d,
 *               nsplit) bytes, 256-byte aligned, caller-owned; its contents
 *               on entry do not matter and are overwritten
 * Errors: as shard_attn_fwd, plus SP_EUNSUPPORTED (SP_F32), SP_EINVAL (nsplit
 * out of range, null or misaligned workspace), SP_ERANGE (workspace too
 * small; the attention grid over all ranges or the merge grid, one thread per
 * four output columns, beyond 2^32 - 1 work-items: both are checked before
 * either launch), SP_EOVERLAP (workspace overlaps another buffer).
 */
int shard_attn_fwd_split(int32_t dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t sq, int64_t skv, int32_t H, int32_t d, float scale, int32_t nsplit,
                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sp_attn_split_workspace -- bytes of workspace shard_attn_fwd_split needs:
 * nsplit*rows*H*d float32 partial outputs (rounded up to 256 bytes) followed
 * by nsplit*H*sq float32 partial log-sum-exps, where rows = sq, or at d = 512
 * sq rounded up to a multiple of 128 (that kernel writes whole 128-query
 * blocks).  Negative status on bad arguments (SP_EINVAL) or overflow
 * (SP_ERANGE).  Host-only.
 */
int64_t sp_attn_split_workspace(int64_t sq, int32_t H, int32_t d, int32_t nsplit);

/*
 * shard_attn_fwd_split_noalloc -- shard_attn_fwd_split without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The float32 partials live in a 64 MiB device array
 * inside the library (one per device, held until the process ends), so
 * sp_attn_split_workspace(sq, H, d, nsplit) must not exceed 67,108,864 bytes
 * (the 128 x 128 VAE block of 4,096 queries at d = 512 with 4 key ranges needs
 * 32 MiB).  The array's previous contents are never read.  Every call on one
 * device shares that device's array: calls that overlap in time on one device
 * (other streams, other threads) race and must be serialised by the caller.
 * The device address is looked up on the first call on each device (with it
 * current); no allocating routine is called.
 *   arguments as shard_attn_fwd_split, without workspace / workspace_bytes
 * Errors: as shard_attn_fwd_split, plus SP_ERANGE (partials beyond 64 MiB),
 * SP_EHIP (the scratch address could not be obtained).
 */
int shard_attn_fwd_split_noalloc(int32_t dtype, const void* q, const void* k, const void* v, void* o,
                                 float* lse, int64_t sq, int64_t skv, int32_t H, int32_t d, float scale,
                                 int32_t nsplit, void* stream);

/*
 * shard_attn_fwd_gv -- shard_attn_fwd against K/V left in the W per-rank
 * shards, without the gather into one buffer.  Section 后端 A reassembles
 * the full sequence by concatenating the ranks' blocks in rank order; here
 * the kernel reads each K/V tile straight from the shard that holds it, so
 * the sequence is the same concatenation and the result is bit-identical to
 * shard_attn_fwd on the gathered buffers (same keys, same order, same
 * arithmetic).
 *   q          device [sq, H, d]
 *   W          number of shards, 1 <= W <= 16
 *   k_shards, v_shards  host arrays of W device pointers; shard r is a
 *              contiguous [seq_lens[r], H, d] tensor (may be NULL when
 *              seq_lens[r] == 0)
 *   seq_lens   host array of W token counts (>= 0, sum >= 1)
 *   o, lse, sq, H, d, scale, stream  as in shard_attn_fwd
 * Errors: as shard_attn_fwd, plus SP_EINVAL (W < 1, null host arrays, a
 * negative length, a null shard with tokens, a shard with tokens not aligned
 * as k and v must be), SP_EUNSUPPORTED (W > 16, or
 * d = 512: head sizes 64 and 128 only),
 * SP_ERANGE (lengths overflow), SP_EOVERLAP (o or lse overlaps q, a shard or
 * each other).  sq == 0 enqueues nothing.
 */
int shard_attn_fwd_gv(int32_t dtype, const void* q, int32_t W, const void* const* k_shards,
                      const void* const* v_shards, const int64_t* seq_lens, void* o, float* lse,
                      int64_t sq, int32_t H, int32_t d, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPATTN_H */

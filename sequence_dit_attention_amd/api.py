"""Torch-facing wrappers of the libspattn C ABI (argument marshalling only).

Each function has the name of the C entry point it calls.  Device tensors
must be contiguous HIP tensors of the right dtype; work is enqueued on
torch's current stream and nothing is synchronised.  Every computation runs
in the HIP library: there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import check, lib

SP_F32, SP_BF16 = 0, 1
SP_ROPE_HALF, SP_ROPE_INTERLEAVED = 0, 1
_STYLES = {"half": SP_ROPE_HALF, "interleaved": SP_ROPE_INTERLEAVED}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SP_F32
    if t.dtype == torch.bfloat16:
        return SP_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _i64s(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(x) for x in vals])
    return arr


def sp_abi_version() -> int:
    return int(lib().sp_abi_version())


def sp_shard_bounds(S: int, W: int, r: int) -> tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    check("sp_shard_bounds", lib().sp_shard_bounds(S, W, r, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def sp_allgatherv_layout(S: int, W: int, outer: int = 1, inner: int = 1):
    counts, displs = (ctypes.c_int64 * max(W, 1))(), (ctypes.c_int64 * max(W, 1))()
    check("sp_allgatherv_layout", lib().sp_allgatherv_layout(S, W, outer, inner, counts, displs))
    return list(counts)[:W], list(displs)[:W]


def sp_allgatherv_layout_lens(seq_lens, outer: int = 1, inner: int = 1):
    """AllGatherV (counts, displs) of tensors [outer, seq_lens[r], inner], blocks in rank order."""
    W = len(seq_lens)
    counts, displs = (ctypes.c_int64 * max(W, 1))(), (ctypes.c_int64 * max(W, 1))()
    check("sp_allgatherv_layout_lens",
          lib().sp_allgatherv_layout_lens(W, _i64s(seq_lens) if W else None, outer, inner, counts, displs))
    return list(counts)[:W], list(displs)[:W]


def varlen_pack(sends, counts, displs, flat: torch.Tensor) -> torch.Tensor:
    """flat[displs[r] : displs[r] + counts[r]] = sends[r] (flattened), in place on `flat`."""
    code = _dtype_code(flat)
    W = len(sends)
    ptrs = (ctypes.c_void_p * W)()
    for r, s in enumerate(sends):
        if s.dtype != flat.dtype:
            raise TypeError("send and flat dtypes differ")
        if int(counts[r]) > s.numel():
            raise ValueError(f"send[{r}] holds fewer than counts[{r}] elements")
        ptrs[r] = _dev(s, f"send[{r}]") if s.numel() else None
    check("varlen_pack", lib().varlen_pack(code, W, ptrs, _i64s(counts), _i64s(displs),
                                           _dev(flat, "flat"), flat.numel(), _stream(flat)))
    return flat


def varlen_unpack(flat: torch.Tensor, displs, seq_lens, outer: int, inner: int,
                  out: torch.Tensor) -> torch.Tensor:
    """out[o, a_r + t, k] = flat[displs[r] + (o*seq_lens[r] + t)*inner + k], in place on `out`."""
    code = _dtype_code(flat)
    if out.dtype != flat.dtype:
        raise TypeError("flat and out dtypes differ")
    need = int(outer) * sum(int(s) for s in seq_lens) * int(inner)
    if out.numel() != need:
        raise ValueError(f"out must hold outer*sum(seq_lens)*inner = {need} elements")
    W = len(seq_lens)
    check("varlen_unpack", lib().varlen_unpack(code, W, _dev(flat, "flat"), flat.numel(), _i64s(displs),
                                               _i64s(seq_lens), outer, inner, _dev(out, "out"),
                                               _stream(flat)))
    return out


def rope_apply(x: torch.Tensor, pos0: int, theta: float = 10000.0, style: str = "half",
               out: torch.Tensor | None = None) -> torch.Tensor:
    """RoPE of x [s, H, d] at positions pos0 + t; in place when out is None or out is x."""
    if x.dim() != 3:
        raise ValueError("x must be [s, H, d]")
    y = x if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    s, H, d = x.shape
    check("rope_apply", lib().rope_apply(_dtype_code(x), _dev(x, "x"), _dev(y, "out"), s, H, d, int(pos0),
                                         float(theta), _STYLES[style], _stream(x)))
    return y


def rope_apply_mx(x: torch.Tensor, pos: torch.Tensor, sections, theta: float = 10000.0, style: str = "half",
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Multi-axis RoPE of x [s, H, d] with positions pos (device int64 [s, 3]) and pairs per axis
    `sections` (3 ints summing to d/2); in place when out is None or out is x."""
    if x.dim() != 3:
        raise ValueError("x must be [s, H, d]")
    y = x if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    s, H, d = x.shape
    if pos.dtype != torch.int64 or tuple(pos.shape) != (s, 3):
        raise ValueError("pos must be int64 [s, 3]")
    sec = (ctypes.c_int32 * 3)(*[int(v) for v in sections])
    check("rope_apply_mx", lib().rope_apply_mx(_dtype_code(x), _dev(x, "x"), _dev(y, "out"), s, H, d,
                                               _dev(pos, "pos"), sec, float(theta), _STYLES[style], _stream(x)))
    return y


def qk_norm_rope(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, pos0: int = 0,
                 pos: torch.Tensor | None = None, sections=None, theta: float = 10000.0, style: str = "half",
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-head RMSNorm (weight gamma, float32 [d]) then RoPE of x [s, H, d]: 1-D positions pos0 + t when
    pos is None, else multi-axis with pos (device int64 [s, 3]) and sections; in place when out is None."""
    if x.dim() != 3:
        raise ValueError("x must be [s, H, d]")
    y = x if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    s, H, d = x.shape
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (d,):
        raise ValueError("gamma must be float32 [d]")
    pp, sec = None, None
    if pos is not None:
        if pos.dtype != torch.int64 or tuple(pos.shape) != (s, 3):
            raise ValueError("pos must be int64 [s, 3]")
        if sections is None:
            raise ValueError("sections are needed with pos")
        pp = _dev(pos, "pos")
        sec = (ctypes.c_int32 * 3)(*[int(v) for v in sections])
    check("qk_norm_rope", lib().qk_norm_rope(_dtype_code(x), _dev(x, "x"), _dev(y, "out"), s, H, d,
                                             _dev(gamma, "gamma"), float(eps), int(pos0), pp, sec, float(theta),
                                             _STYLES[style], _stream(x)))
    return y


def sp_tile_bounds(Hh: int, Ww: int, pr: int, pc: int, p: int) -> tuple[int, int, int, int]:
    """Block (r0, r1, c0, c1) of process p when an Hh x Ww grid is cut into pr x pc blocks."""
    out = (ctypes.c_int64 * 4)()
    check("sp_tile_bounds", lib().sp_tile_bounds(Hh, Ww, pr, pc, p, out))
    return out[0], out[1], out[2], out[3]


def tile_pack(raster: torch.Tensor, pr: int, pc: int, flat: torch.Tensor | None = None) -> torch.Tensor:
    """Blocks of raster [Hh, Ww, C] in process order, each row-major: flat [Hh*Ww, C] (or a given buffer)."""
    if raster.dim() != 3:
        raise ValueError("raster must be [Hh, Ww, C]")
    Hh, Ww, C = raster.shape
    if flat is None:
        flat = torch.empty(Hh * Ww, C, dtype=raster.dtype, device=raster.device)
    if flat.dtype != raster.dtype:
        raise ValueError("flat must match raster's dtype")
    check("tile_pack", lib().tile_pack(_dtype_code(raster), _dev(raster, "raster"), Hh, Ww, C, pr, pc,
                                       _dev(flat, "flat"), flat.numel(), _stream(raster)))
    return flat


def tile_pack_n(rasters, pr: int, pc: int, flats=None) -> list:
    """tile_pack of several rasters [Hh, Ww, C] of one shape and dtype in one batch of copies."""
    rasters = list(rasters)
    if not rasters or any(r.dim() != 3 for r in rasters):
        raise ValueError("rasters must be a non-empty list of [Hh, Ww, C]")
    Hh, Ww, C = rasters[0].shape
    if any(r.shape != rasters[0].shape or r.dtype != rasters[0].dtype for r in rasters):
        raise ValueError("rasters must share shape and dtype")
    if flats is None:
        flats = [torch.empty(Hh * Ww, C, dtype=r.dtype, device=r.device) for r in rasters]
    flats = list(flats)
    if len(flats) != len(rasters) or any(f.dtype != rasters[0].dtype for f in flats):
        raise ValueError("one flat per raster, of the rasters' dtype")
    n = len(rasters)
    cap = min(f.numel() for f in flats)
    rp = (ctypes.c_void_p * n)(*[_dev(r, "raster") for r in rasters])
    fp = (ctypes.c_void_p * n)(*[_dev(f, "flat") for f in flats])
    check("tile_pack_n", lib().tile_pack_n(_dtype_code(rasters[0]), n, rp, Hh, Ww, C, pr, pc, fp, cap,
                                           _stream(rasters[0])))
    return flats


def tile_unpack(flat: torch.Tensor, Hh: int, Ww: int, pr: int, pc: int,
                raster: torch.Tensor | None = None) -> torch.Tensor:
    """Put the blocks of flat (process order, each row-major, C channels) back into raster [Hh, Ww, C]."""
    C = flat.shape[-1]
    if raster is None:
        raster = torch.empty(Hh, Ww, C, dtype=flat.dtype, device=flat.device)
    if raster.dtype != flat.dtype or tuple(raster.shape) != (Hh, Ww, C):
        raise ValueError("raster must be [Hh, Ww, C] of flat's dtype")
    check("tile_unpack", lib().tile_unpack(_dtype_code(flat), _dev(flat, "flat"), flat.numel(), Hh, Ww, C, pr, pc,
                                           _dev(raster, "raster"), _stream(flat)))
    return raster


def sp_av_positions(T: int, Hh: int, Ww: int, n_audio: int, a: int, b: int) -> torch.Tensor:
    """Axis positions (host int64 tensor [b - a, 3]) of tokens [a, b) of a packed video + audio sequence."""
    outn = max(b - a, 0)
    arr = (ctypes.c_int64 * (3 * outn if outn else 1))()
    check("sp_av_positions", lib().sp_av_positions(T, Hh, Ww, n_audio, a, b, arr))
    return torch.tensor(list(arr)[: 3 * outn], dtype=torch.int64).reshape(outn, 3)


def shard_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, scale: float | None = None) -> torch.Tensor:
    """Attention of q [sq, H, d] against k, v [skv, H, d]; returns O [sq, H, d] (lse [H, sq] if given)."""
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q [sq,H,d], k and v [skv,H,d] with matching H, d")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v dtypes differ")
    sq, H, d = q.shape
    skv = k.shape[0]
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or lse.shape != (H, sq):
            raise ValueError("lse must be float32 [H, sq]")
        lp = _dev(lse, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    check("shard_attn_fwd", lib().shard_attn_fwd(_dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                                 _dev(out, "out"), lp, sq, skv, H, d, float(scale),
                                                 _stream(q)))
    return out


def split_workspace_bytes(sq: int, H: int, d: int, nsplit: int) -> int:
    """Bytes of device workspace shard_attn_fwd_split needs."""
    n = lib().sp_attn_split_workspace(sq, H, d, nsplit)
    if n < 0:
        check("sp_attn_split_workspace", int(n))
    return int(n)


def shard_attn_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, nsplit: int,
                         out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                         scale: float | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """shard_attn_fwd with the keys cut into nsplit ranges (bf16); workspace: a device uint8 buffer of at
    least split_workspace_bytes(...) bytes (allocated here with torch when None)."""
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q [sq,H,d], k and v [skv,H,d] with matching H, d")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v dtypes differ")
    sq, H, d = q.shape
    skv = k.shape[0]
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or lse.shape != (H, sq):
            raise ValueError("lse must be float32 [H, sq]")
        lp = _dev(lse, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = split_workspace_bytes(sq, H, d, nsplit)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    check("shard_attn_fwd_split", lib().shard_attn_fwd_split(
        _dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), lp, sq, skv, H, d,
        float(scale), int(nsplit), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(q)))
    return out


def shard_attn_fwd_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, nsplit: int,
                                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                                 scale: float | None = None) -> torch.Tensor:
    """shard_attn_fwd_split with its float32 partials in the library's device scratch (no workspace, no
    allocation inside the call; calls that overlap on one device race)."""
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q [sq,H,d], k and v [skv,H,d] with matching H, d")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v dtypes differ")
    sq, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or lse.shape != (H, sq):
            raise ValueError("lse must be float32 [H, sq]")
        lp = _dev(lse, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    check("shard_attn_fwd_split_noalloc", lib().shard_attn_fwd_split_noalloc(
        _dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), lp, sq, k.shape[0], H, d,
        float(scale), int(nsplit), _stream(q)))
    return out


def exchange_sim(shards, cat_dim: int = 0):
    """Single-GPU stand-in for exchange(rank, tensors, cat_dims): AllGatherV of
    per-rank shards (tensors of one dtype and device that agree in every size
    except along cat_dim) through a flat buffer, then narrow/view/concat.
    Counts and displacements come from sp_allgatherv_layout_lens.  Returns the
    concatenated tensor."""
    shards = list(shards)
    if not shards:
        raise ValueError("exchange_sim needs at least one shard")
    ref = shards[0]
    nd = ref.dim()
    if nd == 0:
        raise ValueError("shards must have at least one dimension")
    if not -nd <= cat_dim < nd:
        raise ValueError(f"cat_dim {cat_dim} out of range for {nd}-d shards")
    cat_dim %= nd
    shape = list(ref.shape)
    for r, s in enumerate(shards):
        if s.dtype != ref.dtype or s.device != ref.device:
            raise TypeError(f"shard {r} differs from shard 0 in dtype or device")
        if s.dim() != nd or any(s.shape[i] != shape[i] for i in range(nd) if i != cat_dim):
            raise ValueError(f"shard {r} has shape {tuple(s.shape)}: shards may differ only along dim {cat_dim}")
        if not s.is_contiguous():
            raise ValueError(f"shard {r} must be contiguous")
    outer = math.prod(shape[:cat_dim])
    inner = math.prod(shape[cat_dim + 1:])
    lens = [int(s.shape[cat_dim]) for s in shards]
    counts, displs = sp_allgatherv_layout_lens(lens, outer, inner)
    flat = torch.empty(sum(counts), dtype=ref.dtype, device=ref.device)
    varlen_pack([s.view(-1) for s in shards], counts, displs, flat)
    shape[cat_dim] = sum(lens)
    out = torch.empty(shape, dtype=ref.dtype, device=ref.device)
    varlen_unpack(flat, displs, lens, outer, inner, out)
    return out


def shard_attn_fwd_gv(q: torch.Tensor, k_shards, v_shards, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, scale: float | None = None) -> torch.Tensor:
    """shard_attn_fwd of q [sq, H, d] against K/V given as per-rank shards [s_r, H, d] (sequence =
    their concatenation in rank order), read in place without a gather."""
    if q.dim() != 3:
        raise ValueError("q must be [sq, H, d]")
    W = len(k_shards)
    if len(v_shards) != W or W < 1:
        raise ValueError("k_shards and v_shards must be non-empty lists of equal length")
    sq, H, d = q.shape
    for kt, vt in zip(k_shards, v_shards):
        if kt.dim() != 3 or kt.shape != vt.shape or kt.shape[1:] != (H, d):
            raise ValueError("every shard must be [s_r, H, d] with q's H and d, K and V alike")
        if kt.dtype != q.dtype or vt.dtype != q.dtype:
            raise TypeError("shard dtype differs from q")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    lp = None
    if lse is not None:
        if lse.dtype != torch.float32 or lse.shape != (H, sq):
            raise ValueError("lse must be float32 [H, sq]")
        lp = _dev(lse, "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kp = (ctypes.c_void_p * W)(*[(_dev(t, "k shard") if t.numel() else None) for t in k_shards])
    vp = (ctypes.c_void_p * W)(*[(_dev(t, "v shard") if t.numel() else None) for t in v_shards])
    lens = (ctypes.c_int64 * W)(*[int(t.shape[0]) for t in k_shards])
    check("shard_attn_fwd_gv", lib().shard_attn_fwd_gv(_dtype_code(q), _dev(q, "q"), W, kp, vp, lens,
                                                       _dev(out, "out"), lp, sq, H, d, float(scale),
                                                       _stream(q)))
    return out

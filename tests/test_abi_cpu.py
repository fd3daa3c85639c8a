"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/spattn.h declares, the host-only entry points agree bit-exactly with
the oracle, and every argument error is reported before anything is enqueued.
(Entry points that compute on the device are only called here with arguments
that fail validation, so no HIP work is ever started.)"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sequence_dit_attention_amd import _lib
from sequence_dit_attention_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spattn.h")

SP_EINVAL, SP_EUNSUPPORTED, SP_ERANGE, SP_EOVERLAP = -1, -2, -3, -4


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "shard_attn_fwd" in names and "shard_attn_fwd_gv" in names and len(names) == 20
    h = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == names
    assert api.sp_abi_version() == 1


def test_shard_bounds_match_oracle():
    for S in list(range(0, 300)) + [16383, 25640, 125117, 367287, 2**62 + 5]:
        for W in (1, 2, 3, 4, 7, 8, 16):
            for r in range(W):
                assert api.sp_shard_bounds(S, W, r) == oracle.shard_bounds(S, W, r)


def test_layout_matches_oracle():
    for S, W, outer, inner in [(16383, 4, 1, 2048), (1001, 4, 1, 128), (7, 4, 3, 5), (3, 8, 2, 1)]:
        assert api.sp_allgatherv_layout(S, W, outer, inner) == oracle.allgatherv_layout(S, W, outer, inner)


def test_layout_lens_matches_oracle():
    for lens, outer, inner in [([4095, 4096, 4096, 4096], 1, 16 * 128), ([3, 0, 5, 1], 2, 4), ([0], 3, 2),
                               ([2, 7], 1, 1), ([1, 1, 1], 5, 0), ([6, 2, 9], 0, 3), ([250, 250, 250, 251], 1, 128)]:
        assert api.sp_allgatherv_layout_lens(lens, outer, inner) == oracle.allgatherv_layout_lens(lens, outer, inner)
    for S, W in [(16383, 4), (367287, 4), (7, 8)]:
        lens = [b - a for a, b in oracle.all_shard_bounds(S, W)]
        assert api.sp_allgatherv_layout_lens(lens, 1, 3072) == api.sp_allgatherv_layout(S, W, 1, 3072)


def test_layout_lens_errors_leave_outputs_untouched():
    L = _lib.lib()
    c, d = (ctypes.c_int64 * 3)(-7, -7, -7), (ctypes.c_int64 * 3)(-7, -7, -7)
    assert L.sp_allgatherv_layout_lens(3, _arr([1, 2, -1]), 1, 1, c, d) == SP_EINVAL
    assert L.sp_allgatherv_layout_lens(3, _arr([2**42, 2**42, 2**42]), 2**10, 2**10, c, d) == SP_ERANGE
    assert b"overflow" in L.sp_last_error()
    assert L.sp_allgatherv_layout_lens(0, _arr([1]), 1, 1, c, d) == SP_EINVAL
    assert L.sp_allgatherv_layout_lens(3, None, 1, 1, c, d) == SP_EINVAL
    assert L.sp_allgatherv_layout_lens(3, _arr([1, 2, 3]), -1, 1, c, d) == SP_EINVAL
    assert L.sp_allgatherv_layout_lens(3, _arr([1, 2, 3]), 1, 1, None, d) == SP_EINVAL
    assert list(c) == [-7, -7, -7] and list(d) == [-7, -7, -7]


def test_exchange_sim_validates_shards():
    import torch

    a = torch.zeros(2, 3, 4)
    with pytest.raises(ValueError, match="at least one"):
        api.exchange_sim([])
    with pytest.raises(ValueError, match="out of range"):
        api.exchange_sim([a], 3)
    with pytest.raises(ValueError, match="differ only along"):
        api.exchange_sim([a, torch.zeros(2, 3, 5)], 1)
    with pytest.raises(ValueError, match="differ only along"):
        api.exchange_sim([a, torch.zeros(2, 3)], 0)
    with pytest.raises(TypeError, match="dtype or device"):
        api.exchange_sim([a, torch.zeros(2, 3, 4, dtype=torch.float64)], -1)


def _code(fn, *args):
    return fn(*args)


def test_host_errors():
    L = _lib.lib()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert L.sp_shard_bounds(10, 0, 0, ctypes.byref(a), ctypes.byref(b)) == SP_EINVAL
    assert L.sp_shard_bounds(10, 4, 4, ctypes.byref(a), ctypes.byref(b)) == SP_EINVAL
    assert L.sp_shard_bounds(-1, 4, 0, ctypes.byref(a), ctypes.byref(b)) == SP_EINVAL
    assert L.sp_shard_bounds(10, 4, 0, None, ctypes.byref(b)) == SP_EINVAL
    assert b"rank" in L.sp_last_error() or b"null" in L.sp_last_error()
    c, d = (ctypes.c_int64 * 4)(), (ctypes.c_int64 * 4)()
    assert L.sp_allgatherv_layout(2**40, 4, 2**20, 2**10, c, d) == SP_ERANGE
    assert L.sp_allgatherv_layout(10, 4, -1, 1, c, d) == SP_EINVAL
    assert L.sp_shard_bounds(10, 4, 1, ctypes.byref(a), ctypes.byref(b)) == 0
    assert L.sp_last_error() == b""


def _arr(vals, t=ctypes.c_int64):
    return (t * len(vals))(*vals)


FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def test_pack_validation():
    L = _lib.lib()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE + 10_000)
    cnt, dsp = _arr([4, 4]), _arr([0, 4])
    assert L.varlen_pack(7, 2, ptrs, cnt, dsp, FAKE * 2, 8, None) == SP_EINVAL          # dtype
    assert L.varlen_pack(1, 0, ptrs, cnt, dsp, FAKE * 2, 8, None) == SP_EINVAL          # W
    assert L.varlen_pack(1, 2, ptrs, _arr([-1, 4]), dsp, FAKE * 2, 8, None) == SP_EINVAL
    assert L.varlen_pack(1, 2, ptrs, cnt, _arr([0, 5]), FAKE * 2, 8, None) == SP_ERANGE  # past end
    assert L.varlen_pack(1, 2, ptrs, cnt, _arr([0, 3]), FAKE * 2, 8, None) == SP_EOVERLAP
    assert L.varlen_pack(1, 2, (ctypes.c_void_p * 2)(FAKE, None), cnt, dsp, FAKE * 2, 8, None) == SP_EINVAL
    # source overlapping the destination
    assert L.varlen_pack(1, 2, (ctypes.c_void_p * 2)(FAKE, FAKE * 2 + 4), cnt, dsp, FAKE * 2, 8, None) == SP_EOVERLAP
    assert b"overlap" in L.sp_last_error()


def test_unpack_validation():
    L = _lib.lib()
    dsp, lens = _arr([0, 6]), _arr([2, 2])
    assert L.varlen_unpack(9, 2, FAKE, 12, dsp, lens, 1, 3, FAKE * 2, None) == SP_EINVAL
    assert L.varlen_unpack(1, 2, FAKE, 11, dsp, lens, 1, 3, FAKE * 2, None) == SP_ERANGE
    assert L.varlen_unpack(1, 2, FAKE, 12, _arr([0, 5]), lens, 1, 3, FAKE * 2, None) == SP_EOVERLAP
    assert L.varlen_unpack(1, 2, FAKE, 12, dsp, _arr([2, -2]), 1, 3, FAKE * 2, None) == SP_EINVAL
    assert L.varlen_unpack(1, 2, FAKE, 12, dsp, lens, 1, 3, FAKE + 4, None) == SP_EOVERLAP


def test_rope_validation():
    L = _lib.lib()
    assert L.rope_apply(1, FAKE, FAKE, 10, 2, 7, 0, 1e4, 0, None) == SP_EINVAL      # odd d
    assert L.rope_apply(1, FAKE, FAKE, 10, 2, 8, 0, -1.0, 0, None) == SP_EINVAL     # theta
    assert L.rope_apply(1, FAKE, FAKE, 10, 2, 8, 0, 1e4, 5, None) == SP_EINVAL      # style
    assert L.rope_apply(1, FAKE, FAKE, 10, 0, 8, 0, 1e4, 0, None) == SP_EINVAL      # H
    assert L.rope_apply(1, FAKE, FAKE, 10, 2, 8, 2**53, 1e4, 0, None) == SP_EINVAL  # positions
    assert L.rope_apply(1, FAKE, FAKE, 2**62, 2, 8, 2**53 - 1, 1e4, 0, None) == SP_EINVAL  # pos0 + s, no wrap
    assert L.rope_apply(1, FAKE, FAKE + 2, 10, 2, 8, 0, 1e4, 0, None) == SP_EOVERLAP


def test_rope_mx_validation():
    L = _lib.lib()
    sec = (ctypes.c_int32 * 3)(2, 1, 1)
    f = L.rope_apply_mx
    bad = (ctypes.c_int32 * 3)(2, 1, 2)
    assert f(1, FAKE, FAKE, 10, 2, 8, FAKE * 2, bad, 1e4, 0, None) == SP_EINVAL          # sections != d/2
    neg = (ctypes.c_int32 * 3)(5, -1, 0)
    assert f(1, FAKE, FAKE, 10, 2, 8, FAKE * 2, neg, 1e4, 0, None) == SP_EINVAL
    assert f(1, FAKE, FAKE, 10, 2, 8, FAKE * 2, None, 1e4, 0, None) == SP_EINVAL         # null sections
    assert f(1, FAKE, FAKE, 10, 2, 8, None, sec, 1e4, 0, None) == SP_EINVAL              # null positions
    assert f(1, FAKE, FAKE, 10, 2, 7, FAKE * 2, sec, 1e4, 0, None) == SP_EINVAL          # odd d
    assert f(1, FAKE, FAKE + 2, 10, 2, 8, FAKE * 2, sec, 1e4, 0, None) == SP_EOVERLAP    # partial x/y overlap
    assert f(1, FAKE, FAKE, 10, 2, 8, FAKE + 16, sec, 1e4, 0, None) == SP_EOVERLAP       # positions inside y
    assert f(1, FAKE, FAKE, 0, 2, 8, None, sec, 1e4, 0, None) == 0                        # s == 0: nothing to do


def test_qk_norm_rope_validation():
    L = _lib.lib()
    f = L.qk_norm_rope
    sec = (ctypes.c_int32 * 3)(2, 1, 1)
    bad = (ctypes.c_int32 * 3)(2, 1, 2)
    G = FAKE * 4  # a gamma address away from x and y
    assert f(1, FAKE, FAKE, 10, 2, 8, G, -1e-6, 0, None, None, 1e4, 0, None) == SP_EINVAL        # eps < 0
    assert f(1, FAKE, FAKE, 10, 2, 8, G, float("nan"), 0, None, None, 1e4, 0, None) == SP_EINVAL  # eps NaN
    assert f(1, FAKE, FAKE, 10, 2, 8, None, 1e-6, 0, None, None, 1e4, 0, None) == SP_EINVAL      # null gamma
    assert f(1, FAKE, FAKE, 10, 2, 130, G, 1e-6, 0, None, None, 1e4, 0, None) == SP_EUNSUPPORTED  # 65 pairs
    assert f(1, FAKE, FAKE, 10, 2, 7, G, 1e-6, 0, None, None, 1e4, 0, None) == SP_EINVAL         # odd d
    assert f(1, FAKE, FAKE, 10, 2, 8, G, 1e-6, 0, FAKE * 2, bad, 1e4, 0, None) == SP_EINVAL      # sections
    assert f(1, FAKE, FAKE, 10, 2, 8, G, 1e-6, 0, FAKE * 2, None, 1e4, 0, None) == SP_EINVAL     # null sections
    assert f(1, FAKE, FAKE, 10, 2, 8, G, 1e-6, 2**53, None, None, 1e4, 0, None) == SP_EINVAL     # 1-D positions
    assert f(1, FAKE, FAKE + 2, 10, 2, 8, G, 1e-6, 0, None, None, 1e4, 0, None) == SP_EOVERLAP   # x / y
    assert f(1, FAKE, FAKE, 10, 2, 8, FAKE + 8, 1e-6, 0, None, None, 1e4, 0, None) == SP_EOVERLAP  # gamma in y
    assert f(1, FAKE, FAKE, 10, 2, 8, G, 1e-6, 0, FAKE + 16, sec, 1e4, 0, None) == SP_EOVERLAP   # pos in y
    assert f(1, FAKE, FAKE, 10, 2, 8, G, 1e-6, 0, None, None, 1e4, 9, None) == SP_EINVAL         # style
    assert f(1, FAKE, FAKE, 0, 2, 8, None, 1e-6, 0, None, None, 1e4, 0, None) == 0               # s == 0


def test_tile_bounds_match_oracle_and_validation():
    for Hh, Ww, pr, pc in [(7, 5, 2, 3), (128, 128, 2, 2), (84, 48, 3, 3), (0, 9, 2, 2), (5, 3, 7, 1),
                           (2**40 + 3, 2**35 + 1, 5, 7)]:
        for p in range(pr * pc):
            assert api.sp_tile_bounds(Hh, Ww, pr, pc, p) == oracle.tile_bounds(Hh, Ww, pr, pc, p)
    L = _lib.lib()
    out = (ctypes.c_int64 * 4)()
    assert L.sp_tile_bounds(4, 4, 2, 2, 4, out) == SP_EINVAL
    assert L.sp_tile_bounds(4, 4, 0, 2, 0, out) == SP_EINVAL
    assert L.sp_tile_bounds(-1, 4, 2, 2, 0, out) == SP_EINVAL
    assert L.sp_tile_bounds(4, 4, 2, 2, 0, None) == SP_EINVAL
    f, g = L.tile_pack, L.tile_unpack
    assert f(1, FAKE, 4, 4, 8, 2, 2, FAKE * 2, 127, None) == SP_ERANGE      # flat too small
    assert f(1, FAKE, 4, 4, 8, 2, 2, FAKE + 64, 128, None) == SP_EOVERLAP    # raster overlaps flat
    assert f(7, FAKE, 4, 4, 8, 2, 2, FAKE * 2, 128, None) == SP_EINVAL      # dtype
    assert f(1, FAKE, 4, 4, 8, 0, 2, FAKE * 2, 128, None) == SP_EINVAL      # pr
    assert f(1, None, 4, 4, 8, 2, 2, FAKE * 2, 128, None) == SP_EINVAL      # null raster
    assert g(1, FAKE * 2, 128, 4, 4, 8, 2, 2, None, None) == SP_EINVAL      # null raster
    assert g(1, FAKE * 2, 100, 4, 4, 8, 2, 2, FAKE, None) == SP_ERANGE
    assert g(1, FAKE * 2, 0, 0, 4, 8, 2, 2, None, None) == 0                # nothing to do


def test_tile_pack_n_validation():
    """The multi-tensor block gather checks every pair (and the pairs against each
    other) before anything is enqueued; 4 x 4 x 8 bf16 rasters are 256 bytes."""
    L = _lib.lib()
    P = ctypes.c_void_p
    tab = lambda *a: (P * len(a))(*a)
    f = L.tile_pack_n
    R = tab(FAKE, FAKE * 3)
    assert f(1, 0, R, 4, 4, 8, 2, 2, tab(FAKE * 2), 128, None) == SP_EINVAL           # n = 0
    assert f(1, 17, R, 4, 4, 8, 2, 2, R, 128, None) == SP_EINVAL                       # n > 16
    assert f(1, 2, None, 4, 4, 8, 2, 2, tab(FAKE * 2, FAKE * 4), 128, None) == SP_EINVAL  # null table
    assert f(1, 2, R, 4, 4, 8, 2, 2, tab(FAKE * 2, None), 128, None) == SP_EINVAL      # null flat
    assert f(1, 2, R, 4, 4, 8, 2, 2, tab(FAKE * 2, FAKE * 4), 127, None) == SP_ERANGE  # flats too small
    assert f(1, 2, R, 4, 4, 8, 2, 2, tab(FAKE * 2, FAKE * 3 + 64), 128, None) == SP_EOVERLAP  # flat on a raster
    assert f(1, 2, R, 4, 4, 8, 2, 2, tab(FAKE * 3 + 256, FAKE), 128, None) == SP_EOVERLAP     # flat 1 on raster 0
    assert f(1, 2, R, 4, 4, 8, 2, 2, tab(FAKE * 2, FAKE * 2 + 128), 128, None) == SP_EOVERLAP  # flats overlap
    assert f(7, 2, R, 4, 4, 8, 2, 2, tab(FAKE * 2, FAKE * 4), 128, None) == SP_EINVAL  # dtype
    assert f(1, 2, R, 0, 4, 8, 2, 2, tab(FAKE * 2, FAKE * 4), 0, None) == 0            # nothing to do


def test_split_attention_validation():
    L = _lib.lib()
    ws = L.sp_attn_split_workspace
    assert ws(100, 2, 128, 3) == ((3 * 100 * 2 * 128 * 4 + 255) // 256) * 256 + 3 * 2 * 100 * 4
    # head size 512 writes whole 128-query blocks of partials: rows rounded up to 128
    assert ws(100, 2, 512, 3) == ((3 * 128 * 2 * 512 * 4 + 255) // 256) * 256 + 3 * 2 * 100 * 4
    assert ws(4096, 1, 512, 8) == 8 * 4096 * 512 * 4 + 8 * 4096 * 4
    assert ws(-1, 2, 128, 3) == SP_EINVAL and ws(10, 2, 128, 0) == SP_EINVAL
    assert ws(2**40, 2**20, 512, 1024) == SP_ERANGE
    f = L.shard_attn_fwd_split
    need = ws(64, 1, 512, 2)
    W = FAKE * 8  # a workspace address away from the others (256-byte aligned)
    args = (1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 64, 300, 1, 512, 0.04)
    assert f(*args, 0, W, need, None) == SP_EINVAL                  # nsplit < 1
    assert f(*args, 6, W, 10**9, None) == SP_EINVAL                 # more ranges than 64-key tiles
    assert f(*args, 2, W, need - 1, None) == SP_ERANGE              # workspace too small
    assert f(*args, 2, W + 16, need, None) == SP_EINVAL             # misaligned
    assert f(*args, 2, None, need, None) == SP_EINVAL               # null workspace
    assert f(*args, 2, FAKE * 4, need, None) == SP_EOVERLAP         # workspace on top of o
    assert f(0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 64, 300, 1, 128, 0.08, 2, W, need, None) == SP_EUNSUPPORTED
    assert f(1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 64, 300, 1, 256, 0.06, 2, W, need, None) == SP_EUNSUPPORTED


def test_split_noalloc_validation():
    """The allocation-free split call validates like the workspace form and refuses
    partials beyond its 64 MiB device scratch (all before touching a device)."""
    L = _lib.lib()
    f = L.shard_attn_fwd_split_noalloc
    args = (1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 64, 300, 1, 512, 0.04)
    assert f(*args, 0, None) == SP_EINVAL                           # nsplit < 1
    assert f(*args, 6, None) == SP_EINVAL                           # more ranges than 64-key tiles
    assert f(1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4 + 8, None, 64, 300, 1, 512, 0.04, 2, None) == SP_EINVAL
    assert f(1, FAKE, FAKE * 2, FAKE * 3, FAKE, None, 64, 300, 1, 512, 0.04, 2, None) == SP_EOVERLAP
    assert f(0, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 64, 300, 1, 128, 0.08, 2, None) == SP_EUNSUPPORTED
    # 4,096 queries x 512 channels x 8 ranges = 64 MiB of partials + LSEs: one byte too many
    assert L.sp_attn_split_workspace(4096, 1, 512, 8) > 64 << 20
    assert f(1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 4096, 16384, 1, 512, 0.04, 8, None) == SP_ERANGE
    assert b"scratch" in L.sp_last_error()
    assert f(1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 0, 300, 1, 512, 0.04, 2, None) == 0  # sq == 0


def test_av_positions_match_oracle():
    for T, Hh, Ww, A, a, b in [(3, 4, 5, 7, 0, 67), (3, 4, 5, 7, 13, 61), (91, 48, 84, 375, 91000, 91900),
                               (91, 48, 84, 375, 366900, 367287), (2, 1, 1, 0, 0, 2), (0, 3, 3, 4, 0, 4)]:
        got = api.sp_av_positions(T, Hh, Ww, A, a, b).numpy()
        assert np.array_equal(got, oracle.av_positions(T, Hh, Ww, A, a, b))
    L = _lib.lib()
    out = (ctypes.c_int64 * 3)()
    assert L.sp_av_positions(3, 4, 5, 7, 0, 68, out) == SP_EINVAL   # past the end
    assert L.sp_av_positions(-1, 4, 5, 7, 0, 1, out) == SP_EINVAL
    assert L.sp_av_positions(2**40, 2**20, 2**10, 0, 0, 1, out) == SP_ERANGE
    assert L.sp_av_positions(3, 4, 5, 7, 0, 1, None) == SP_EINVAL


def test_attn_validation():
    L = _lib.lib()
    f = L.shard_attn_fwd
    q, k, v, o = FAKE, FAKE * 2, FAKE * 3, FAKE * 4
    assert f(1, q, k, v, o, None, 10, 20, 2, 96, 0.1, None) == SP_EUNSUPPORTED
    assert f(3, q, k, v, o, None, 10, 20, 2, 128, 0.1, None) == SP_EINVAL
    assert f(1, q, k, v, o, None, 10, 0, 2, 128, 0.1, None) == SP_EINVAL
    assert f(1, q, k, v, o, None, 10, 20, 2, 128, 0.0, None) == SP_EINVAL
    assert f(1, q, k, v, o, None, 10, 20, 2, 128, float("nan"), None) == SP_EINVAL
    assert f(1, q, k, v, q + 64, None, 10, 20, 2, 128, 0.1, None) == SP_EOVERLAP
    assert f(1, q, k, v, o, o + 8, 10, 20, 2, 128, 0.1, None) == SP_EOVERLAP
    assert f(1, None, k, v, o, None, 10, 20, 2, 128, 0.1, None) == SP_EINVAL
    assert f(1, q, k, v, o, None, 0, 20, 2, 128, 0.1, None) == 0   # sq == 0: nothing enqueued
    assert f(1, q, k, v, o, None, 2**31, 20, 1, 128, 0.1, None) == SP_ERANGE  # sq beyond 32-bit row indices
    assert f(1, q, k, v, o, None, 10, 2**31, 1, 128, 0.1, None) == SP_ERANGE  # skv likewise


def test_attn_gv_validation():
    L = _lib.lib()
    f = L.shard_attn_fwd_gv
    q, o = FAKE, FAKE * 4
    P = ctypes.c_void_p

    def call(W, ks, vs, lens, qq=q, oo=o, lse=None, sq=10, H=2, d=128, scale=0.1, dtype=1):
        return f(dtype, qq, W, (P * len(ks))(*ks), (P * len(vs))(*vs), _arr(lens), oo, lse, sq, H, d, scale, None)

    ks, vs = [FAKE * 2, FAKE * 2 + 10_000], [FAKE * 3, FAKE * 3 + 10_000]
    assert call(0, ks, vs, [5, 6]) == SP_EINVAL                          # W
    assert call(17, ks * 9, vs * 9, [1] * 18) == SP_EUNSUPPORTED        # too many shards
    assert call(2, ks, vs, [5, -1]) == SP_EINVAL                         # negative length
    assert call(2, ks, vs, [0, 0]) == SP_EINVAL                          # empty sequence
    assert call(2, ks, vs, [5, 6], d=96) == SP_EUNSUPPORTED
    assert call(2, [FAKE * 2, None], vs, [5, 6]) == SP_EINVAL            # null shard with tokens
    assert call(2, ks, vs, [5, 6], oo=FAKE * 2 + 512) == SP_EOVERLAP     # o over a K shard
    assert call(2, ks, vs, [5, 6], lse=FAKE * 3 + 64) == SP_EOVERLAP     # lse over a V shard
    assert call(2, ks, vs, [5, 6], oo=q + 64) == SP_EOVERLAP             # o over q
    assert f(1, q, 2, None, (P * 2)(*vs), _arr([5, 6]), o, None, 10, 2, 128, 0.1, None) == SP_EINVAL
    assert call(2, ks, vs, [5, 6], sq=0) == 0                            # nothing enqueued
    assert call(2, [None, FAKE * 2], [None, FAKE * 3], [0, 6], sq=0) == 0


def test_python_wrapper_raises():
    with pytest.raises(_lib.SpattnError) as ei:
        api.sp_shard_bounds(5, 2, 2)
    assert ei.value.code == SP_EINVAL


def test_attn_pointer_alignment():
    """bf16 attention moves Q/K/V in 16-byte vectors and O in 8-byte ones: every
    tensor must be 16-byte aligned (float32: 4), lse 4-byte aligned."""
    L = _lib.lib()
    f = L.shard_attn_fwd
    q, k, v, o = FAKE, FAKE * 2, FAKE * 3, FAKE * 4
    for bad in [(q + 8, k, v, o), (q, k + 2, v, o), (q, k, v + 4, o), (q, k, v, o + 8)]:
        assert f(1, *bad, None, 10, 20, 2, 128, 0.1, None) == SP_EINVAL
        assert b"aligned" in L.sp_last_error()
    assert f(1, q, k, v, o, FAKE * 5 + 2, 10, 20, 2, 128, 0.1, None) == SP_EINVAL   # lse
    assert f(0, q + 2, k, v, o, None, 10, 20, 2, 64, 0.1, None) == SP_EINVAL        # f32: element alignment
    P = ctypes.c_void_p
    g = L.shard_attn_fwd_gv
    ks, vs = (P * 2)(FAKE * 2, FAKE * 2 + 10_008), (P * 2)(FAKE * 3, FAKE * 3 + 10_000)
    assert g(1, q, 2, ks, vs, _arr([5, 6]), o, None, 10, 2, 128, 0.1, None) == SP_EINVAL   # K shard 1
    ks = (P * 2)(FAKE * 2, FAKE * 2 + 10_000)
    assert g(1, q, 2, ks, vs, _arr([5, 6]), o + 8, None, 10, 2, 128, 0.1, None) == SP_EINVAL
    # an empty shard's pointer is never read: its alignment does not matter
    assert g(1, q, 2, (P * 2)(FAKE * 2 + 1, FAKE * 2), (P * 2)(FAKE * 3 + 1, FAKE * 3), _arr([0, 6]), o, None,
             0, 2, 128, 0.1, None) == 0
    s = L.shard_attn_fwd_split
    need = L.sp_attn_split_workspace(64, 1, 512, 2)
    assert s(1, q, k + 8, v, o, None, 64, 300, 1, 512, 0.04, 2, FAKE * 8, need, None) == SP_EINVAL


def test_launch_grids_checked_before_enqueue():
    """A launch grid holds at most 2^32-1 work-items: calls needing more are
    refused with SP_ERANGE by the host, before anything is enqueued."""
    L = _lib.lib()
    f = L.shard_attn_fwd
    q, k, v, o = FAKE, FAKE * 2, FAKE * 3, FAKE * 4
    # 2^23 query tiles x 8 heads x 256 threads = 2^34 work-items
    assert f(1, q, FAKE * 64, FAKE * 96, FAKE * 128, None, 2**31 - 512, 20, 8, 128, 0.1, None) == SP_ERANGE
    assert b"work-items" in L.sp_last_error()
    s = L.shard_attn_fwd_split
    # split: the plain grid fits (2^26 items) but 1,024 key ranges do not
    need = L.sp_attn_split_workspace(2**20, 64, 128, 1024)
    assert need > 0
    assert s(1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 2**20, 2**20, 64, 128, 0.08, 1024, FAKE * 64, need,
             None) == SP_ERANGE
    assert b"work-items" in L.sp_last_error()
    # split: the attention fits, its merge (one thread per 4 output columns) does not
    need = L.sp_attn_split_workspace(2**25, 16, 128, 1)
    assert s(1, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 2**25, 64, 16, 128, 0.08, 1, FAKE * 64, need,
             None) == SP_ERANGE
    assert b"work-items" in L.sp_last_error()
    # a single 128 GiB copy segment: 2^25 chunks of 4 KiB x 256 threads
    ptrs = (ctypes.c_void_p * 1)(FAKE)
    assert L.varlen_pack(1, 1, ptrs, _arr([2**36]), _arr([0]), FAKE * 4, 2**36, None) == SP_ERANGE
    assert b"work-items" in L.sp_last_error()
    # RoPE: one wave per token
    assert L.rope_apply(1, FAKE, FAKE, 2**27, 1, 8, 0, 1e4, 0, None) == SP_ERANGE

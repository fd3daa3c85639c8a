"""ctypes loader for libspattn.so.  Fails loudly if the library was not built."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspattn.so")

# (name, restype, argtypes) of every exported entry point; mirrors include/spattn.h.
_I64, _I32, _VP, _PI64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
SIGNATURES = [
    ("sp_abi_version", ctypes.c_int, []),
    ("sp_last_error", ctypes.c_char_p, []),
    ("sp_shard_bounds", ctypes.c_int, [_I64, _I32, _I32, _PI64, _PI64]),
    ("sp_allgatherv_layout", ctypes.c_int, [_I64, _I32, _I64, _I64, _PI64, _PI64]),
    ("sp_allgatherv_layout_lens", ctypes.c_int, [_I32, _PI64, _I64, _I64, _PI64, _PI64]),
    ("varlen_pack", ctypes.c_int, [_I32, _I32, ctypes.POINTER(_VP), _PI64, _PI64, _VP, _I64, _VP]),
    ("varlen_unpack", ctypes.c_int, [_I32, _I32, _VP, _I64, _PI64, _PI64, _I64, _I64, _VP, _VP]),
    ("rope_apply", ctypes.c_int, [_I32, _VP, _VP, _I64, _I32, _I32, _I64, ctypes.c_double, _I32, _VP]),
    ("rope_apply_mx", ctypes.c_int, [_I32, _VP, _VP, _I64, _I32, _I32, _VP, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.c_double, _I32, _VP]),
    ("qk_norm_rope", ctypes.c_int, [_I32, _VP, _VP, _I64, _I32, _I32, _VP, ctypes.c_double, _I64, _VP,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.c_double, _I32, _VP]),
    ("sp_tile_bounds", ctypes.c_int, [_I64, _I64, _I32, _I32, _I32, _PI64]),
    ("tile_pack", ctypes.c_int, [_I32, _VP, _I64, _I64, _I64, _I32, _I32, _VP, _I64, _VP]),
    ("tile_unpack", ctypes.c_int, [_I32, _VP, _I64, _I64, _I64, _I64, _I32, _I32, _VP, _VP]),
    ("tile_pack_n", ctypes.c_int, [_I32, _I32, ctypes.POINTER(_VP), _I64, _I64, _I64, _I32, _I32,
                                   ctypes.POINTER(_VP), _I64, _VP]),
    ("shard_attn_fwd_split", ctypes.c_int, [_I32, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I32, _I32, ctypes.c_float,
                                            _I32, _VP, _I64, _VP]),
    ("shard_attn_fwd_split_noalloc", ctypes.c_int, [_I32, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I32, _I32,
                                                    ctypes.c_float, _I32, _VP]),
    ("sp_attn_split_workspace", ctypes.c_int64, [_I64, _I32, _I32, _I32]),
    ("sp_av_positions", ctypes.c_int, [_I64, _I64, _I64, _I64, _I64, _I64, _PI64]),
    ("shard_attn_fwd", ctypes.c_int, [_I32, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I32, _I32,
                                      ctypes.c_float, _VP]),
    ("shard_attn_fwd_gv", ctypes.c_int, [_I32, _VP, _I32, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _PI64,
                                         _VP, _VP, _I64, _I32, _I32, ctypes.c_float, _VP]),
]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first with "
                "`python -c 'import __graft_entry__ as g; g.build()'` "
                "(or python sequence_dit_attention_amd/build.py)")
        h = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


class SpattnError(RuntimeError):
    """A negative status from libspattn; .code holds it."""

    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} failed ({code}): {msg}")
        self.code = code


def check(func: str, code: int) -> None:
    if code != 0:
        raise SpattnError(func, code, lib().sp_last_error().decode(errors="replace"))

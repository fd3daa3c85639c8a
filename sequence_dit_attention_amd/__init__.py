"""MI355X-native (gfx950) one-rank share of packed-token sequence-parallel DiT attention.

The computation lives in libspattn.so (C ABI declared in include/spattn.h);
this package only loads it and marshals torch tensors into its calls.
"""
from .api import (  # noqa: F401
    SP_BF16,
    SP_F32,
    exchange_sim,
    qk_norm_rope,
    rope_apply,
    rope_apply_mx,
    shard_attn_fwd,
    shard_attn_fwd_gv,
    shard_attn_fwd_split,
    shard_attn_fwd_split_noalloc,
    split_workspace_bytes,
    sp_abi_version,
    sp_allgatherv_layout,
    sp_allgatherv_layout_lens,
    sp_av_positions,
    sp_shard_bounds,
    sp_tile_bounds,
    tile_pack,
    tile_pack_n,
    tile_unpack,
    varlen_pack,
    varlen_unpack,
)
from ._lib import LIB_PATH, SpattnError, lib  # noqa: F401

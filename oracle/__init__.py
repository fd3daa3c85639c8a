"""CPU oracle for one rank's share of packed-token sequence-parallel DiT attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test-suite, the smoke check of the graft entry
point and the CPU-baseline leg of the benchmark use it.  It shares no code,
tables or helpers with the HIP library under sequence_dit_attention_amd/ and
imports nothing from it.

Every function is a plain, slow, obviously correct definition in float64
(integers as Python ints) of what the pages define; see spattn_oracle.py.
"""
from .spattn_oracle import (  # noqa: F401
    shard_bounds,
    all_shard_bounds,
    allgatherv_layout,
    allgatherv_layout_lens,
    varlen_pack,
    varlen_unpack,
    rope_inv_freq,
    rope_apply,
    rope_apply_mx,
    av_positions,
    tile_bounds,
    tile_pack,
    tile_unpack,
    rms_norm,
    qk_norm_rope,
    attention,
    attention_rows,
    output_concat,
)

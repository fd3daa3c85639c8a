"""GPU parity of shard_attn_fwd_gv: attention reading K/V straight from the per-rank shards.

The gathered sequence is the concatenation of the ranks' shards in rank order
(MiniMax-H3-Comfy-NPU, 后端 A: narrow -> view -> concat of the AllGatherV
blocks).  Reading each key tile from the shard that holds it visits the same
keys in the same order with the same arithmetic, so the result must be
bit-identical to shard_attn_fwd on the gathered buffers; one case is also
checked against the float64 oracle.  Shard layouts cover tiles inside one
shard, tiles across boundaries, empty shards, shards shorter than a tile and
the ragged end of the sequence.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_tensor
from tests._helpers import attn_errors, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _inputs(seed, sq, lens, H, d, dtype):
    S = sum(lens)
    q = to_dev(gen_tensor(seed, 0, sq, H, d, dtype), dtype)
    k = to_dev(gen_tensor(seed, 1, S, H, d, dtype), dtype)
    v = to_dev(gen_tensor(seed, 2, S, H, d, dtype), dtype)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    ks = [k[starts[r]:starts[r + 1]].clone() for r in range(len(lens))]
    vs = [v[starts[r]:starts[r + 1]].clone() for r in range(len(lens))]
    return q, k, v, ks, vs


LAYOUTS = [
    [1000],                              # one shard (the gathered case)
    [250, 250, 250, 251],                # 768P-like split: every boundary inside a tile
    [64, 128, 192, 64],                  # boundaries on tile edges
    [0, 300, 0, 5, 1, 0, 427],           # empty shards and shards shorter than a tile
    [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16],  # 16 shards, several per tile
    [40],                                # one ragged tile
    [3, 0, 29, 0],                       # whole sequence shorter than one 32-key block
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lens", LAYOUTS, ids=lambda l: "x".join(map(str, l))[:40])
def test_gv_bitwise_equals_gathered(dtype, lens):
    sq, H, d = 300, 3, 128
    q, k, v, ks, vs = _inputs(11, sq, lens, H, d, dtype)
    lse_g = torch.empty(H, sq, dtype=torch.float32, device="cuda")
    lse_s = torch.empty_like(lse_g)
    og = sp.shard_attn_fwd(q, k, v, lse=lse_g)
    os_ = sp.shard_attn_fwd_gv(q, ks, vs, lse=lse_s)
    torch.cuda.synchronize()
    assert torch.equal(og.view(torch.int16) if dtype == "bf16" else og, os_.view(torch.int16) if dtype == "bf16" else os_)
    assert torch.equal(lse_g, lse_s)


@pytest.mark.parametrize("d", [64, 128])
def test_gv_head_size_64_and_128(d):
    lens = [97, 0, 200, 63]
    q, k, v, ks, vs = _inputs(12, 129, lens, 2, d, "bf16")
    og = sp.shard_attn_fwd(q, k, v)
    os_ = sp.shard_attn_fwd_gv(q, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(og.view(torch.int16), os_.view(torch.int16))


def test_gv_against_oracle():
    lens = [333, 1, 0, 700, 66]
    sq, H, d = 257, 2, 128
    q, k, v, ks, vs = _inputs(13, sq, lens, H, d, "bf16")
    o = sp.shard_attn_fwd_gv(q, ks, vs)
    torch.cuda.synchronize()
    ref = np.stack([oracle.attention(to_f64(q)[:, h:h + 1], to_f64(k)[:, h:h + 1], to_f64(v)[:, h:h + 1])[0][:, 0]
                    for h in range(H)], axis=1)
    err, rel = attn_errors(to_f64(o), ref)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)


def test_gv_rank_shards_of_the_768p_sequence():
    """The four rank shards of the 768P/15 s packed sequence (S = 367,287, W = 4), 24 heads,
    against 300 query rows: bit-identical to the gathered call."""
    S, W, H, d = 367287, 4, 24, 128
    bounds = [sp.sp_shard_bounds(S, W, r) for r in range(W)]
    lens = [b - a for a, b in bounds]
    q, k, v, ks, vs = _inputs(14, 300, lens, H, d, "bf16")
    og = sp.shard_attn_fwd(q, k, v)
    os_ = sp.shard_attn_fwd_gv(q, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(og.view(torch.int16), os_.view(torch.int16))


def test_gv_wrapper_rejects_mismatched_shards():
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16, device="cuda")
    k = [torch.zeros(5, 2, 64, dtype=torch.bfloat16, device="cuda")]
    with pytest.raises(ValueError):
        sp.shard_attn_fwd_gv(q, k, [torch.zeros(6, 2, 64, dtype=torch.bfloat16, device="cuda")])
    with pytest.raises(ValueError):
        sp.shard_attn_fwd_gv(q, k, k[:0])

"""GPU parity of the bf16 attention when the softmax reference has to rise.

The kernels keep a per-row reference maximum and raise it only when a 32-key
block holds a logit more than 8 (base 2) above it; part of a block's
probabilities is made one step early, under the reference of the time, and is
made again when the block's check raises it.  These inputs force that to
happen at chosen keys: every query row leans on axis 0 (even rows) or axis 1
(odd rows), and "spike" keys on those axes grow by about 10 (base 2) from one
spike of an axis to the next.  The spikes sit at the first and last key of a
block, at tile edges, in the ragged last tile and on the very last key, so
the raise happens in the first step, in either step of a tile, in the masked
tail and in the last step; the two axes make neighbouring columns of a wave
raise at different blocks.  The final output is dominated by the last spike of
the row's axis; bars as for shard_attn_fwd (bf16: 2e-2 absolute and 1e-2 of
max |O|), checked against the float64 oracle, plus the LSE.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import f32_to_bf16_bits
from tests._helpers import attn_errors, to_dev, to_f64, to_host_bits

pytestmark = pytest.mark.gpu


def _inputs(sq, skv, H, d, seed):
    rng = np.random.default_rng(seed)
    q = 0.5 * rng.standard_normal((sq, H, d))
    k = 0.5 * rng.standard_normal((skv, H, d))
    v = rng.standard_normal((skv, H, d))
    q[0::2, :, 0] += 4.0
    q[1::2, :, 1] += 4.0
    # logit gain of one spike step on an axis: 4 * step / sqrt(d) * log2(e) ~ 10 (base 2)
    step = 10.0 * np.sqrt(d) / (4.0 * np.log2(np.e))
    spikes = sorted({p for p in (0, 31, 32, 33, 63, 64, 65, 127, 128, 160, skv - 40, skv - 2, skv - 1)
                     if 0 <= p < skv})
    for i, p in enumerate(spikes):
        k[p, :, i % 2] += 4.0 + step * (i // 2)
    bits = [f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v)]
    return bits


def _check(o, lse, qb, kb, vb):
    ro, rl = oracle.attention(to_f64(qb), to_f64(kb), to_f64(vb))
    err, rel = attn_errors(to_f64(o), ro)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    assert float(np.max(np.abs(ro))) > 0.5  # dominated by spikes, not averaged out
    if lse is not None:
        assert np.max(np.abs(lse.cpu().numpy() - rl)) <= 2e-2


@pytest.mark.parametrize("d", [64, 128, 512])
@pytest.mark.parametrize("skv", [192, 1000])
def test_reference_raises(d, skv):
    H = 1 if d == 512 else 2
    sq = 293
    qb, kb, vb = _inputs(sq, skv, H, d, seed=d + skv)
    q, k, v = (to_dev(a, "bf16") for a in (qb, kb, vb))
    lse = torch.empty(H, sq, dtype=torch.float32, device="cuda")
    o = sp.shard_attn_fwd(q, k, v, lse=lse)
    torch.cuda.synchronize()
    _check(o, lse, qb, kb, vb)
    if d != 512:  # the shard table walks the same keys: bit-identical
        cut = [0, 100, 500, skv] if skv > 500 else [0, 64, 65, skv]
        ks = [k[a:b].contiguous() for a, b in zip(cut, cut[1:])]
        vs = [v[a:b].contiguous() for a, b in zip(cut, cut[1:])]
        o2 = sp.shard_attn_fwd_gv(q, ks, vs)
        torch.cuda.synchronize()
        assert to_host_bits(o2).tobytes() == to_host_bits(o).tobytes()


@pytest.mark.parametrize("d", [128, 512])
def test_reference_raises_split(d):
    H = 1 if d == 512 else 2
    sq, skv = 160, 1000
    qb, kb, vb = _inputs(sq, skv, H, d, seed=7 + d)
    q, k, v = (to_dev(a, "bf16") for a in (qb, kb, vb))
    lse = torch.empty(H, sq, dtype=torch.float32, device="cuda")
    o = sp.shard_attn_fwd_split(q, k, v, nsplit=3, lse=lse)
    torch.cuda.synchronize()
    _check(o, lse, qb, kb, vb)


def _restart_inputs(sq, skv, d, seed, positions):
    """Spikes that climb by about 120 (base 2) from one spike of an axis to the next:
    more than the head-size-512 kernel absorbs without a larger reference."""
    rng = np.random.default_rng(seed)
    q = 0.5 * rng.standard_normal((sq, 1, d))
    k = 0.5 * rng.standard_normal((skv, 1, d))
    v = rng.standard_normal((skv, 1, d))
    q[0::2, :, 0] += 4.0
    q[1::2, :, 1] += 4.0
    step = 120.0 * np.sqrt(d) / (4.0 * np.log2(np.e))
    for i, p in enumerate(positions):
        k[p, :, i % 2] += 4.0 + step * (i // 2)
    return [f32_to_bf16_bits(a.astype(np.float32)) for a in (q, k, v)]


@pytest.mark.parametrize("nsplit", [1, 2, 3])
def test_d512_restarts_on_large_score_jumps(nsplit):
    """Head size 512 keeps its accumulators unscaled and restarts the key loop when a
    score tops its query's first-tile maximum by more than 104 (base 2).  Spikes
    climbing ~120 per step force several restarts per work-group: at a tile's first
    key, at a tile edge, deep in the keys, in the ragged last tile and on the last
    key (two axes, so neighbouring query blocks restart at different tiles); with
    key ranges, some ranges restart and others do not.  Checked against the float64
    oracle (output dominated by the last spike of the row's axis) and its LSE."""
    sq, skv, d = 293, 1000, 512
    pos = [0, 1, 40, 63, 100, 300, 700, 990, 999]
    qb, kb, vb = _restart_inputs(sq, skv, d, 11 + nsplit, pos)
    q, k, v = (to_dev(a, "bf16") for a in (qb, kb, vb))
    lse = torch.empty(1, sq, dtype=torch.float32, device="cuda")
    if nsplit == 1:
        o = sp.shard_attn_fwd(q, k, v, lse=lse)
    else:
        o = sp.shard_attn_fwd_split(q, k, v, nsplit=nsplit, lse=lse)
    torch.cuda.synchronize()
    assert np.isfinite(to_f64(o)).all()
    _check(o, lse, qb, kb, vb)


@pytest.mark.parametrize("skv,nsplit,pos", [(96, 1, [0, 1, 40, 70]), (128, 2, [0, 1, 40, 41, 64, 65, 100, 101]),
                                            (64, 1, [0, 1, 33, 34]), (33, 1, [0, 1, 32])],
                         ids=["3tiles", "2x2tiles", "2tiles", "ragged2"])
def test_d512_restart_in_the_last_step_of_short_ranges(skv, nsplit, pos):
    """Head size 512 on ranges of two or three 32-key tiles, with the spike that forces a
    restart in the range's last tile: the restart comes after the last step, whose
    scores of the tile past the range are discarded, and the K tile of that step's
    load is the last one again.  The first spike of each axis sits in the first tile
    (it sets the reference); the later ones climb ~120 each.  In the 2 x 2 case each
    range restarts in its own last step; the ragged case has one key in its last
    tile, the spike."""
    sq, d = 160, 512
    qb, kb, vb = _restart_inputs(sq, skv, d, 21 + skv, pos)
    q, k, v = (to_dev(a, "bf16") for a in (qb, kb, vb))
    lse = torch.empty(1, sq, dtype=torch.float32, device="cuda")
    if nsplit == 1:
        o = sp.shard_attn_fwd(q, k, v, lse=lse)
    else:
        o = sp.shard_attn_fwd_split(q, k, v, nsplit=nsplit, lse=lse)
    torch.cuda.synchronize()
    assert np.isfinite(to_f64(o)).all()
    _check(o, lse, qb, kb, vb)

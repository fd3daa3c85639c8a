"""GPU parity of rope_apply_mx (multi-axis RoPE with explicit positions) against the float64 oracle.

The frequency table that MiniMax-H3-Comfy-NPU (机制一) slices per rank is read
as the multi-axis form for packed video tokens (frame, row, column) with 1-D
positions for the audio tokens that follow; the reading is the oracle's
(parity unpinned by the pages).  Tolerances as for rope_apply: float32 within
2e-6 absolute, bf16 within one bf16 ulp of the exact result plus 1e-6.  With a
single axis the call must reproduce rope_apply bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_tensor
from tests._helpers import bf16_ulp, to_dev, to_f64, to_host_bits

pytestmark = pytest.mark.gpu


def _check(got, ref, dtype):
    if dtype == "f32":
        assert np.max(np.abs(got - ref)) <= 2e-6
    else:
        assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-6)


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("s,H,d,sections", [(301, 3, 128, (22, 21, 21)), (64, 2, 64, (8, 12, 12)),
                                             (17, 1, 16, (2, 3, 3)), (9, 2, 12, (6, 0, 0)),
                                             (33, 4, 128, (0, 32, 32)), (5, 1, 8, (1, 2, 1))])
def test_rope_mx_vs_oracle(style, dtype, s, H, d, sections):
    rng = np.random.default_rng(s + d)
    pos = rng.integers(0, 100000, size=(s, 3)).astype(np.int64)
    x = gen_tensor(seed=s + d + 1, tensor_id=0, S=s, H=H, d=d, dtype=dtype)
    xd = to_dev(x, dtype)
    y = torch.empty_like(xd)
    sp.rope_apply_mx(xd, torch.from_numpy(pos).cuda(), sections, 10000.0, style, out=y)
    torch.cuda.synchronize()
    _check(to_f64(y), oracle.rope_apply_mx(to_f64(x), pos, sections, 10000.0, style), dtype)
    assert to_host_bits(xd).tobytes() == x.tobytes()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_axis_equals_rope_apply_bitwise(dtype):
    s, H, d, pos0 = 4099, 6, 128, 91821
    x = to_dev(gen_tensor(seed=3, tensor_id=1, S=s, H=H, d=d, dtype=dtype), dtype)
    pos = torch.zeros(s, 3, dtype=torch.int64)
    pos[:, 0] = torch.arange(pos0, pos0 + s)
    a = sp.rope_apply(x, pos0, out=torch.empty_like(x))
    b = sp.rope_apply_mx(x, pos.cuda(), (d // 2, 0, 0), out=torch.empty_like(x))
    torch.cuda.synchronize()
    assert to_host_bits(a).tobytes() == to_host_bits(b).tobytes()


def test_packed_768p_positions_in_place():
    """Rank 0 of the 768P/15 s packed sequence (91 x 48 x 84 video grid + 375 audio tokens) and the
    last rank's slice, which ends in the audio tokens: video with 3 axes, audio with 1-D positions."""
    T, Hh, Ww, A = 91, 48, 84, 375
    S, W, H, d = T * Hh * Ww + A, 4, 2, 128
    V = T * Hh * Ww
    for r in (0, W - 1):
        a, b = sp.sp_shard_bounds(S, W, r)
        x = gen_tensor(seed=8, tensor_id=1, S=S, H=H, d=d, dtype="bf16", tok0=a, tok1=b)
        xd = to_dev(x, "bf16")
        pos = sp.sp_av_positions(T, Hh, Ww, A, a, b)
        v_end = min(b, V) - a  # video tokens of the slice come first
        if v_end > 0:
            sp.rope_apply_mx(xd[:v_end], pos[:v_end].cuda(), (22, 21, 21))
        if v_end < b - a:
            sp.rope_apply_mx(xd[v_end:], pos[v_end:].cuda(), (d // 2, 0, 0))
        torch.cuda.synchronize()
        got = to_f64(xd)
        ref = np.empty_like(got)
        if v_end > 0:
            ref[:v_end] = oracle.rope_apply_mx(to_f64(x[:v_end]), oracle.av_positions(T, Hh, Ww, A, a, a + v_end),
                                               (22, 21, 21))
        if v_end < b - a:
            ref[v_end:] = oracle.rope_apply_mx(to_f64(x[v_end:]), oracle.av_positions(T, Hh, Ww, A, a + v_end, b),
                                               (d // 2, 0, 0))
        _check(got, ref, "bf16")

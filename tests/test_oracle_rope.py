"""Pins of the oracle's rotary embedding (CPU only).

Rotary embedding on q and k (NPU HunyuanImage-3.0模型推理优化实践, section
消除旋转位置编码冗余cast算子) at absolute packed positions, the rank's slice of
the frequency table starting at its first token (MiniMax-H3-Comfy-NPU, 机制一).
Pinned by complex multiplication (an independent formulation of a rotation),
textbook cos/sin values, and the rotation group properties.
"""
import cmath
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_d2():
    with open(os.path.join(GOLD, "rope_closed_form.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float64).reshape(1, 1, 2)
        y = oracle.rope_apply(x, pos0=c["p"], theta=10000.0, style="half")
        assert np.allclose(y.ravel(), c["y"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_complex_multiplication(style):
    rng = np.random.default_rng(3)
    s, H, d, theta = 5, 2, 8, 10000.0
    x = rng.standard_normal((s, H, d))
    for pos0 in (0, 17, 367282):
        y = oracle.rope_apply(x, pos0, theta, style)
        for t in range(s):
            p = pos0 + t
            for h in range(H):
                for j in range(d // 2):
                    i1, i2 = (j, j + d // 2) if style == "half" else (2 * j, 2 * j + 1)
                    z = complex(x[t, h, i1], x[t, h, i2]) * cmath.exp(1j * p * theta ** (-2.0 * j / d))
                    assert abs(y[t, h, i1] - z.real) < 1e-9 and abs(y[t, h, i2] - z.imag) < 1e-9


def test_position_zero_identity_and_v_untouched_pairs():
    x = np.random.default_rng(4).standard_normal((1, 3, 16))
    assert np.array_equal(oracle.rope_apply(x, 0), x)
    assert np.array_equal(oracle.rope_apply(x, 0, style="interleaved"), x)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_norm_relative_inverse_and_shard(style):
    rng = np.random.default_rng(5)
    S, H, d = 64, 2, 16
    x = rng.standard_normal((S, H, d))
    y = oracle.rope_apply(x, 1000, style=style)
    # pair norms preserved
    if style == "half":
        n0 = x[..., :8] ** 2 + x[..., 8:] ** 2
        n1 = y[..., :8] ** 2 + y[..., 8:] ** 2
    else:
        n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n0, n1, atol=1e-12)
    # inverse rotation: rotating by -p undoes p (per token: same p for one token)
    one = x[:1]
    back = oracle.rope_apply(oracle.rope_apply(one, 777, style=style), -777, style=style)
    assert np.allclose(back, one, atol=1e-12)
    # relative position: <R_m q, R_n k> depends on m - n only
    q, k = x[:1], x[1:2]
    for m, n, t in [(3, 10, 5), (100, 7, 12345)]:
        a = np.sum(oracle.rope_apply(q, m, style=style) * oracle.rope_apply(k, n, style=style), axis=-1)
        b = np.sum(oracle.rope_apply(q, m + t, style=style) * oracle.rope_apply(k, n + t, style=style), axis=-1)
        assert np.allclose(a, b, atol=1e-9)
    # shard consistency: rope of a slice at its absolute start equals the slice of rope
    full = oracle.rope_apply(x, 0, style=style)
    for a, b in oracle.all_shard_bounds(S, 3):
        assert np.allclose(oracle.rope_apply(x[a:b], a, style=style), full[a:b], atol=0, rtol=0)


def test_frequency_table():
    f = oracle.rope_inv_freq(8, 10000.0)
    assert f[0] == 1.0
    assert np.allclose(f, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)

"""Pins of the oracle's RMSNorm and fused QK-norm + RoPE (CPU only).

RmsNorm is LayerNorm without the mean subtraction (NPU HunyuanImage-3.0模型推理
优化实践, RmsNorm算子优化); q and k heads are normalised, then rotated, before
attention (same page, 计算分解; 消除旋转位置编码冗余cast算子).  Pinned by an
explicit per-row loop, the scale invariance of the normalisation, the unit
mean square it produces, and the rotation's norm preservation.
"""
import math

import numpy as np

import oracle


def test_rms_norm_by_loops():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 2, 8))
    g = rng.standard_normal(8)
    eps = 1e-3
    y = oracle.rms_norm(x, g, eps)
    for t in range(3):
        for h in range(2):
            row = x[t, h]
            r = math.sqrt(math.fsum(v * v for v in row) / 8 + eps)
            for i in range(8):
                assert math.isclose(y[t, h, i], row[i] / r * g[i], rel_tol=1e-14, abs_tol=1e-15)


def test_scale_invariance_and_unit_mean_square():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 3, 16))
    ones = np.ones(16)
    a = oracle.rms_norm(x, ones, 0.0)
    b = oracle.rms_norm(x * 37.5, ones, 0.0)
    assert np.allclose(a, b, rtol=0, atol=1e-14)
    assert np.allclose(np.mean(a * a, axis=-1), 1.0, rtol=0, atol=1e-14)
    # the rotation keeps every pair's norm, so the row mean square stays 1 after RoPE
    y = oracle.qk_norm_rope(x, ones, 0.0, pos0=123)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-13)


def test_norm_then_rope_composition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 2, 8))
    g = rng.standard_normal(8)
    y = oracle.qk_norm_rope(x, g, 1e-6, pos0=7, style="interleaved")
    assert np.array_equal(y, oracle.rope_apply(oracle.rms_norm(x, g, 1e-6), 7, style="interleaved"))
    pos = rng.integers(0, 50, size=(5, 3))
    z = oracle.qk_norm_rope(x, g, 1e-6, pos=pos, sections=(2, 1, 1))
    assert np.array_equal(z, oracle.rope_apply_mx(oracle.rms_norm(x, g, 1e-6), pos, (2, 1, 1)))

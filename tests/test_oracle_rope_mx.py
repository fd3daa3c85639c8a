"""Pins of the oracle's multi-axis rotary embedding and packed video+audio positions (CPU only).

The pages slice a RoPE frequency table by the rank's token range
(MiniMax-H3-Comfy-NPU, 机制一) and apply the rotation to q and k
(NPU HunyuanImage-3.0模型推理优化实践, 消除旋转位置编码冗余cast算子); the
multi-axis split and the packed positions are readings (parity unpinned by the
pages).  Pinned here by: reduction to the 1-D oracle, an independent
complex-number formulation per axis, rotation-group properties (identity,
norms, relative positions per axis), and brute-force enumeration of the packed
grid.
"""
import cmath
import math

import numpy as np
import pytest

import oracle


def test_single_axis_reduces_to_1d():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 3, 16))
    for style in ("half", "interleaved"):
        pos = np.stack([np.arange(7) + 123, np.zeros(7), np.zeros(7)], axis=1)
        y = oracle.rope_apply_mx(x, pos, (8, 0, 0), 10000.0, style)
        assert np.array_equal(y, oracle.rope_apply(x, 123, 10000.0, style))


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_complex_multiplication_per_axis(style):
    rng = np.random.default_rng(6)
    s, H, d, theta = 4, 2, 12, 500.0
    sections = (2, 3, 1)
    x = rng.standard_normal((s, H, d))
    pos = rng.integers(0, 400, size=(s, 3))
    y = oracle.rope_apply_mx(x, pos, sections, theta, style)
    half = d // 2
    for t in range(s):
        for h in range(H):
            j = 0
            for a, n in enumerate(sections):
                for jj in range(n):
                    ang = pos[t, a] * theta ** (-2.0 * jj / (2 * n))
                    i1, i2 = (j, j + half) if style == "half" else (2 * j, 2 * j + 1)
                    z = complex(x[t, h, i1], x[t, h, i2]) * cmath.exp(1j * ang)
                    assert math.isclose(y[t, h, i1], z.real, abs_tol=1e-12)
                    assert math.isclose(y[t, h, i2], z.imag, abs_tol=1e-12)
                    j += 1


def test_identity_norms_and_relative_positions():
    rng = np.random.default_rng(7)
    d, sections = 16, (3, 3, 2)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    zero = np.zeros((1, 3))
    assert np.array_equal(oracle.rope_apply_mx(q, zero, sections), q)
    p = np.array([[5.0, 17.0, 3.0]])
    y = oracle.rope_apply_mx(q, p, sections)
    # pair norms are kept
    n0 = q[0, 0, :8] ** 2 + q[0, 0, 8:] ** 2
    n1 = y[0, 0, :8] ** 2 + y[0, 0, 8:] ** 2
    assert np.allclose(n0, n1, rtol=0, atol=1e-12)
    # <R(pq) q, R(pk) k> depends only on pq - pk, axis by axis
    pk = np.array([[2.0, 40.0, 9.0]])
    shift = np.array([[11.0, -6.0, 30.0]])
    a = np.dot(oracle.rope_apply_mx(q, p, sections).ravel(), oracle.rope_apply_mx(k, pk, sections).ravel())
    b = np.dot(oracle.rope_apply_mx(q, p + shift, sections).ravel(),
               oracle.rope_apply_mx(k, pk + shift, sections).ravel())
    assert math.isclose(a, b, rel_tol=0, abs_tol=1e-10)


def test_sections_must_cover_the_head():
    with pytest.raises(ValueError):
        oracle.rope_apply_mx(np.zeros((1, 1, 8)), np.zeros((1, 3)), (1, 1, 1))


def test_av_positions_brute_force():
    T, Hh, Ww, A = 3, 4, 5, 7
    full = []
    for t in range(T):
        for h in range(Hh):
            for w in range(Ww):
                full.append((t, h, w))
    full += [(j, 0, 0) for j in range(A)]
    full = np.array(full, dtype=np.int64)
    S = T * Hh * Ww + A
    assert np.array_equal(oracle.av_positions(T, Hh, Ww, A, 0, S), full)
    for a, b in [(0, 0), (5, 23), (59, 61), (60, 67), (17, 67)]:
        assert np.array_equal(oracle.av_positions(T, Hh, Ww, A, a, b), full[a:b])
    with pytest.raises(ValueError):
        oracle.av_positions(T, Hh, Ww, A, 0, S + 1)


def test_av_positions_768p_grid():
    """The 768P/15 s sequence: 91 latent frames of 48 x 84 video tokens, then 375 audio tokens."""
    T, Hh, Ww, A = 91, 48, 84, 375
    V = T * Hh * Ww
    assert V + A == 367287
    p = oracle.av_positions(T, Hh, Ww, A, V - 2, V + 2)
    assert p.tolist() == [[90, 47, 82], [90, 47, 83], [0, 0, 0], [1, 0, 0]]
    assert oracle.av_positions(T, Hh, Ww, A, 91821, 91822).tolist() == [[22, 37, 9]]  # 91821 = 22*4032 + 37*84 + 9

"""Pins of the oracle's attention (CPU only).

Local queries against the full key/value sequence (MiniMax-H3-Comfy-NPU,
机制一), unmasked softmax with scale 1/sqrt(d) (NPU HunyuanImage-3.0模型推理优化
实践, 消除FA中scale的冗余计算).  Pinned by a pure-Python brute force with
math.fsum, by torch's own scaled-dot-product attention in float64 on the CPU,
and by closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _brute(q, k, v, scale):
    sq, H, d = q.shape
    skv = k.shape[0]
    o = np.zeros((sq, H, d))
    lse = np.zeros((H, sq))
    for h in range(H):
        for i in range(sq):
            logits = [scale * math.fsum(q[i, h, c] * k[j, h, c] for c in range(d)) for j in range(skv)]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            z = math.fsum(w)
            lse[h, i] = mx + math.log(z)
            for c in range(d):
                o[i, h, c] = math.fsum(w[j] * v[j, h, c] for j in range(skv)) / z
    return o, lse


def test_brute_force_tiny():
    rng = np.random.default_rng(10)
    for sq, skv, H, d in [(5, 1, 1, 4), (7, 33, 2, 8), (3, 48, 2, 6)]:
        q, k, v = (rng.standard_normal((n, H, d)) for n in (sq, skv, skv))
        scale = 1 / math.sqrt(d)
        o, lse = oracle.attention(q, k, v)
        ob, lb = _brute(q, k, v, scale)
        assert np.max(np.abs(o - ob)) < 1e-12
        assert np.max(np.abs(lse - lb)) < 1e-12


def test_torch_sdpa_float64():
    rng = np.random.default_rng(11)
    for sq, skv, H, d in [(37, 91, 3, 16), (64, 300, 2, 64)]:
        q, k, v = (rng.standard_normal((n, H, d)) for n in (sq, skv, skv))
        o, lse = oracle.attention(q, k, v)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2))) for a in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy().transpose(1, 0, 2)
        assert np.max(np.abs(o - ref)) < 1e-12
        logits = torch.einsum("hid,hjd->hij", tq, tk) / math.sqrt(d)
        assert np.max(np.abs(lse - torch.logsumexp(logits, dim=-1).numpy())) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(12)
    sq, skv, H, d = 9, 57, 2, 8
    q, k, v = (rng.standard_normal((n, H, d)) for n in (sq, skv, skv))
    # rows of the softmax sum to one: V = 1 gives O = 1
    o, lse = oracle.attention(q, k, np.ones_like(v))
    assert np.allclose(o, 1.0, atol=1e-14)
    # Q = 0: uniform weights, O is the mean of V, LSE = log(skv)
    o, lse = oracle.attention(np.zeros_like(q), k, v)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14)
    assert np.allclose(lse, math.log(skv), atol=1e-14)
    # one key: O = v_0, LSE = scale <q, k_0>
    o, lse = oracle.attention(q, k[:1], v[:1])
    assert np.allclose(o, np.broadcast_to(v[0], o.shape), atol=1e-14)
    assert np.allclose(lse, np.einsum("ihd,hd->hi", q, k[0]) / math.sqrt(d), atol=1e-13)
    # a dominant key wins: q aligned with k_5 and scaled up
    qd = np.repeat(k[5:6] * 50.0, sq, axis=0)
    o, _ = oracle.attention(qd, k, v)
    assert np.allclose(o, np.broadcast_to(v[5], o.shape), atol=1e-9)


def test_softmax_weights_sum_to_one_from_lse():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((n, 2, 16)) for n in (4, 100, 100))
    _, lse = oracle.attention(q, k, v)
    for h in range(2):
        L = (q[:, h] @ k[:, h].T) / 4.0
        assert np.allclose(np.exp(L - lse[h][:, None]).sum(axis=1), 1.0, atol=1e-13)


def test_large_logits_no_overflow():
    rng = np.random.default_rng(14)
    q, k, v = (rng.standard_normal((n, 1, 8)) for n in (3, 20, 20))
    o, lse = oracle.attention(q * 400.0, k, v)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_permutation_invariance_and_shard_concat():
    rng = np.random.default_rng(15)
    S, H, d, W = 61, 2, 8, 4
    q, k, v = (rng.standard_normal((S, H, d)) for _ in range(3))
    full, lse = oracle.attention(q, k, v)
    perm = rng.permutation(S)
    o2, _ = oracle.attention(q, k[perm], v[perm])
    assert np.allclose(full, o2, atol=1e-13)
    parts = [oracle.attention(q[a:b], k, v)[0] for a, b in oracle.all_shard_bounds(S, W)]
    assert np.array_equal(oracle.output_concat(parts), full)


def test_attention_rows_matches_full():
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((n, 3, 16)) for n in (50, 77, 77))
    full, lse = oracle.attention(q, k, v)
    rows = np.array([0, 7, 49])
    o, l = oracle.attention_rows(q[rows], k, v)
    assert np.allclose(o, full[rows], atol=1e-14) and np.allclose(l, lse[:, rows], atol=1e-14)


@pytest.mark.parametrize("bad", ["k", "v"])
def test_shape_mismatch(bad):
    q = np.zeros((2, 2, 4))
    k = np.zeros((3, 2, 4))
    v = np.zeros((3, 2, 4))
    if bad == "k":
        k = np.zeros((3, 1, 4))
    else:
        v = np.zeros((4, 2, 4))
    with pytest.raises(ValueError):
        oracle.attention(q, k, v)

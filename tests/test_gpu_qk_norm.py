"""GPU parity of qk_norm_rope (per-head RMSNorm fused with RoPE) against the float64 oracle.

Page NPU HunyuanImage-3.0模型推理优化实践: q and k heads are normalised after
the QKV projection and then rotated (计算分解); RmsNorm is LayerNorm without the
mean subtraction (RmsNorm算子优化).  Tolerances from the float32 arithmetic:
the row's sum of squares, rsqrt, scaling and rotation each stay within a few
float32 ulps, about 16 u (|n1| + |n2|) <= 2e-6 * max|y| per element in all,
so float32 results must lie within 4e-6 * max|ref|; bf16 results are that
float32 value rounded once, so within one bf16 ulp of the exact result plus
4e-6 * max|ref|.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_gamma, gen_tensor
from tests._helpers import bf16_ulp, to_dev, to_f64, to_host_bits

pytestmark = pytest.mark.gpu


def _check(got, ref, dtype):
    tol = 4e-6 * float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    if dtype == "f32":
        assert np.max(err) <= tol, (np.max(err), tol)
    else:
        assert np.all(err <= bf16_ulp(ref) + tol), np.max(err - bf16_ulp(ref))


SHAPES = [(301, 3, 128), (64, 2, 64), (17, 1, 12), (9, 5, 2), (33, 9, 256), (5, 2, 1024), (40, 2, 120)]


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("s,H,d", SHAPES)
def test_qk_norm_rope_1d_vs_oracle(style, dtype, s, H, d):
    pos0, eps = 91821, 1e-6
    x = gen_tensor(seed=s + d, tensor_id=0, S=s, H=H, d=d, dtype=dtype)
    g = gen_gamma(s, d)
    xd = to_dev(x, dtype)
    y = sp.qk_norm_rope(xd, torch.from_numpy(g).cuda(), eps, pos0, style=style, out=torch.empty_like(xd))
    torch.cuda.synchronize()
    ref = oracle.qk_norm_rope(to_f64(x), g.astype(np.float64), eps, pos0=pos0, style=style)
    _check(to_f64(y), ref, dtype)
    assert to_host_bits(xd).tobytes() == x.tobytes()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("s,H,d,sections", [(301, 3, 128, (22, 21, 21)), (17, 2, 12, (2, 2, 2)),
                                             (33, 9, 256, (0, 64, 64))])
def test_qk_norm_rope_multi_axis_vs_oracle(dtype, s, H, d, sections):
    rng = np.random.default_rng(s)
    pos = rng.integers(0, 100000, size=(s, 3)).astype(np.int64)
    x = gen_tensor(seed=s, tensor_id=1, S=s, H=H, d=d, dtype=dtype)
    g = gen_gamma(s + 1, d)
    xd = to_dev(x, dtype)
    y = sp.qk_norm_rope(xd, torch.from_numpy(g).cuda(), 1e-5, pos=torch.from_numpy(pos).cuda(), sections=sections,
                        out=torch.empty_like(xd))
    torch.cuda.synchronize()
    ref = oracle.qk_norm_rope(to_f64(x), g.astype(np.float64), 1e-5, pos=pos, sections=sections)
    _check(to_f64(y), ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place_equals_out_of_place(dtype):
    s, H, d = 1031, 24, 128
    x = to_dev(gen_tensor(seed=5, tensor_id=2, S=s, H=H, d=d, dtype=dtype), dtype)
    g = torch.from_numpy(gen_gamma(5, d)).cuda()
    a = sp.qk_norm_rope(x, g, 1e-6, 7, out=torch.empty_like(x))
    b = sp.qk_norm_rope(x.clone(), g, 1e-6, 7)
    torch.cuda.synchronize()
    assert to_host_bits(a).tobytes() == to_host_bits(b).tobytes()


def test_zero_rows_scaled_rows_and_unit_weight():
    """All-zero rows stay zero (eps > 0); with eps = 0 a row times 2^10 gives the same bits as the
    row itself (float32 scales the sum of squares, sqrt and reciprocal exactly by powers of two);
    with gamma = 1 token 0 at position 0 comes out as the normalised input (rotation by angle 0)."""
    s, H, d = 64, 4, 128
    x = gen_tensor(seed=9, tensor_id=0, S=s, H=H, d=d, dtype="f32")
    x[3] = 0.0
    ones = torch.ones(d, dtype=torch.float32, device="cuda")
    y = sp.qk_norm_rope(to_dev(x, "f32"), ones, 1e-6, 0, out=torch.empty(s, H, d, device="cuda")).cpu().numpy()
    assert np.all(y[3] == 0.0)
    x0 = x[0].astype(np.float64)
    r0 = x0 / np.sqrt(np.mean(x0 ** 2, axis=-1, keepdims=True) + 1e-6)
    assert np.max(np.abs(y[0] - r0)) <= 4e-6 * np.max(np.abs(r0))
    pair = np.stack([x[4], x[4] * np.float32(1024.0)])  # two tokens, the second a scaled copy
    one = to_dev(pair, "f32")
    ya = sp.qk_norm_rope(one[0:1], ones, 0.0, 100, out=torch.empty(1, H, d, device="cuda"))
    yb = sp.qk_norm_rope(one[1:2], ones, 0.0, 100, out=torch.empty(1, H, d, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)


def test_packed_768p_rank_slices_sampled():
    """Rank 0's query slice of the 768P/15 s sequence (91,821 tokens x 24 heads) with 1-D absolute
    positions, and the last rank's slice with packed video+audio positions, 2,000 sampled tokens each
    (first and last included) against the oracle."""
    T, Hh, Ww, A = 91, 48, 84, 375
    S, W, H, d = T * Hh * Ww + A, 4, 24, 128
    V = T * Hh * Ww
    g = gen_gamma(11, d)
    gd = torch.from_numpy(g).cuda()
    rng = np.random.default_rng(12)
    for r in (0, W - 1):
        a, b = sp.sp_shard_bounds(S, W, r)
        x = gen_tensor(seed=13, tensor_id=0, S=S, H=H, d=d, dtype="bf16", tok0=a, tok1=b)
        xd = to_dev(x, "bf16")
        idx = np.unique(np.concatenate([[0, b - a - 1], rng.integers(0, b - a, 2000)]))
        if r == 0:
            sp.qk_norm_rope(xd, gd, 1e-6, a)
            pos = np.zeros((len(idx), 3), dtype=np.int64)
            pos[:, 0] = a + idx
            ref = oracle.qk_norm_rope(to_f64(x[idx]), g.astype(np.float64), 1e-6, pos=pos, sections=(d // 2, 0, 0))
        else:
            posd = sp.sp_av_positions(T, Hh, Ww, A, a, b)
            v_end = min(b, V) - a
            sp.qk_norm_rope(xd[:v_end], gd, 1e-6, pos=posd[:v_end].cuda(), sections=(22, 21, 21))
            sp.qk_norm_rope(xd[v_end:], gd, 1e-6, pos=posd[v_end:].cuda(), sections=(d // 2, 0, 0))
            pos = oracle.av_positions(T, Hh, Ww, A, a, b)[idx]
            vid = idx < v_end
            ref = np.empty((len(idx), H, d))
            ref[vid] = oracle.qk_norm_rope(to_f64(x[idx[vid]]), g.astype(np.float64), 1e-6, pos=pos[vid],
                                           sections=(22, 21, 21))
            ref[~vid] = oracle.qk_norm_rope(to_f64(x[idx[~vid]]), g.astype(np.float64), 1e-6, pos=pos[~vid],
                                            sections=(d // 2, 0, 0))
        torch.cuda.synchronize()
        _check(to_f64(xd)[idx], ref, "bf16")


def test_wrapper_and_unsupported_head_size():
    x = torch.zeros(4, 2, 130, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sp.SpattnError):
        sp.qk_norm_rope(x, torch.ones(130, device="cuda"))          # d/2 = 65 pairs do not fit one wave
    with pytest.raises(ValueError):
        sp.qk_norm_rope(x[..., :128].contiguous(), torch.ones(130, device="cuda"))
    with pytest.raises(ValueError):
        sp.qk_norm_rope(x[..., :128].contiguous(), torch.ones(128, device="cuda"), pos=torch.zeros(4, 3,
                        dtype=torch.int64, device="cuda"))          # sections missing


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,offset", [(128, 1), (128, 2), (64, 1)])
def test_qk_norm_rope_unaligned_buffers(style, dtype, d, offset):
    """Buffers starting a few elements into an allocation take narrower vector accesses (fewer
    pairs per lane, so the row's sum of squares is added in another order): within the bars of
    the oracle, like the aligned call."""
    s, H = 21, 6
    x = gen_tensor(seed=d + offset, tensor_id=1, S=s, H=H, d=d, dtype=dtype)
    xd = to_dev(x, dtype)
    g = torch.from_numpy(gen_gamma(3, d)).cuda()
    n = s * H * d
    src = torch.empty(n + offset, dtype=xd.dtype, device="cuda")[offset:].view(s, H, d)
    src.copy_(xd)
    out = torch.empty(n + offset, dtype=xd.dtype, device="cuda")[offset:].view(s, H, d)
    sp.qk_norm_rope(src, g, 1e-6, 99, style=style, out=out)
    aligned = sp.qk_norm_rope(xd, g, 1e-6, 99, style=style, out=torch.empty_like(xd))
    torch.cuda.synchronize()
    ref = oracle.qk_norm_rope(to_f64(x), gen_gamma(3, d).astype(np.float64), 1e-6, pos0=99, style=style)
    _check(to_f64(aligned), ref, dtype)
    _check(to_f64(out), oracle.qk_norm_rope(to_f64(x), gen_gamma(3, d).astype(np.float64), 1e-6, pos0=99,
                                            style=style), dtype)

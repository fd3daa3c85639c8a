"""GPU parity of rope_apply against the float64 oracle.

Rotary embedding of the rank's local slice at absolute packed positions
(MiniMax-H3-Comfy-NPU, 机制一; rotate_half form of NPU HunyuanImage-3.0模型推理优化
实践, 消除旋转位置编码冗余cast算子).  Tolerance: float32 storage within 2e-6
absolute (float32 rotation of |x| < 6 inputs with float32 cos/sin); bf16 storage
within one bf16 ulp of the exact result plus 1e-6 (one rounding of a float32
result that is itself within a few float32 ulps of |x|).
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_tensor, get_workload
from tests._helpers import bf16_ulp, to_dev, to_f64, to_host_bits

pytestmark = pytest.mark.gpu


def _check(got, ref, dtype):
    if dtype == "f32":
        assert np.max(np.abs(got - ref)) <= 2e-6
    else:
        # one bf16 ulp, plus the float32 rotation's own error where the pair cancels
        assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-6)


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("s,H,d,pos0", [(250, 2, 64, 250), (4096, 16, 128, 12287), (33, 3, 6, 5),
                                        (7, 1, 2, 0), (129, 24, 128, 367000), (5, 2, 8, -40)])
def test_rope_vs_oracle(style, dtype, s, H, d, pos0):
    x = gen_tensor(seed=s + d, tensor_id=0, S=s, H=H, d=d, dtype=dtype)
    xd = to_dev(x, dtype)
    y = torch.empty_like(xd)
    sp.rope_apply(xd, pos0, 10000.0, style, out=y)
    torch.cuda.synchronize()
    ref = oracle.rope_apply(to_f64(x), pos0, 10000.0, style)
    _check(to_f64(y), ref, dtype)
    # input untouched by an out-of-place call
    assert to_host_bits(xd).tobytes() == x.tobytes()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_shard_equals_full_bitwise_and_in_place(dtype):
    wl = get_workload("uneven_bf16")
    x = gen_tensor(wl.seed, 1, wl.S, wl.H, wl.d, dtype)
    xd = to_dev(x, dtype)
    full = sp.rope_apply(xd, 0, out=torch.empty_like(xd))
    parts = []
    for r in range(wl.W):
        a, b = sp.sp_shard_bounds(wl.S, wl.W, r)
        parts.append(sp.rope_apply(xd[a:b].clone(), a))  # in place on a copy
    torch.cuda.synchronize()
    assert to_host_bits(torch.cat(parts)).tobytes() == to_host_bits(full).tobytes()
    # position 0 rotates by angle 0: the first token is unchanged, bit for bit
    assert to_host_bits(full[0]).tobytes() == x[0].tobytes()


def test_rope_workload_ranks_bf16():
    wl = get_workload("uneven_bf16")
    q = gen_tensor(wl.seed, 0, wl.S, wl.H, wl.d, wl.dtype)
    for r in wl.ranks:
        a, b = sp.sp_shard_bounds(wl.S, wl.W, r)
        yd = sp.rope_apply(to_dev(q[a:b], "bf16"), a, wl.theta)
        torch.cuda.synchronize()
        _check(to_f64(yd), oracle.rope_apply(to_f64(q[a:b]), a, wl.theta), "bf16")


def test_rope_empty_is_noop():
    x = torch.zeros(0, 2, 8, device="cuda", dtype=torch.bfloat16)
    sp.rope_apply(x, 5)
    torch.cuda.synchronize()


@pytest.mark.parametrize("style", ["half", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,offset", [(128, 1), (128, 2), (130, 0), (256, 1), (1024, 0), (24, 3)])
def test_rope_layouts_and_alignments_vs_oracle(style, dtype, d, offset):
    """Buffers that start `offset` elements into an allocation (narrower vector accesses or the
    element-wise kernel) and head sizes whose rows do not fit one wave in groups of 1, 2, 4 or 8
    pairs (d = 130) give the same results as the aligned case, within the RoPE bars."""
    s, H, pos0 = 37, 5, 366000
    x = gen_tensor(seed=d + offset, tensor_id=0, S=s, H=H, d=d, dtype=dtype)
    xd = to_dev(x, dtype)
    n = s * H * d
    buf = torch.empty(n + offset, dtype=xd.dtype, device="cuda")
    src = buf[offset:].view(s, H, d)
    src.copy_(xd)
    out = torch.empty(n + offset, dtype=xd.dtype, device="cuda")[offset:].view(s, H, d)
    sp.rope_apply(src, pos0, style=style, out=out)
    aligned = sp.rope_apply(xd, pos0, style=style, out=torch.empty_like(xd))
    torch.cuda.synchronize()
    _check(to_f64(out), oracle.rope_apply(to_f64(x), pos0, style=style), dtype)
    assert to_host_bits(out).tobytes() == to_host_bits(aligned).tobytes()

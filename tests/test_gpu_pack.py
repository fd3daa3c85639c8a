"""GPU parity of varlen_pack / varlen_unpack against the oracle: bit-exact.

AllGatherV data movement (MiniMax-H3-Comfy-NPU, 后端 A): counts and
displacements into a flat buffer, then narrow/view/concat.  W separate device
buffers stand in for the W ranks.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from sequence_dit_attention_amd import SpattnError
from synth import gen_tensor, get_workload
from tests._helpers import to_dev, to_host_bits

pytestmark = pytest.mark.gpu

SENT = {"bf16": 0x7FC1, "f32": np.float32(-12345.5)}


def _host_rand(rng, n, dtype):
    if dtype == "bf16":
        return rng.integers(0, 0x7F00, size=n, dtype=np.uint16)
    return rng.standard_normal(n).astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,displs,flat_n", [
    ([5, 0, 7, 3], [20, 2, 0, 9], 30),                  # odd sizes, permuted order, gaps
    ([4096, 4097, 1, 8191], [0, 4096, 8193, 8194], 16385),
    ([40000, 39999], [39999, 0], 80000),
    ([0], [0], 0),
    ([123457], [1], 123460),
    # 45 ranks, every third one empty: more segments than one copy launch takes (32)
    ([0 if r % 3 == 1 else 100 + r for r in range(45)],
     [sum(0 if q % 3 == 1 else 100 + q for q in range(r)) for r in range(45)], 4000),
])
def test_pack_bit_exact(dtype, counts, displs, flat_n):
    rng = np.random.default_rng(sum(counts) + 7)
    sends = [_host_rand(rng, c, dtype) for c in counts]
    guard = 64
    flat0 = np.full(flat_n + 2 * guard, SENT[dtype], dtype=np.uint16 if dtype == "bf16" else np.float32)
    dev_flat = to_dev(flat0, dtype)
    sp.varlen_pack([to_dev(s, dtype) for s in sends], counts, [d + guard for d in displs], dev_flat)
    torch.cuda.synchronize()
    want = oracle.varlen_pack(sends, counts, [d + guard for d in displs], flat0)
    got = to_host_bits(dev_flat)
    assert got.tobytes() == want.tobytes()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,W,outer,inner", [(16383, 4, 1, 64), (11, 4, 3, 5), (3, 5, 2, 7), (1000, 1, 1, 33),
                                             (257, 3, 4, 16)])
def test_unpack_bit_exact_and_round_trip(dtype, S, W, outer, inner):
    rng = np.random.default_rng(S * W + outer)
    x = _host_rand(rng, outer * S * inner, dtype).reshape(outer, S, inner)
    bounds = oracle.all_shard_bounds(S, W)
    lens = [b - a for a, b in bounds]
    counts, displs = sp.sp_allgatherv_layout(S, W, outer, inner)
    shards = [np.ascontiguousarray(x[:, a:b, :]).ravel() for a, b in bounds]
    flat = torch.zeros(sum(counts), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
    sp.varlen_pack([to_dev(s, dtype) for s in shards], counts, displs, flat)
    guard = 32
    out_buf = to_dev(np.full(outer * S * inner + 2 * guard, SENT[dtype],
                             dtype=np.uint16 if dtype == "bf16" else np.float32), dtype)
    out = out_buf[guard:guard + outer * S * inner]
    sp.varlen_unpack(flat, displs, lens, outer, inner, out)
    torch.cuda.synchronize()
    want = oracle.varlen_unpack(oracle.varlen_pack(shards, counts, displs, np.zeros(sum(counts), x.dtype)),
                                displs, lens, outer, inner)
    got_all = to_host_bits(out_buf)
    assert got_all[guard:-guard].tobytes() == want.tobytes()
    assert got_all[guard:-guard].tobytes() == x.tobytes()
    assert np.all(got_all[:guard] == SENT[dtype]) and np.all(got_all[-guard:] == SENT[dtype])


def test_uneven_workload_kv_pack():
    wl = get_workload("uneven_bf16")
    k = gen_tensor(wl.seed, 1, wl.S, wl.H, wl.d, wl.dtype)
    bounds = [sp.sp_shard_bounds(wl.S, wl.W, r) for r in range(wl.W)]
    assert [b - a for a, b in bounds] == [4095, 4096, 4096, 4096]
    counts, displs = sp.sp_allgatherv_layout(wl.S, wl.W, 1, wl.H * wl.d)
    kd = to_dev(k, "bf16")
    flat = torch.empty(sum(counts), dtype=torch.bfloat16, device="cuda")
    sp.varlen_pack([kd[a:b].reshape(-1) for a, b in bounds], counts, displs, flat)
    full = torch.empty_like(kd)
    sp.varlen_unpack(flat, displs, [b - a for a, b in bounds], 1, wl.H * wl.d, full)
    torch.cuda.synchronize()
    want = oracle.varlen_pack([k[a:b].ravel() for a, b in bounds], counts, displs, np.zeros(sum(counts), np.uint16))
    assert to_host_bits(flat).tobytes() == want.tobytes()
    assert to_host_bits(full).tobytes() == k.tobytes()


def test_exchange_sim_cat_dims():
    x = torch.randn(2, 37, 3, 4, device="cuda").to(torch.bfloat16)
    for cat_dim in (0, 1, 2, -1, -4):
        n = x.shape[cat_dim]
        cuts = [0, n // 3, n // 3, n]  # includes an empty shard
        shards = [x.narrow(cat_dim, cuts[i], cuts[i + 1] - cuts[i]).contiguous() for i in range(3)]
        got = sp.exchange_sim(shards, cat_dim)
        torch.cuda.synchronize()
        assert to_host_bits(got).tobytes() == to_host_bits(x.contiguous()).tobytes()


def test_device_errors():
    a = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    flat = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(SpattnError) as ei:
        sp.varlen_pack([a, a], [8, 8], [0, 4], flat)
    assert ei.value.code == -4
    with pytest.raises(SpattnError) as ei:
        sp.varlen_pack([a], [16], [1], flat)
    assert ei.value.code == -3
    with pytest.raises(SpattnError) as ei:
        sp.varlen_pack([flat[2:10]], [8], [0], flat)
    assert ei.value.code == -4

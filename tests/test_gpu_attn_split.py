"""GPU parity of shard_attn_fwd_split: attention with the keys cut into ranges, merged by their LSE.

The single-head attention of the VAE block split (NPU HunyuanImage-3.0模型推理优化实践,
VAE并行优化) has a few thousand queries per process, too few work-groups to fill
the GPU; cutting the gathered keys into ranges and combining the per-range
softmax results by their log-sum-exp is the same softmax over the union.  Bars:
nsplit = 1 bit-identical to shard_attn_fwd (one weight of exactly 1); otherwise
the bf16 attention bars against the oracle (max abs error <= 2e-2 and
<= 1e-2 * max|O_ref|, LSE within 2e-2), on ragged key counts, ranges of one
tile, and the workload size of a 128 x 128 latent split 2 x 2.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import bf16_bits_to_f32, gen_tensor, sample_rows
from tests._helpers import attn_errors, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _inputs(seed, sq, skv, H, d):
    q = gen_tensor(seed, 0, sq, H, d, "bf16")
    k = gen_tensor(seed, 1, skv, H, d, "bf16")
    v = gen_tensor(seed, 2, skv, H, d, "bf16")
    return q, k, v, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")


@pytest.mark.parametrize("d", [64, 128, 512])
def test_one_range_is_bitwise_the_plain_call(d):
    sq, skv, H = 300, 1000, 2
    _, _, _, qd, kd, vd = _inputs(31, sq, skv, H, d)
    l1 = torch.empty(H, sq, device="cuda")
    l2 = torch.empty_like(l1)
    o1 = sp.shard_attn_fwd(qd, kd, vd, lse=l1)
    o2 = sp.shard_attn_fwd_split(qd, kd, vd, 1, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("d,sq,skv,H,nsplit", [(128, 257, 1000, 2, 3), (128, 64, 4096, 1, 64), (64, 100, 777, 3, 7),
                                               (512, 129, 300, 1, 5), (512, 33, 1000, 2, 16), (512, 300, 65, 1, 2)])
def test_split_vs_oracle(d, sq, skv, H, nsplit):
    q, k, v, qd, kd, vd = _inputs(32 + d, sq, skv, H, d)
    ws = torch.full((sp.split_workspace_bytes(sq, H, d, nsplit),), 255, dtype=torch.uint8, device="cuda")  # NaNs
    lse = torch.empty(H, sq, device="cuda")
    o = sp.shard_attn_fwd_split(qd, kd, vd, nsplit, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    err, rel = attn_errors(to_f64(o), ro)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    assert np.max(np.abs(lse.cpu().numpy() - rl)) <= 2e-2


def test_vae_128x128_block_sampled_rows():
    """Process 0 of a 128 x 128 latent split 2 x 2: 4,096 queries of its block against the 16,384
    gathered keys, 512 channels, 4 key ranges; 48 sampled query rows against the oracle."""
    Hh = Ww = 128
    C, pr, pc = 512, 2, 2
    n = Hh * Ww
    q = gen_tensor(33, 0, n, 1, C, "bf16").reshape(Hh, Ww, C)
    k = gen_tensor(33, 1, n, 1, C, "bf16")
    v = gen_tensor(33, 2, n, 1, C, "bf16")
    r0, r1, c0, c1 = sp.sp_tile_bounds(Hh, Ww, pr, pc, 0)
    qb = np.ascontiguousarray(q[r0:r1, c0:c1].reshape(-1, 1, C))
    kf = sp.tile_pack(to_dev(k.reshape(Hh, Ww, C), "bf16"), pr, pc).reshape(n, 1, C)
    vf = sp.tile_pack(to_dev(v.reshape(Hh, Ww, C), "bf16"), pr, pc).reshape(n, 1, C)
    o = sp.shard_attn_fwd_split(to_dev(qb, "bf16"), kf, vf, 4)
    torch.cuda.synchronize()
    rows = sample_rows(qb.shape[0], 48, seed=5)
    widen = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    ro, _ = oracle.attention_rows(widen(qb[rows]), k, v, widen=widen)   # raster-order keys
    err, rel = attn_errors(to_f64(o)[rows], ro)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)


def test_split_at_the_768p_5s_rank_share_sampled_rows():
    """Rank 3 of the 768P/5 s workload (31,280 queries x 125,117 keys x 24 heads of 128) with 3 key ranges:
    32 sampled query rows x all heads against the oracle, and the whole output within the bf16 bars of the
    plain call."""
    S, W, H, d = 125117, 4, 24, 128
    a, b = sp.sp_shard_bounds(S, W, 3)
    q = gen_tensor(4, 0, S, H, d, "bf16", tok0=a, tok1=b)
    k = gen_tensor(4, 1, S, H, d, "bf16")
    v = gen_tensor(4, 2, S, H, d, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o_split = sp.shard_attn_fwd_split(qd, kd, vd, 3)
    o_plain = sp.shard_attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    rows = sample_rows(b - a, 32, seed=6)
    widen = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    ro, _ = oracle.attention_rows(widen(q[rows]), k, v, widen=widen)
    err, rel = attn_errors(to_f64(o_split)[rows], ro)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    d_all = (o_split.float() - o_plain.float()).abs().max().item()
    assert d_all <= 2e-2 and d_all <= 1e-2 * o_plain.float().abs().max().item(), d_all

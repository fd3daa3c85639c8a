"""GPU parity of the head-size-512 bf16 attention and of the VAE block-split attention.

NPU HunyuanImage-3.0模型推理优化实践, VAE并行优化: each process holds one
spatial block of the feature map; attention gathers K and V of all blocks; the
outputs are gathered back into place in two stages.  The attention is read as
the usual single-head VAE attention over all C = 512 channels.  Bars as for the
other bf16 attention: max abs error <= 2e-2 and <= 1e-2 * max|O_ref|; LSE
within 2e-2.  The block split changes the order in which keys arrive, so the
block-split result is compared with the unsplit one within tolerance, not bit
for bit; each run on its own is deterministic.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_tensor
from tests._helpers import attn_errors, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _bf16_ok(got, ref):
    err, rel = attn_errors(got, ref)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)


@pytest.mark.parametrize("sq,skv,H", [(1, 1, 1), (100, 37, 1), (129, 300, 2), (257, 1000, 1), (128, 64, 1),
                                      (33, 31, 3)])
def test_d512_vs_oracle(sq, skv, H):
    d = 512
    q = gen_tensor(21, 0, sq, H, d, "bf16")
    k = gen_tensor(21, 1, skv, H, d, "bf16")
    v = gen_tensor(21, 2, skv, H, d, "bf16")
    lse = torch.empty(H, sq, dtype=torch.float32, device="cuda")
    o = sp.shard_attn_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    _bf16_ok(to_f64(o), ro)
    assert np.max(np.abs(lse.cpu().numpy() - rl)) <= 2e-2


def test_d512_peaky_scores_and_determinism():
    """Q x 4 (exact in bf16) makes the softmax peaky; two runs agree bit for bit, and a query
    row gives the same bits wherever it sits in q."""
    sq, skv, d = 200, 777, 512
    q = gen_tensor(22, 0, sq, 1, d, "bf16")
    k = gen_tensor(22, 1, skv, 1, d, "bf16")
    v = gen_tensor(22, 2, skv, 1, d, "bf16")
    qd = to_dev(q, "bf16") * 4
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    o1 = sp.shard_attn_fwd(qd, kd, vd)
    o2 = sp.shard_attn_fwd(qd, kd, vd)
    o3 = sp.shard_attn_fwd(qd[57:60].contiguous(), kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1[57:60].view(torch.int16), o3.view(torch.int16))
    ro, _ = oracle.attention(to_f64(qd), to_f64(k), to_f64(v))
    _bf16_ok(to_f64(o1), ro)


def test_f32_and_gather_free_reject_d512():
    x = torch.zeros(4, 1, 512, device="cuda")
    with pytest.raises(sp.SpattnError):
        sp.shard_attn_fwd(x, x, x)
    xb = x.to(torch.bfloat16)
    with pytest.raises(sp.SpattnError):
        sp.shard_attn_fwd_gv(xb, [xb], [xb])


@pytest.mark.parametrize("Hh,Ww,pr,pc", [(24, 20, 2, 2), (17, 30, 3, 2)])
def test_vae_block_split_attention(Hh, Ww, pr, pc):
    """Every process: its block's queries against the K/V of all blocks gathered in process order;
    the outputs gathered in process order and put back in place equal the attention of the whole
    feature map (oracle), and the unsplit GPU attention, within tolerance."""
    C = 512
    n = Hh * Ww
    q = gen_tensor(23, 0, n, 1, C, "bf16").reshape(Hh, Ww, C)
    k = gen_tensor(23, 1, n, 1, C, "bf16").reshape(Hh, Ww, C)
    v = gen_tensor(23, 2, n, 1, C, "bf16").reshape(Hh, Ww, C)
    qd, kd, vd = (to_dev(t, "bf16") for t in (q, k, v))
    kf = sp.tile_pack(kd, pr, pc)                    # the AllGatherV of the K blocks, process order
    vf = sp.tile_pack(vd, pr, pc)
    qf = sp.tile_pack(qd, pr, pc)                    # block p's queries sit at its offset
    of = torch.empty_like(qf)
    off = 0
    for p in range(pr * pc):
        r0, r1, c0, c1 = sp.sp_tile_bounds(Hh, Ww, pr, pc, p)
        m = (r1 - r0) * (c1 - c0)
        sp.shard_attn_fwd(qf[off:off + m].reshape(m, 1, C), kf.reshape(n, 1, C), vf.reshape(n, 1, C),
                          out=of[off:off + m].reshape(m, 1, C))
        off += m
    o = sp.tile_unpack(of, Hh, Ww, pr, pc)
    whole = sp.shard_attn_fwd(qd.reshape(n, 1, C), kd.reshape(n, 1, C), vd.reshape(n, 1, C))
    torch.cuda.synchronize()
    ro, _ = oracle.attention(to_f64(q).reshape(n, 1, C), to_f64(k).reshape(n, 1, C), to_f64(v).reshape(n, 1, C))
    _bf16_ok(to_f64(o).reshape(n, 1, C), ro)
    _bf16_ok(to_f64(whole), ro)


def test_vae_block_share_step():
    """The pipeline's step for process 4 of a 40 x 36 map cut 2 x 3: gather, split attention into the
    process's slot, placement; its block of the output raster matches the oracle, other blocks keep
    their stand-in zeros."""
    from sequence_dit_attention_amd.pipeline import VaeBlockShare
    Hh, Ww, C, pr, pc, p = 40, 36, 512, 2, 3, 4
    n = Hh * Ww
    q, k, v = (gen_tensor(24, t, n, 1, C, "bf16").reshape(Hh, Ww, C) for t in range(3))
    vs = VaeBlockShare(Hh, Ww, C, pr, pc, p, nsplit=3)
    vs.set_inputs(*(to_dev(t, "bf16") for t in (q, k, v)))
    vs.step()
    torch.cuda.synchronize()
    got = to_f64(vs.o)
    r0, r1, c0, c1 = oracle.tile_bounds(Hh, Ww, pr, pc, p)
    qb = to_f64(q)[r0:r1, c0:c1].reshape(-1, 1, C)
    ro, _ = oracle.attention(qb, to_f64(k).reshape(n, 1, C), to_f64(v).reshape(n, 1, C))
    _bf16_ok(got[r0:r1, c0:c1].reshape(-1, 1, C), ro)
    mask = np.ones((Hh, Ww), dtype=bool)
    mask[r0:r1, c0:c1] = False
    assert np.all(got[mask] == 0.0)


def test_vae_128x128_all_processes_reassembled():
    """All 4 processes of a 128 x 128 x 512 map cut 2 x 2, each with split-key attention (4 ranges)
    against the gathered keys; the outputs gathered in process order and placed with tile_unpack match the
    unsplit attention of the whole map within the bf16 bars, and 24 sampled pixels match the oracle."""
    from synth import bf16_bits_to_f32
    Hh = Ww = 128
    C, pr, pc = 512, 2, 2
    n = Hh * Ww
    q, k, v = (gen_tensor(25, t, n, 1, C, "bf16").reshape(Hh, Ww, C) for t in range(3))
    qd, kd, vd = (to_dev(t, "bf16") for t in (q, k, v))
    kf = sp.tile_pack(kd, pr, pc).view(n, 1, C)
    vf = sp.tile_pack(vd, pr, pc).view(n, 1, C)
    qf = sp.tile_pack(qd, pr, pc)
    of = torch.empty_like(qf)
    off = 0
    for p in range(pr * pc):
        r0, r1, c0, c1 = sp.sp_tile_bounds(Hh, Ww, pr, pc, p)
        m = (r1 - r0) * (c1 - c0)
        sp.shard_attn_fwd_split(qf[off:off + m].view(m, 1, C), kf, vf, 4, out=of[off:off + m].view(m, 1, C))
        off += m
    o = sp.tile_unpack(of, Hh, Ww, pr, pc)
    whole = sp.shard_attn_fwd(qd.view(n, 1, C), kd.view(n, 1, C), vd.view(n, 1, C))
    torch.cuda.synchronize()
    dif = (o.view(n, 1, C).float() - whole.float()).abs().max().item()
    assert dif <= 2e-2 and dif <= 1e-2 * whole.float().abs().max().item(), dif
    rng = np.random.default_rng(9)
    pix = rng.integers(0, n, 24)
    widen = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    ro, _ = oracle.attention_rows(widen(q.reshape(n, 1, C)[pix]), k.reshape(n, 1, C), v.reshape(n, 1, C),
                                  widen=widen)
    err, rel = attn_errors(to_f64(o).reshape(n, 1, C)[pix], ro)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)


def test_vae_block_share_graph_replays_match_eager():
    """The VAE share's step recorded as a HIP graph: every replay, with eager work and
    synchronisations between replays and the output raster poisoned before each, gives
    the eager step's raster bit for bit; after the V raster changes in place, a replay
    gives what an eager step gives on the new values."""
    from sequence_dit_attention_amd.pipeline import VaeBlockShare
    Hh, Ww, C, pr, pc, p = 40, 36, 512, 2, 3, 4
    n = Hh * Ww
    q, k, v = (gen_tensor(26, t, n, 1, C, "bf16").reshape(Hh, Ww, C) for t in range(3))
    vs = VaeBlockShare(Hh, Ww, C, pr, pc, p, nsplit=3)
    vs.set_inputs(*(to_dev(t, "bf16") for t in (q, k, v)))
    vs.step()
    torch.cuda.synchronize()
    eager = vs.o.clone()
    g = vs.capture()
    torch.cuda.synchronize()
    side = torch.randn(512, 512, device="cuda")
    for i in range(4):
        vs.o.fill_(float("nan"))
        side = torch.tanh(side @ side.T / 512.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(vs.o.view(torch.int16), eager.view(torch.int16)), i
    vs.v.neg_()
    vs.step()
    torch.cuda.synchronize()
    eager2 = vs.o.clone()
    assert not torch.equal(eager2.view(torch.int16), eager.view(torch.int16))
    vs.o.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(vs.o.view(torch.int16), eager2.view(torch.int16))

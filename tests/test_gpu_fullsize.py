"""Full-size workloads in the launch configuration the benchmark times.

The whole rank share (RoPE, K/V AllGatherV pack + unpack, attention, output
concat) runs through sequence_dit_attention_amd.pipeline.RankShare at the
workloads' real shapes.  The fp64 oracle is too slow for every output at these
sizes, so it is evaluated on sampled query rows (first/last rows, both sides
of 128-row tile edges, both sides of 256-row work-group boundaries spread over the
shard, the final partial work-group, random rows) for every head; pack/unpack are checked
bit-exactly on sampled elements and by the exact round-trip property, RoPE on
the sampled rows.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from sequence_dit_attention_amd.pipeline import RankShare
from synth import gen_qkv, get_workload, sample_rows
from tests._helpers import attn_errors, bf16_ulp, to_dev, to_f64, to_host_bits

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


def oracle_rows(q, k, v, rows_abs, theta, head_chunk=6):
    """fp64 oracle output/LSE of the given absolute query rows (RoPE applied)."""
    H, d = q.shape[1], q.shape[2]
    qrot = np.concatenate([oracle.rope_apply(to_f64(q[i:i + 1]), int(i), theta) for i in rows_abs])
    o = np.empty((len(rows_abs), H, d))
    lse = np.empty((H, len(rows_abs)))
    for h0 in range(0, H, head_chunk):
        h1 = min(H, h0 + head_chunk)
        kr = oracle.rope_apply(to_f64(k[:, h0:h1, :]), 0, theta)
        vr = to_f64(v[:, h0:h1, :])
        oo, ll = oracle.attention(qrot[:, h0:h1, :], kr, vr)
        o[:, h0:h1], lse[h0:h1] = oo, ll
        del kr, vr
    return qrot, o, lse


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["p480_w1", "p768_5s_w4", "p768_15s_w4"])
def test_fullsize_rank_share(name):
    wl = get_workload(name)
    r = wl.ranks[0]
    t0 = time.time()
    _log(f"{name}: generating S={wl.S} H={wl.H} d={wl.d}")
    q, k, v = gen_qkv(wl)
    share = RankShare(wl.S, wl.W, r, wl.H, wl.d, torch.bfloat16, wl.theta)
    share.set_inputs(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"))
    _log(f"{name}: inputs on device after {time.time() - t0:.1f}s; running the rank share")
    share.step()
    torch.cuda.synchronize()
    a, b = share.a, share.b
    # 32 sampled rows (first/last, 128-row tile edges, random), plus both sides of 24 work-group
    # boundaries (every 512 query rows form one work-group of the head-size-128 kernel, every 256
    # one of 64 rows per wave) spread evenly over the shard, and the first and last rows of the
    # final, partial work-group
    n = b - a
    wg = np.unique(np.linspace(1, max(1, (n - 1) // 256), 24).astype(np.int64)) * 256
    edges = np.concatenate([wg - 1, wg, [((n - 1) // 512) * 512, ((n - 1) // 256) * 256, n - 1]])
    rows = np.unique(np.concatenate([sample_rows(n, 32, seed=wl.seed), edges[(edges >= 0) & (edges < n)]]))
    rows_abs = rows + a
    _log(f"{name}: GPU done; oracle on {len(rows)} rows x {wl.H} heads")

    # pack/unpack: exact round trip, sampled elements of the flat buffers vs the definition
    for i, (lo, hi) in enumerate(share.bounds):
        assert torch.equal(share.k_full[lo:hi], share.k_rot[i])
        assert torch.equal(share.v_full[lo:hi], share.v[lo:hi])
        assert torch.equal(share.o_full[lo:hi], share.o_shards[i])
    rng = np.random.default_rng(wl.seed)
    for i, (lo, hi) in enumerate(share.bounds):
        n = (hi - lo) * share.inner
        if n == 0:
            continue
        idx = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 2000)]))
        ti = torch.from_numpy(idx).cuda()
        got = to_host_bits(share.flat_v[share.displs[i] + ti])
        want = v[lo:hi].reshape(-1)[idx]
        assert got.tobytes() == want.tobytes()

    qrot_ref, o_ref, lse_ref = oracle_rows(q, k, v, rows_abs, wl.theta)
    ti = torch.from_numpy(rows).cuda()
    q_got = to_f64(share.q_rot[ti])
    assert np.all(np.abs(q_got - qrot_ref) <= bf16_ulp(qrot_ref) + 1e-6)
    o_got = to_f64(share.o_shards[r][ti])
    err, rel = attn_errors(o_got, o_ref)
    lse_got = share.lse[:, ti].cpu().numpy()
    lerr = float(np.max(np.abs(lse_got - lse_ref)))
    _log(f"{name}: max abs err {err:.3e}, rel-to-max {rel:.3e}, max|O_ref| {np.max(np.abs(o_ref)):.3e}, "
         f"lse err {lerr:.3e}, total {time.time() - t0:.1f}s")
    assert err <= 2e-2 and rel <= 1e-2
    assert lerr <= 2e-2

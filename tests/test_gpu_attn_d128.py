"""GPU parity of the head-size-128 attention kernel at the edges of its own structure.

Page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", 机制一: local queries
against the full K/V, no mask.  The kernel works in 32-key steps, two tile
sets in flight, and 512-row work-groups (two 32-query blocks per wave), or
256-row ones (one block per wave) when the 512-row grid would leave CUs idle.
A row's arithmetic must not depend on which form runs it, so the same rows
computed in a small call (one head: the one-block form) and inside a large one
(256 heads: the two-block form) must agree bit for bit; both are checked
against the float64 oracle (bf16 bars: max abs error <= 2e-2 and
<= 1e-2 * max|O_ref|, LSE within 2e-2) at key counts around the step and tile
edges and query counts around the work-group edges.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_tensor
from tests._helpers import attn_errors, to_dev, to_f64

pytestmark = pytest.mark.gpu

WIDE = 256  # heads of the large call: at least 256 work-groups even for one 512-row tile per head


def _check_head(o, lse, q, k, v, h):
    ro, rl = oracle.attention(to_f64(q[:, h:h + 1]), to_f64(k[:, h:h + 1]), to_f64(v[:, h:h + 1]))
    err, rel = attn_errors(to_f64(o[:, h:h + 1]), ro)
    assert err <= 2e-2 and rel <= 1e-2, (h, err, rel)
    assert np.max(np.abs(lse[h].cpu().numpy() - rl[0])) <= 2e-2


@pytest.mark.parametrize("sq,skv", [(1, 1), (255, 31), (256, 32), (257, 33), (511, 63), (512, 64), (513, 65),
                                    (700, 97), (513, 129)])
def test_rows_identical_in_both_work_group_forms(sq, skv):
    d = 128
    q = gen_tensor(40, 0, sq, WIDE, d, "bf16")
    k = gen_tensor(40, 1, skv, WIDE, d, "bf16")
    v = gen_tensor(40, 2, skv, WIDE, d, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    lse_w = torch.empty(WIDE, sq, device="cuda")
    o_w = sp.shard_attn_fwd(qd, kd, vd, lse=lse_w)  # two query blocks per wave
    for h in (0, WIDE // 2, WIDE - 1):
        q1, k1, v1 = (t[:, h:h + 1].contiguous() for t in (qd, kd, vd))
        lse_1 = torch.empty(1, sq, device="cuda")
        o_1 = sp.shard_attn_fwd(q1, k1, v1, lse=lse_1)  # one head: one query block per wave
        torch.cuda.synchronize()
        assert torch.equal(o_1.view(torch.int16), o_w[:, h:h + 1].view(torch.int16)), h
        assert torch.equal(lse_1[0], lse_w[h]), h
        _check_head(o_w, lse_w, q, k, v, h)


@pytest.mark.parametrize("lens", [[5, 27, 100, 1], [32, 1, 31], [0, 0, 33], [31, 0, 2, 30, 33]],
                         ids=lambda l: "x".join(map(str, l)))
@pytest.mark.parametrize("H", [1, WIDE])
def test_gather_free_shard_edges_in_first_and_last_tiles(lens, H):
    sq, d = 300, 128
    S = sum(lens)
    qd = to_dev(gen_tensor(41, 0, sq, H, d, "bf16"), "bf16")
    kd = to_dev(gen_tensor(41, 1, S, H, d, "bf16"), "bf16")
    vd = to_dev(gen_tensor(41, 2, S, H, d, "bf16"), "bf16")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    ks = [kd[starts[r]:starts[r + 1]].clone() for r in range(len(lens))]
    vs = [vd[starts[r]:starts[r + 1]].clone() for r in range(len(lens))]
    lse_g = torch.empty(H, sq, device="cuda")
    lse_s = torch.empty_like(lse_g)
    og = sp.shard_attn_fwd(qd, kd, vd, lse=lse_g)
    os_ = sp.shard_attn_fwd_gv(qd, ks, vs, lse=lse_s)
    torch.cuda.synchronize()
    assert torch.equal(og.view(torch.int16), os_.view(torch.int16))
    assert torch.equal(lse_g, lse_s)


def test_one_key_range_is_the_plain_call_in_the_two_block_form():
    sq, skv, H, d = 300, 1000, WIDE, 128
    qd = to_dev(gen_tensor(42, 0, sq, H, d, "bf16"), "bf16")
    kd = to_dev(gen_tensor(42, 1, skv, H, d, "bf16"), "bf16")
    vd = to_dev(gen_tensor(42, 2, skv, H, d, "bf16"), "bf16")
    l1 = torch.empty(H, sq, device="cuda")
    l2 = torch.empty_like(l1)
    o1 = sp.shard_attn_fwd(qd, kd, vd, lse=l1)
    o2 = sp.shard_attn_fwd_split(qd, kd, vd, 1, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)

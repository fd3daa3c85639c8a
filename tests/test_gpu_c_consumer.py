"""GPU parity of one rank's share driven from plain C through the C ABI.

tests/c/abi_rank_share (built by the graft entry's build(), not here) runs
shard bounds, RoPE of every rank's K slice and of the rank's Q slice, the
AllGatherV pack and unpack of K and V and the attention, with hipMalloc'd
buffers and its own stream, and checks an overlapping-displacement call is
rejected.  Its output is compared with the float64 oracle at the bf16 bars
(2e-2 absolute and 1e-2 of max |O|; LSE within 2e-2).
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth import Workload, bf16_bits_to_f32, gen_qkv
from tests._helpers import attn_errors
from tests.c import build_consumer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,W,r", [(301, 4, 1), (1000, 3, 2), (64, 1, 0)])
def test_c_consumer_rank_share(tmp_path, S, W, r):
    exe = build_consumer.EXE
    assert os.path.exists(exe), "tests/c/abi_rank_share is built by the graft entry's build()"
    H, d = 2, 128
    wl = Workload("c_consumer", S=S, W=W, ranks=(r,), H=H, d=d, dtype="bf16", seed=S + W)
    q, k, v = gen_qkv(wl)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(np.array([S, W, r, H, d], dtype=np.int64).tobytes())
        for a in (q, k, v):
            f.write(np.ascontiguousarray(a).view(np.uint16).tobytes())
    dst = tmp_path / "out.bin"
    print(f"[c consumer] S={S} W={W} r={r}", flush=True)
    res = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    if W > 1:
        assert "error path: status -4" in res.stdout, res.stdout

    a, b = oracle.shard_bounds(S, W, r)
    sq = b - a
    raw = np.fromfile(dst, dtype=np.uint8)
    ob = sq * H * d * 2
    assert raw.size == ob + H * sq * 4
    o = bf16_bits_to_f32(raw[:ob].view(np.uint16).reshape(sq, H, d)).astype(np.float64)
    lse = raw[ob:].view(np.float32).reshape(H, sq).astype(np.float64)

    qf, kf, vf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    qr = oracle.rope_apply(qf[a:b], a)
    kr = oracle.rope_apply(kf, 0)  # every rank's slice at its absolute positions is the whole sequence's rotation
    ro, rl = oracle.attention(qr, kr, vf)
    err, rel = attn_errors(o, ro)
    assert err <= 2e-2 and rel <= 1e-2, (err, rel)
    assert np.max(np.abs(lse - rl)) <= 2e-2

"""GPU check of shard_attn_fwd_split_noalloc: the split-key attention with its
float32 partials in the library's device scratch instead of a caller workspace.

Called through the C ABI (ctypes, the library's exported symbol) and compared
with shard_attn_fwd_split on the same inputs: both run the same kernels on the
same partial layout, so outputs and LSEs must be bit-identical.  Two calls in a
row, the second on a smaller input (the scratch keeps the first call's
contents, which must not leak into the second), and the single-head VAE block
shape (4,096 queries x 16,384 keys x 512 channels, 4 ranges: 32 MiB of
partials) against the oracle's bars on sampled rows.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from sequence_dit_attention_amd import _lib
from synth import bf16_bits_to_f32, gen_tensor, sample_rows
from tests._helpers import attn_errors, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _inputs(seed, sq, skv, H, d):
    q = gen_tensor(seed, 0, sq, H, d, "bf16")
    k = gen_tensor(seed, 1, skv, H, d, "bf16")
    v = gen_tensor(seed, 2, skv, H, d, "bf16")
    return q, k, v, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")


def _noalloc(qd, kd, vd, nsplit, o, lse):
    """Direct C-ABI call of shard_attn_fwd_split_noalloc on torch's current stream."""
    sq, H, d = qd.shape
    rc = _lib.lib().shard_attn_fwd_split_noalloc(
        1, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), ctypes.c_void_p(lse.data_ptr()), sq,
        kd.shape[0], H, d, ctypes.c_float(1.0 / math.sqrt(d)), nsplit,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, _lib.lib().sp_last_error()


@pytest.mark.parametrize("first,second", [
    ((512, 300, 4000, 1, 6), (512, 129, 333, 1, 3)),      # VAE head size, ragged keys, fewer ranges
    ((128, 1000, 5000, 4, 8), (128, 257, 1000, 2, 3)),
    ((64, 700, 3000, 3, 5), (64, 100, 777, 1, 2)),
])
def test_noalloc_equals_workspace_call_twice(first, second):
    for i, (d, sq, skv, H, nsplit) in enumerate((first, second)):
        _, _, _, qd, kd, vd = _inputs(71 + 10 * i + d, sq, skv, H, d)
        o_ref = torch.empty_like(qd)
        l_ref = torch.empty(H, sq, device="cuda")
        ws = torch.full((sp.split_workspace_bytes(sq, H, d, nsplit),), 255, dtype=torch.uint8, device="cuda")
        sp.shard_attn_fwd_split(qd, kd, vd, nsplit, out=o_ref, lse=l_ref, workspace=ws)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((H, sq), float("nan"), device="cuda")
        _noalloc(qd, kd, vd, nsplit, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (i, d, sq, skv)
        assert torch.equal(lse, l_ref), (i, d, sq, skv)


def test_noalloc_vae_block_then_smaller_vs_oracle():
    """The 128 x 128 x 512 block of process 0 (32 MiB of partials), then a smaller call; sampled rows of
    both against the oracle (bf16 bars: 2e-2 absolute and 1e-2 of max|O|)."""
    widen = lambda a: bf16_bits_to_f32(a).astype(np.float64)
    for seed, sq, skv, nsplit in [(81, 4096, 16384, 4), (82, 700, 2048, 2)]:
        q, k, v, qd, kd, vd = _inputs(seed, sq, skv, 1, 512)
        o = torch.empty_like(qd)
        lse = torch.empty(1, sq, device="cuda")
        _noalloc(qd, kd, vd, nsplit, o, lse)
        torch.cuda.synchronize()
        rows = sample_rows(sq, 32, seed=seed)
        ro, rl = oracle.attention_rows(widen(q[rows]), k, v, widen=widen)
        err, rel = attn_errors(to_f64(o)[rows], ro)
        assert err <= 2e-2 and rel <= 1e-2, (seed, err, rel)
        assert np.max(np.abs(lse.cpu().numpy()[:, rows] - rl)) <= 2e-2


def test_noalloc_refuses_partials_beyond_the_scratch():
    _, _, _, qd, kd, vd = _inputs(83, 4096, 1024, 1, 512)
    with pytest.raises(sp.SpattnError) as ei:
        sp.shard_attn_fwd_split_noalloc(qd, kd, vd, 16)   # 4096 x 512 x 16 x 4 B = 128 MiB of partials
    assert ei.value.code == -3

"""GPU parity of the VAE block split: tile_pack / tile_unpack against the oracle, bit for bit.

NPU HunyuanImage-3.0模型推理优化实践, VAE并行优化: the input is cut along height
and width into one block per process and the results are gathered back into
place in two stages.  Copies are exact, so the bar is bit equality, on grids
with uneven blocks, empty blocks, one-row/one-column blocks and both dtypes.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from tests._helpers import to_dev, to_host_bits

pytestmark = pytest.mark.gpu

# the last three grids have more blocks than one copy launch takes (32), with empty blocks in between
GRIDS = [(7, 5, 3, 2, 3), (128, 128, 512, 2, 2), (84, 48, 512, 3, 3), (5, 3, 4, 7, 1), (9, 1, 2, 2, 4),
         (33, 65, 17, 4, 4), (1, 1, 8, 1, 1), (3, 2, 8, 3, 20), (2, 50, 3, 5, 10), (40, 40, 6, 6, 7)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hh,Ww,C,pr,pc", GRIDS)
def test_tile_pack_unpack_bitwise(dtype, Hh, Ww, C, pr, pc):
    rng = np.random.default_rng(Hh * 1000 + Ww)
    bits = rng.integers(0, 2**16, size=(Hh, Ww, C), dtype=np.uint16) if dtype == "bf16" else \
        rng.standard_normal((Hh, Ww, C)).astype(np.float32)
    raster = to_dev(bits, dtype)
    flat = sp.tile_pack(raster, pr, pc)
    back = sp.tile_unpack(flat, Hh, Ww, pr, pc)
    torch.cuda.synchronize()
    want = oracle.tile_pack(bits, pr, pc)
    assert to_host_bits(flat).tobytes() == np.ascontiguousarray(want).tobytes()
    assert to_host_bits(back).tobytes() == bits.tobytes()


def test_unpack_leaves_a_larger_flat_tail_alone_and_writes_every_raster_element():
    Hh, Ww, C, pr, pc = 10, 6, 4, 3, 2
    vals = np.arange(Hh * Ww * C, dtype=np.float32).reshape(Hh * Ww, C)
    flat = torch.full((Hh * Ww + 5, C), -1.0, device="cuda")
    flat[:Hh * Ww] = torch.from_numpy(vals).cuda()
    raster = torch.full((Hh, Ww, C), float("nan"), device="cuda")
    sp.tile_unpack(flat, Hh, Ww, pr, pc, raster)
    torch.cuda.synchronize()
    assert np.array_equal(raster.cpu().numpy(), oracle.tile_unpack(vals, Hh, Ww, pr, pc))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hh,Ww,C,pr,pc,n", [(7, 5, 3, 2, 3, 2), (128, 128, 512, 2, 2, 2), (84, 48, 512, 3, 3, 3),
                                            (3, 2, 8, 3, 20, 2), (40, 40, 6, 6, 7, 5), (9, 1, 2, 2, 4, 16)])
def test_tile_pack_n_bitwise_into_guarded_flats(dtype, Hh, Ww, C, pr, pc, n):
    """Several rasters in one batch of copies (the K and V gathers of the VAE split): each
    flat equals the oracle's block gather of its raster bit for bit, and the bytes
    around every flat (one buffer holding all of them with gaps) stay untouched.
    Grids with more than 32 segments in total span several launches."""
    rng = np.random.default_rng(Hh * 7 + Ww * 3 + n)
    rasters = []
    for _ in range(n):
        bits = rng.integers(0, 0x7F00, size=(Hh, Ww, C), dtype=np.uint16) if dtype == "bf16" else \
            rng.standard_normal((Hh, Ww, C)).astype(np.float32)
        rasters.append(bits)
    dev = [to_dev(b, dtype) for b in rasters]
    m = Hh * Ww * C
    gap = 256  # elements between flats (and before the first / after the last)
    tdt = dev[0].dtype
    sent = -7.0
    buf = torch.full((gap + n * (m + gap),), sent, dtype=tdt, device="cuda")
    flats = [buf[gap + a * (m + gap): gap + a * (m + gap) + m].view(Hh * Ww, C) for a in range(n)]
    sp.tile_pack_n(dev, pr, pc, flats)
    torch.cuda.synchronize()
    for a in range(n):
        want = oracle.tile_pack(rasters[a], pr, pc)
        assert to_host_bits(flats[a]).tobytes() == np.ascontiguousarray(want).tobytes(), a
    host = buf.float().cpu().numpy()
    for a in range(n + 1):
        g0 = a * (m + gap)
        assert np.all(host[g0:g0 + gap] == sent), a

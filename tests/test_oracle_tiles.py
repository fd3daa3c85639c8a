"""Pins of the oracle's 2-D spatial blocks of the VAE (CPU only).

NPU HunyuanImage-3.0模型推理优化实践, VAE并行优化: the image is cut along height
and width into one block per process; attention gathers all K and V; a
two-stage gather puts the blocks back in place.  Pinned by brute-force
assignment of every pixel to its block, by the block sizes, by the round trip,
and by the invariance of attention to the order in which the gathered keys
arrive (process order versus raster order).
"""
import numpy as np
import pytest

import oracle


def _owner_brute_force(n, parts, x):
    """The part whose floor range [n*i//parts, n*(i+1)//parts) holds x, by counting."""
    hits = [i for i in range(parts) if (n * i) // parts <= x < (n * (i + 1)) // parts]
    assert len(hits) == 1
    return hits[0]


@pytest.mark.parametrize("Hh,Ww,pr,pc", [(7, 5, 2, 3), (4, 4, 4, 4), (13, 1, 3, 1), (2, 9, 1, 4), (10, 10, 3, 3)])
def test_every_pixel_in_exactly_one_block(Hh, Ww, pr, pc):
    owner = -np.ones((Hh, Ww), dtype=int)
    for p in range(pr * pc):
        r0, r1, c0, c1 = oracle.tile_bounds(Hh, Ww, pr, pc, p)
        assert np.all(owner[r0:r1, c0:c1] == -1)
        owner[r0:r1, c0:c1] = p
    assert np.all(owner >= 0)
    for r in range(Hh):
        for c in range(Ww):
            assert owner[r, c] == _owner_brute_force(Hh, pr, r) * pc + _owner_brute_force(Ww, pc, c)


def test_block_sizes_are_floor_or_ceil():
    for Hh in range(0, 40):
        for pr in range(1, 7):
            hs = [oracle.tile_bounds(Hh, 3, pr, 1, p)[1] - oracle.tile_bounds(Hh, 3, pr, 1, p)[0] for p in range(pr)]
            assert sum(hs) == Hh and set(hs) <= {Hh // pr, -(-Hh // pr)}


def test_pack_order_and_round_trip():
    Hh, Ww, C, pr, pc = 5, 7, 3, 2, 3
    raster = np.arange(Hh * Ww * C).reshape(Hh, Ww, C)
    flat = oracle.tile_pack(raster, pr, pc)
    # explicit element loop: block after block in process order, rows then columns inside a block
    k = 0
    for p in range(pr * pc):
        r0, r1, c0, c1 = oracle.tile_bounds(Hh, Ww, pr, pc, p)
        for r in range(r0, r1):
            for c in range(c0, c1):
                assert flat[k].tolist() == raster[r, c].tolist()
                k += 1
    assert k == Hh * Ww
    assert np.array_equal(oracle.tile_unpack(flat, Hh, Ww, pr, pc), raster)
    with pytest.raises(ValueError):
        oracle.tile_unpack(flat[:-1], Hh, Ww, pr, pc)


def test_attention_does_not_depend_on_the_gather_order():
    """Keys gathered block by block (process order) give the attention of the raster order."""
    rng = np.random.default_rng(4)
    Hh, Ww, C, pr, pc = 6, 5, 16, 2, 2
    q, k, v = (rng.standard_normal((Hh, Ww, C)) for _ in range(3))
    kf, vf = oracle.tile_pack(k, pr, pc), oracle.tile_pack(v, pr, pc)
    r0, r1, c0, c1 = oracle.tile_bounds(Hh, Ww, pr, pc, 3)
    qt = q[r0:r1, c0:c1].reshape(-1, 1, C)
    o1, l1 = oracle.attention(qt, kf.reshape(-1, 1, C), vf.reshape(-1, 1, C))
    o2, l2 = oracle.attention(qt, k.reshape(-1, 1, C), v.reshape(-1, 1, C))
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)

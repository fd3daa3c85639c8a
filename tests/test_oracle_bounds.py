"""Pins of the oracle's shard arithmetic and AllGatherV layout (CPU only).

Split rule: MiniMax-H3-Comfy-NPU, section 机制一 (rank r owns
[S*r//W, S*(r+1)//W)); counts/displacements: same page, 后端 A.
"""
import json
import os

import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _count_multiples(n, W):
    # floor(n / W) written as a count: how many t in 1..n are multiples of W
    return sum(1 for t in range(1, n + 1) if t % W == 0)


def test_bounds_brute_force_small():
    for S in range(0, 90):
        for W in range(1, 9):
            for r in range(W):
                a, b = oracle.shard_bounds(S, W, r)
                assert a == _count_multiples(S * r, W)
                assert b == _count_multiples(S * (r + 1), W)


def test_bounds_tile_exhaustive():
    for S in range(0, 2001):
        for W in range(1, 17):
            bs = oracle.all_shard_bounds(S, W)
            assert bs[0][0] == 0 and bs[-1][1] == S
            for r in range(W - 1):
                assert bs[r][1] == bs[r + 1][0]
            lens = [b - a for a, b in bs]
            assert set(lens) <= {S // W, -(-S // W)}
            assert sum(lens) == S


def test_bounds_golden():
    with open(os.path.join(GOLD, "shard_lengths.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        S, W = c["S"], c["W"]
        if "lengths" in c:
            assert [b - a for a, b in oracle.all_shard_bounds(S, W)] == c["lengths"]
        else:
            a, b = oracle.shard_bounds(S, W, c["rank"])
            if "start" in c:
                assert (a, b) == (c["start"], c["end"])
            assert b - a == c.get("length", b - a)


def test_bounds_large_no_overflow():
    S = 2**62 + 12345
    a, b = oracle.shard_bounds(S, 7, 6)
    assert b == S and a == (S * 6) // 7


@pytest.mark.parametrize("args", [(-1, 4, 0), (10, 0, 0), (10, 4, 4), (10, 4, -1)])
def test_bounds_invalid(args):
    with pytest.raises(ValueError):
        oracle.shard_bounds(*args)


def test_layout():
    for S, W, outer, inner in [(16383, 4, 1, 2048), (7, 4, 3, 5), (3, 8, 2, 1), (0, 3, 1, 4)]:
        counts, displs = oracle.allgatherv_layout(S, W, outer, inner)
        lens = [b - a for a, b in oracle.all_shard_bounds(S, W)]
        assert counts == [outer * s * inner for s in lens]
        assert displs[0] == 0
        for r in range(1, W):
            assert displs[r] == displs[r - 1] + counts[r - 1]
        assert sum(counts) == outer * S * inner


def test_layout_lens_matches_numpy_concatenation():
    """counts/displs of arbitrary per-rank lengths are where numpy's own
    concatenation of the flattened rank tensors puts each rank's elements."""
    import numpy as np

    for lens, outer, inner in [([3, 0, 5, 1], 2, 4), ([4095, 4096, 4096, 4096], 1, 16 * 128), ([0], 3, 2),
                               ([2, 7], 1, 1), ([1, 1, 1], 5, 0), ([6, 2, 9], 0, 3)]:
        counts, displs = oracle.allgatherv_layout_lens(lens, outer, inner)
        tensors = [np.arange(outer * s * inner, dtype=np.int64).reshape(outer, s, inner) + 10**9 * (r + 1)
                   for r, s in enumerate(lens)]
        flat = np.concatenate([t.ravel() for t in tensors]) if tensors else np.zeros(0)
        assert flat.size == sum(counts)
        for r, t in enumerate(tensors):
            assert counts[r] == t.size
            assert np.array_equal(flat[displs[r]:displs[r] + counts[r]], t.ravel())


def test_layout_lens_concat_on_a_middle_axis():
    """exchange(rank, tensors, cat_dims) on axis 1 of [2, s_r, 3, 4] tensors:
    pack by the layout, unpack with outer = 2, inner = 12, and the result is
    numpy's concatenation along that axis."""
    import numpy as np

    rng = np.random.default_rng(11)
    lens = [2, 5, 0, 3]
    tensors = [rng.integers(0, 1000, size=(2, s, 3, 4)) for s in lens]
    counts, displs = oracle.allgatherv_layout_lens(lens, 2, 12)
    assert sum(counts) == sum(t.size for t in tensors)
    flat = oracle.varlen_pack([t.ravel() for t in tensors], counts, displs, np.zeros(sum(counts), np.int64))
    out = oracle.varlen_unpack(flat, displs, lens, 2, 12).reshape(2, sum(lens), 3, 4)
    assert np.array_equal(out, np.concatenate(tensors, axis=1))


def test_layout_lens_equals_split_layout():
    for S, W, outer, inner in [(16383, 4, 1, 2048), (7, 4, 3, 5), (3, 8, 2, 1)]:
        lens = [b - a for a, b in oracle.all_shard_bounds(S, W)]
        assert oracle.allgatherv_layout_lens(lens, outer, inner) == oracle.allgatherv_layout(S, W, outer, inner)


@pytest.mark.parametrize("args", [([], 1, 1), ([1, -1], 1, 1), ([1], -1, 1), ([1], 1, -2)])
def test_layout_lens_invalid(args):
    with pytest.raises(ValueError):
        oracle.allgatherv_layout_lens(*args)

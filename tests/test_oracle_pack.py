"""Pins of the oracle's AllGatherV pack/unpack (CPU only).

MiniMax-H3-Comfy-NPU, section 后端 A: per-rank counts (elements) and
displacements (target offsets) into a flat receive buffer, then narrow, view
to each rank's shape and concatenate.  Checked against explicit per-element
index loops, not against numpy slicing.
"""
import numpy as np

import oracle


def _rand(rng, n, dtype):
    if dtype == np.uint16:
        return rng.integers(0, 65536, size=n, dtype=np.uint16)
    return rng.standard_normal(n).astype(dtype)


def test_pack_brute_force_with_gaps_and_sentinels():
    rng = np.random.default_rng(0)
    for dtype in (np.uint16, np.float32):
        counts = [5, 0, 7, 3]
        displs = [20, 2, 0, 9]            # not prefix order, gaps at 7..8, 12..19
        flat0 = np.full(30, 77, dtype=dtype)
        sends = [_rand(rng, c, dtype) for c in counts]
        got = oracle.varlen_pack(sends, counts, displs, flat0)
        want = [flat0[i] for i in range(30)]
        for r in range(4):
            for i in range(counts[r]):
                want[displs[r] + i] = sends[r][i]
        assert got.dtype == dtype
        assert got.tobytes() == np.array(want, dtype=dtype).tobytes()
        assert flat0[0] == 77  # input untouched


def test_unpack_index_formula():
    rng = np.random.default_rng(1)
    outer, inner = 3, 4
    seq = [2, 0, 3, 1]
    counts = [outer * s * inner for s in seq]
    displs = [40, 0, 2, 100]
    flat = rng.standard_normal(200)
    got = oracle.varlen_unpack(flat, displs, seq, outer, inner)
    S = sum(seq)
    assert got.shape == (outer, S, inner)
    a = 0
    for r, s in enumerate(seq):
        for o in range(outer):
            for t in range(s):
                for k in range(inner):
                    assert got[o, a + t, k] == flat[displs[r] + (o * s + t) * inner + k]
        a += s
    assert counts[2] == 36


def test_round_trip_and_identity():
    rng = np.random.default_rng(2)
    for S, W, outer, inner in [(11, 4, 1, 6), (11, 4, 2, 3), (3, 5, 1, 2), (9, 1, 2, 2)]:
        x = rng.standard_normal((outer, S, inner))
        bounds = oracle.all_shard_bounds(S, W)
        shards = [x[:, a:b, :] for a, b in bounds]
        counts, displs = oracle.allgatherv_layout(S, W, outer, inner)
        flat = oracle.varlen_pack([s.ravel() for s in shards], counts, displs,
                                  np.zeros(sum(counts)))
        back = oracle.varlen_unpack(flat, displs, [b - a for a, b in bounds], outer, inner)
        assert np.array_equal(back, x)
        if W == 1 and outer == 1:
            assert np.array_equal(flat, x.ravel())


def test_output_concat():
    parts = [np.arange(6).reshape(2, 3), np.arange(3).reshape(1, 3) + 10]
    got = oracle.output_concat(parts)
    assert got.tolist() == [[0, 1, 2], [3, 4, 5], [10, 11, 12]]

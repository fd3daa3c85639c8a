"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in an oracle function (a wrong rounding, an index
off by one, a transposed index, a dropped factor, a flipped sign, a swapped
pairing, a wrong scale or softmax axis, a LayerNorm in place of RMSNorm, rows
and columns of the block grid swapped) and runs the pin tests of that
function against the planted version: at least one of them must fail.  The
same pins pass on the real oracle (they run as ordinary tests).
"""
import math

import numpy as np
import pytest

import oracle
from tests import test_oracle_attn as ta
from tests import test_oracle_bounds as tb
from tests import test_oracle_pack as tp
from tests import test_oracle_qk_norm as tq
from tests import test_oracle_rope as tr
from tests import test_oracle_rope_mx as tm
from tests import test_oracle_tiles as tt

_real = {name: getattr(oracle, name) for name in dir(oracle) if not name.startswith("_")}


def _caught(monkeypatch, patches, pins):
    """True when at least one pin fails with the planted functions in place."""
    with monkeypatch.context() as m:
        for name, fn in patches.items():
            m.setattr(oracle, name, fn)
        for pin in pins:
            try:
                pin()
            except AssertionError:
                return True
    return False


# ---- planted mistakes -------------------------------------------------------

def _bounds_ceil(S, W, r):  # ceiling instead of floor division
    return -(-S * r // W), -(-S * (r + 1) // W)


def _bounds_fixed_len(S, W, r):  # every shard S // W long: the remainder is lost
    a = S * r // W
    return a, a + S // W


def _all_bounds_of(fn):
    return lambda S, W: [fn(S, W, r) for r in range(W)]


def _pack_off_by_one(sends, counts, displs, flat):
    out = flat.copy()
    for r, s in enumerate(sends):
        c = int(counts[r])
        if c:
            out[displs[r] + 1:displs[r] + 1 + c] = np.asarray(s).reshape(-1)[:c][: len(out) - displs[r] - 1]
    return out


def _unpack_transposed(flat, displs, seq_lens, outer, inner):  # rank block read as [s_r, outer, inner]
    parts = []
    for r, s in enumerate(seq_lens):
        blk = flat[displs[r]:displs[r] + outer * s * inner].reshape(s, outer, inner).transpose(1, 0, 2)
        parts.append(blk)
    return np.concatenate(parts, axis=1)


def _rope_half_freq(x, pos0, theta=10000.0, style="half"):  # theta^(-j/d): the factor 2 dropped
    return _real["rope_apply"](x, pos0, math.sqrt(theta), style)


def _rope_sign(x, pos0, theta=10000.0, style="half"):  # rotation the other way
    s = x.shape[0]
    out = np.empty_like(np.asarray(x, dtype=np.float64))
    for t in range(s):  # the angle of a token is linear in its position: rotate by -(pos0 + t)
        out[t:t + 1] = _real["rope_apply"](x[t:t + 1], -(pos0 + t), theta, style)
    return out


def _rope_pairing_swapped(x, pos0, theta=10000.0, style="half"):
    return _real["rope_apply"](x, pos0, theta, "interleaved" if style == "half" else "half")


def _rope_mx_axes_reversed(x, pos, sections, theta=10000.0, style="half"):
    return _real["rope_apply_mx"](x, np.asarray(pos)[:, ::-1], tuple(sections)[::-1], theta, style)


def _attn_scale_1_over_d(q, k, v, scale=None, **kw):
    d = q.shape[-1]
    return _real["attention"](q, k, v, scale=1.0 / d)


def _attn_softmax_over_queries(q, k, v, scale=None, **kw):
    sq, H, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o = np.empty((sq, H, v.shape[-1]))
    lse = np.empty((H, sq))
    for h in range(H):
        L = sc * (q[:, h, :] @ k[:, h, :].T)
        P = np.exp(L - L.max(axis=0, keepdims=True))
        P /= P.sum(axis=0, keepdims=True)
        o[:, h, :] = P @ v[:, h, :]
        lse[h] = np.log(np.exp(L).sum(axis=1))
    return o, lse


def _layer_norm(x, gamma, eps):  # mean subtracted: LayerNorm, not RMSNorm
    xc = x - x.mean(axis=-1, keepdims=True)
    return xc / np.sqrt(np.mean(xc * xc, axis=-1, keepdims=True) + eps) * gamma


def _rms_eps_outside(x, gamma, eps):
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * gamma


def _layout_lens_inclusive(seq_lens, outer=1, inner=1):  # displacement counts the rank's own block
    counts = [int(outer) * int(n) * int(inner) for n in seq_lens]
    return counts, [sum(counts[:r + 1]) for r in range(len(counts))]


def _layout_lens_no_outer(seq_lens, outer=1, inner=1):  # outer dropped from the counts
    counts = [int(n) * int(inner) for n in seq_lens]
    return counts, [sum(counts[:r]) for r in range(len(counts))]


def _tiles_transposed(Hh, Ww, pr, pc, p):  # process p read column-major over the block grid
    i, j = p % pr, p // pr
    return (Hh * i) // pr, (Hh * (i + 1)) // pr, (Ww * j) // pc, (Ww * (j + 1)) // pc


# ---- cases ------------------------------------------------------------------

BOUNDS_PINS = [tb.test_bounds_brute_force_small, tb.test_bounds_tile_exhaustive, tb.test_bounds_golden]
ROPE_PINS = [tr.test_golden_d2, lambda: tr.test_complex_multiplication("half"),
             lambda: tr.test_complex_multiplication("interleaved")]
ATTN_PINS = [ta.test_brute_force_tiny, ta.test_torch_sdpa_float64, ta.test_closed_forms]

CASES = {
    "bounds: ceiling division": ({"shard_bounds": _bounds_ceil, "all_shard_bounds": _all_bounds_of(_bounds_ceil)},
                                 BOUNDS_PINS),
    "bounds: remainder dropped": ({"shard_bounds": _bounds_fixed_len,
                                   "all_shard_bounds": _all_bounds_of(_bounds_fixed_len)}, BOUNDS_PINS),
    "pack: displacement off by one": ({"varlen_pack": _pack_off_by_one}, [tp.test_pack_brute_force_with_gaps_and_sentinels]),
    "unpack: outer and sequence indices transposed": ({"varlen_unpack": _unpack_transposed},
                                                      [tp.test_unpack_index_formula]),
    "rope: factor 2 of the frequency exponent dropped": ({"rope_apply": _rope_half_freq}, ROPE_PINS),
    "rope: sine sign flipped": ({"rope_apply": _rope_sign}, ROPE_PINS),
    "rope: pairing swapped": ({"rope_apply": _rope_pairing_swapped}, ROPE_PINS),
    "rope_mx: axes reversed": ({"rope_apply_mx": _rope_mx_axes_reversed},
                               [lambda: tm.test_complex_multiplication_per_axis("half")]),
    "attention: scale 1/d": ({"attention": _attn_scale_1_over_d}, ATTN_PINS),
    "attention: softmax over the queries": ({"attention": _attn_softmax_over_queries}, ATTN_PINS),
    "rms_norm: mean subtracted": ({"rms_norm": _layer_norm}, [tq.test_rms_norm_by_loops]),
    "rms_norm: eps outside the root": ({"rms_norm": _rms_eps_outside}, [tq.test_rms_norm_by_loops]),
    "layout: displacements include the rank's own block": ({"allgatherv_layout_lens": _layout_lens_inclusive},
                                                           [tb.test_layout_lens_matches_numpy_concatenation]),
    "layout: outer dropped from the counts": ({"allgatherv_layout_lens": _layout_lens_no_outer},
                                              [tb.test_layout_lens_concat_on_a_middle_axis]),
    "tiles: block grid read column-major": ({"tile_bounds": _tiles_transposed},
                                            [lambda: tt.test_every_pixel_in_exactly_one_block(7, 5, 2, 3)]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_mistake_is_caught(monkeypatch, case):
    patches, pins = CASES[case]
    assert _caught(monkeypatch, patches, pins), f"no pin fails for: {case}"

"""Every device output written into a sentinel-filled buffer with guard bands.

Each kernel's output view sits between two guard bands of a larger buffer
filled with a sentinel bit pattern; after the call the guards must hold the
sentinel bit for bit, and the output must equal (bitwise) the same call on a
plain buffer, which the parity tests check against the oracle.  Shapes are
ragged, so the masked epilogues and the lanes and slots that read past their
work are exercised: attention rows past sq in the last query tile, RoPE /
QK-norm head sizes 12 and 120 (lanes past d/2 per lane group) and head counts
that are not a multiple of the slots per wave, a VAE block grid with unequal
blocks.  Guards are multiples of 256 bytes, so every output keeps the
alignment of the plain call.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_dit_attention_amd as sp
from synth import gen_gamma, gen_tensor
from tests._helpers import attn_errors, to_dev, to_f64, to_host_bits

pytestmark = pytest.mark.gpu

GUARD_BYTES = 512
SENT_BF16 = 0x7FA5          # a NaN pattern no kernel writes
SENT_F32_BITS = 0x7FC0DEAD  # likewise


def _guarded(shape, dtype):
    """(whole buffer, output view) with GUARD_BYTES of sentinel before and after the view."""
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        g = GUARD_BYTES // 2
        buf = torch.full((n + 2 * g,), SENT_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        g = GUARD_BYTES // 4
        buf = torch.full((n + 2 * g,), SENT_F32_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    return buf, buf[g:g + n].view(*shape), g


def _guards_intact(buf, g):
    bits = buf.view(torch.int16 if buf.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    sent = SENT_BF16 if buf.dtype == torch.bfloat16 else np.int32(SENT_F32_BITS)
    return bool(np.all(bits[:g] == sent) and np.all(bits[-g:] == sent))


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _qkv(seed, sq, skv, H, d, dtype):
    q = gen_tensor(seed, 0, sq, H, d, dtype)
    k = gen_tensor(seed, 1, skv, H, d, dtype)
    v = gen_tensor(seed, 2, skv, H, d, dtype)
    return q, k, v, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)


@pytest.mark.parametrize("dtype,d,sq,skv,H", [("bf16", 128, 300, 1000, 3), ("bf16", 64, 257, 777, 2),
                                              ("bf16", 512, 129, 300, 1), ("f32", 64, 250, 1001, 2),
                                              ("f32", 128, 65, 130, 3)])
def test_attention_output_and_lse_guards(dtype, d, sq, skv, H):
    q, k, v, qd, kd, vd = _qkv(91 + d, sq, skv, H, d, dtype)
    tdt = qd.dtype
    obuf, o, go = _guarded((sq, H, d), tdt)
    lbuf, lse, gl = _guarded((H, sq), torch.float32)
    sp.shard_attn_fwd(qd, kd, vd, out=o, lse=lse)
    o_plain = torch.empty_like(qd)
    l_plain = torch.empty(H, sq, device="cuda")
    sp.shard_attn_fwd(qd, kd, vd, out=o_plain, lse=l_plain)
    torch.cuda.synchronize()
    assert _guards_intact(obuf, go) and _guards_intact(lbuf, gl)
    assert _same(o, o_plain) and _same(lse, l_plain)
    ro, _ = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    err, rel = attn_errors(to_f64(o), ro)
    assert err <= (1e-4 if dtype == "f32" else 2e-2) and (dtype == "f32" or rel <= 1e-2), (err, rel)


@pytest.mark.parametrize("dtype,d,lens", [("bf16", 128, [250, 250, 250, 251]), ("bf16", 64, [97, 0, 200, 63]),
                                          ("f32", 64, [97, 0, 200, 63]), ("f32", 64, [3, 0, 29, 0])])
def test_gather_free_guards_and_f32_head_size_64(dtype, d, lens):
    """shard_attn_fwd_gv into guarded O / LSE: bitwise the gathered call (float32 at head size 64 too)."""
    sq, H = 129, 2
    S = sum(lens)
    q, k, v, qd, kd, vd = _qkv(92 + d, sq, S, H, d, dtype)
    st = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    ks = [kd[st[r]:st[r + 1]].clone() for r in range(len(lens))]
    vs = [vd[st[r]:st[r + 1]].clone() for r in range(len(lens))]
    obuf, o, go = _guarded((sq, H, d), qd.dtype)
    lbuf, lse, gl = _guarded((H, sq), torch.float32)
    sp.shard_attn_fwd_gv(qd, ks, vs, out=o, lse=lse)
    l_g = torch.empty(H, sq, device="cuda")
    og = sp.shard_attn_fwd(qd, kd, vd, lse=l_g)
    torch.cuda.synchronize()
    assert _guards_intact(obuf, go) and _guards_intact(lbuf, gl)
    assert _same(o, og) and _same(lse, l_g)
    ro, _ = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    err, rel = attn_errors(to_f64(o), ro)
    assert err <= (1e-4 if dtype == "f32" else 2e-2) and (dtype == "f32" or rel <= 1e-2), (err, rel)


@pytest.mark.parametrize("d,sq,skv,H,nsplit", [(512, 129, 300, 1, 3), (128, 257, 1000, 2, 5), (64, 100, 777, 3, 7)])
def test_split_output_lse_and_workspace_guards(d, sq, skv, H, nsplit):
    """Split attention: guarded O and LSE (written by the merge) and guard bands on both sides of the
    workspace (written by the attention kernel's partials)."""
    _, _, _, qd, kd, vd = _qkv(93 + d, sq, skv, H, d, "bf16")
    need = sp.split_workspace_bytes(sq, H, d, nsplit)
    wbuf = torch.full((need + 2 * GUARD_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = wbuf[GUARD_BYTES:GUARD_BYTES + need]
    obuf, o, go = _guarded((sq, H, d), torch.bfloat16)
    lbuf, lse, gl = _guarded((H, sq), torch.float32)
    sp.shard_attn_fwd_split(qd, kd, vd, nsplit, out=o, lse=lse, workspace=ws)
    l_p = torch.empty(H, sq, device="cuda")
    o_p = sp.shard_attn_fwd_split(qd, kd, vd, nsplit, lse=l_p)
    torch.cuda.synchronize()
    assert _guards_intact(obuf, go) and _guards_intact(lbuf, gl)
    w = wbuf.cpu().numpy()
    assert np.all(w[:GUARD_BYTES] == 0xA5) and np.all(w[-GUARD_BYTES:] == 0xA5)
    assert _same(o, o_p) and _same(lse, l_p)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("s,H,d", [(17, 5, 12), (40, 5, 120), (33, 7, 128), (9, 3, 2)])
def test_rope_and_qk_norm_guards(dtype, s, H, d):
    """RoPE (1-D and multi-axis) and QK-norm + RoPE written out of place into guarded buffers: head
    sizes whose rows leave lanes idle and head counts that are not a multiple of a wave's slots."""
    x = gen_tensor(94 + d, 0, s, H, d, dtype)
    xd = to_dev(x, dtype)
    g = torch.from_numpy(gen_gamma(95, d)).cuda()
    pos = torch.from_numpy(np.random.default_rng(d).integers(0, 50000, size=(s, 3)).astype(np.int64)).cuda()
    sec = (d // 2 - 2 * (d // 6), d // 6, d // 6)
    calls = [lambda out: sp.rope_apply(xd, 91821, out=out),
             lambda out: sp.rope_apply(xd, 7, style="interleaved", out=out),
             lambda out: sp.rope_apply_mx(xd, pos, sec, out=out),
             lambda out: sp.qk_norm_rope(xd, g, 1e-6, 91821, out=out),
             lambda out: sp.qk_norm_rope(xd, g, 1e-6, pos=pos, sections=sec, style="interleaved", out=out)]
    for call in calls:
        buf, y, gy = _guarded((s, H, d), xd.dtype)
        call(y)
        y_plain = call(torch.empty_like(xd))
        torch.cuda.synchronize()
        assert _guards_intact(buf, gy)
        assert _same(y, y_plain)
    assert to_host_bits(xd).tobytes() == x.tobytes()


@pytest.mark.parametrize("Hh,Ww,C,pr,pc", [(7, 5, 8, 2, 3), (128, 128, 512, 2, 2), (30, 53, 16, 3, 4)])
def test_tile_unpack_and_pack_guards(Hh, Ww, C, pr, pc):
    """VAE block gather and placement into guarded buffers, bit-exact against the oracle."""
    rng = np.random.default_rng(Hh * Ww)
    r = rng.integers(0, 0x7F00, size=(Hh, Ww, C), dtype=np.uint16)
    rd = to_dev(r, "bf16")
    fbuf, flat, gf = _guarded((Hh * Ww, C), torch.bfloat16)
    sp.tile_pack(rd, pr, pc, flat)
    rbuf, back, gr = _guarded((Hh, Ww, C), torch.bfloat16)
    sp.tile_unpack(flat, Hh, Ww, pr, pc, back)
    torch.cuda.synchronize()
    assert _guards_intact(fbuf, gf) and _guards_intact(rbuf, gr)
    assert to_host_bits(flat).tobytes() == oracle.tile_pack(r, pr, pc).tobytes()
    assert to_host_bits(back).tobytes() == r.tobytes()

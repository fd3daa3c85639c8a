"""Float64 / integer oracle of one rank's share of sequence-parallel DiT attention.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): used by tests, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.

Sources (page title, then section):
  [MH3] "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU 中 DiT 序列并行与
        peer-copy 双后端机制" (m.nxbn.cn/news/97331)
        - section "机制一 DiT 序列并行": rank r owns the token range
          [seq_len*r // world_size, seq_len*(r+1) // world_size) of the packed
          sequence h; the RoPE frequency table is sliced with it; attention
          takes Q from the local shard and K/V over the full sequence; after the
          last block the per-rank outputs are joined back along the sequence.
        - section "机制二 ... 后端 A: HCCL AllGatherV": every rank contributes
          `counts` elements placed at `displacements` (element offsets) of a
          one-dimensional receive buffer; each rank's block is then narrowed,
          viewed back to that rank's shape and concatenated.
  [HY3] "NPU HunyuanImage-3.0模型推理优化实践" (cf-1.com/news/2296994)
        - section "消除旋转位置编码冗余cast算子": rotary embedding is applied to
          the query and key states only, with cos/sin tables
          (apply_rotary_pos_emb(query_states, key_states, cos, sin)).
        - section "消除FA中scale的冗余计算": the attention scale is 1/sqrt(d),
          computed once.
        - section "VAE并行优化": a large image is cut along height and width
          into blocks, one per process; attention inside the VAE gathers the
          K and V of all blocks; at the end a two-stage gather puts every
          block's result back at its spatial position in the full tensor.

Readings where the pages are silent are listed in the design notes of the
repository; the ones that shape the arithmetic here are: integer division is
floor on non-negative Python ints; RoPE is the usual rotary form with
frequencies theta**(-2j/d) at the token's absolute packed index, pairing
(j, j + d/2) ("half" style, the rotate_half convention) or (2j, 2j+1)
("interleaved"); attention is unmasked (bidirectional) softmax attention.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Shard arithmetic  [MH3, 机制一]
# ---------------------------------------------------------------------------


def shard_bounds(S: int, W: int, r: int) -> tuple[int, int]:
    """Token range [a, b) of rank r when S packed tokens are split over W ranks.

    [MH3, 机制一]: a = S*r // W, b = S*(r+1) // W (the '+' of r+1 is lost in
    the page text).  Exact Python integers, no overflow.
    """
    S, W, r = int(S), int(W), int(r)
    if W < 1 or not (0 <= r < W) or S < 0:
        raise ValueError("need W >= 1, 0 <= r < W, S >= 0")
    return (S * r) // W, (S * (r + 1)) // W


def all_shard_bounds(S: int, W: int) -> list[tuple[int, int]]:
    """[shard_bounds(S, W, r) for every rank r]."""
    return [shard_bounds(S, W, r) for r in range(W)]


def allgatherv_layout(S: int, W: int, outer: int = 1, inner: int = 1):
    """AllGatherV counts and displacements, in elements  [MH3, 后端 A].

    Rank r sends its local tensor of shape [outer, s_r, inner] flattened, so
    counts[r] = outer * s_r * inner; the receive buffer holds the ranks' blocks
    back to back in rank order, so displs[r] = counts[0] + ... + counts[r-1].
    """
    counts = []
    for r in range(W):
        a, b = shard_bounds(S, W, r)
        counts.append(int(outer) * (b - a) * int(inner))
    displs = []
    off = 0
    for c in counts:
        displs.append(off)
        off += c
    return counts, displs


def allgatherv_layout_lens(seq_lens, outer: int = 1, inner: int = 1):
    """AllGatherV counts and displacements for arbitrary per-rank lengths  [MH3, 后端 A].

    exchange(rank, tensors, cat_dims) gathers tensors that agree outside the
    concatenation axis; rank r's tensor is viewed as [outer, seq_lens[r], inner]
    (outer = product of the sizes before cat_dim, inner = product after it).
    Its block in the flat receive buffer holds every one of its elements:
    counts[r] = outer * seq_lens[r] * inner, the blocks back to back in rank
    order: displs[r] = counts[0] + ... + counts[r-1].  Written as element
    counting loops over Python ints.
    """
    outer, inner = int(outer), int(inner)
    if outer < 0 or inner < 0 or any(int(s) < 0 for s in seq_lens) or len(seq_lens) < 1:
        raise ValueError("need at least one rank and non-negative sizes")
    counts, displs = [], []
    next_free = 0
    for s in seq_lens:
        n = 0
        for _o in range(outer):
            for _t in range(int(s)):
                n += inner
        counts.append(n)
        displs.append(next_free)
        next_free += n
    return counts, displs


# ---------------------------------------------------------------------------
# AllGatherV data movement  [MH3, 后端 A]
# ---------------------------------------------------------------------------


def varlen_pack(sends, counts, displs, flat: np.ndarray) -> np.ndarray:
    """Gather step of AllGatherV: flat[displs[r] + i] = sends[r].ravel()[i].

    Returns a copy of `flat` with every rank's block written; elements that no
    block covers keep their previous value.  Bits are copied unchanged.
    """
    out = np.array(flat, copy=True)
    for r, src in enumerate(sends):
        c, dsp = int(counts[r]), int(displs[r])
        src = np.asarray(src).reshape(-1)
        if src.size < c:
            raise ValueError("send buffer shorter than its count")
        if dsp < 0 or dsp + c > out.size:
            raise ValueError("block outside the receive buffer")
        out[dsp:dsp + c] = src[:c]
    return out


def varlen_unpack(flat: np.ndarray, displs, seq_lens, outer: int, inner: int) -> np.ndarray:
    """narrow -> view -> concat of an AllGatherV receive buffer  [MH3, 后端 A].

    Rank r's block flat[displs[r] : displs[r] + outer*s_r*inner] is viewed as
    [outer, s_r, inner]; the views are concatenated along the sequence axis,
    giving [outer, sum(s_r), inner].
    """
    parts = []
    for r, s in enumerate(seq_lens):
        n = int(outer) * int(s) * int(inner)
        dsp = int(displs[r])
        parts.append(np.asarray(flat)[dsp:dsp + n].reshape(int(outer), int(s), int(inner)))
    return np.concatenate(parts, axis=1)


def output_concat(outs) -> np.ndarray:
    """Final merge of the per-rank outputs along the sequence  [MH3, 机制一]."""
    return np.concatenate([np.asarray(o) for o in outs], axis=0)


# ---------------------------------------------------------------------------
# Rotary position embedding on the local slice  [MH3, 机制一; HY3]
# ---------------------------------------------------------------------------


def rope_inv_freq(d: int, theta: float = 10000.0) -> np.ndarray:
    """Frequencies theta**(-2j/d), j = 0 .. d/2-1, in float64."""
    j = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / np.float64(d))


def rope_apply(x: np.ndarray, pos0: int, theta: float = 10000.0, style: str = "half") -> np.ndarray:
    """Rotate each pair of x [s, H, d] by angle p * theta**(-2j/d), p = pos0 + token.

    The rank's slice of the frequency table starts at its first absolute
    position pos0 [MH3, 机制一].  For pair j with components (x1, x2) the result
    is (x1 cos - x2 sin, x2 cos + x1 sin) (rotate_half form [HY3]).  Pairs are
    (j, j + d/2) for style "half" and (2j, 2j+1) for "interleaved".
    Float64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    s, H, d = x.shape
    if d % 2:
        raise ValueError("d must be even")
    pos = np.float64(pos0) + np.arange(s, dtype=np.float64)
    ang = pos[:, None] * rope_inv_freq(d, theta)[None, :]          # [s, d/2]
    cos = np.cos(ang)[:, None, :]                                   # [s, 1, d/2]
    sin = np.sin(ang)[:, None, :]
    if style == "half":
        x1, x2 = x[..., : d // 2], x[..., d // 2:]
    elif style == "interleaved":
        x1, x2 = x[..., 0::2], x[..., 1::2]
    else:
        raise ValueError("style must be 'half' or 'interleaved'")
    y1 = x1 * cos - x2 * sin
    y2 = x2 * cos + x1 * sin
    y = np.empty_like(x)
    if style == "half":
        y[..., : d // 2], y[..., d // 2:] = y1, y2
    else:
        y[..., 0::2], y[..., 1::2] = y1, y2
    return y


def rope_apply_mx(x: np.ndarray, pos: np.ndarray, sections, theta: float = 10000.0,
                  style: str = "half") -> np.ndarray:
    """Multi-axis rotary embedding of x [s, H, d] with explicit positions.

    The pages slice a RoPE frequency table by the rank's token range [MH3, 机制一]
    without defining it; this is the multi-axis form used for packed video
    tokens (the reading is stated in the design notes; parity unpinned by the
    pages).  The d/2 pairs are split into consecutive groups of sections[a]
    pairs, one per axis a; pair j' of axis a (0-based inside its group)
    rotates by pos[token, a] * theta**(-2 j' / d_a) with d_a = 2 * sections[a].
    Pairing and the rotation formula are those of rope_apply.  Float64.
    """
    x = np.asarray(x, dtype=np.float64)
    s, H, d = x.shape
    pos = np.asarray(pos, dtype=np.float64).reshape(s, len(sections))
    if d % 2 or sum(sections) != d // 2:
        raise ValueError("sections must add up to d/2 pairs")
    ang = np.empty((s, d // 2), dtype=np.float64)
    j0 = 0
    for a, n in enumerate(sections):
        if n:
            ang[:, j0:j0 + n] = pos[:, a:a + 1] * rope_inv_freq(2 * n, theta)[None, :]
        j0 += n
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    if style == "half":
        x1, x2 = x[..., : d // 2], x[..., d // 2:]
    elif style == "interleaved":
        x1, x2 = x[..., 0::2], x[..., 1::2]
    else:
        raise ValueError("style must be 'half' or 'interleaved'")
    y = np.empty_like(x)
    y1 = x1 * cos - x2 * sin
    y2 = x2 * cos + x1 * sin
    if style == "half":
        y[..., : d // 2], y[..., d // 2:] = y1, y2
    else:
        y[..., 0::2], y[..., 1::2] = y1, y2
    return y


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x**2) + eps) * gamma, float64.

    [HY3] section "RmsNorm算子优化": RmsNorm is LayerNorm without the mean
    subtraction.  gamma has one weight per feature (the head dimension here).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + np.float64(eps)) * np.asarray(gamma, dtype=np.float64)


def qk_norm_rope(x: np.ndarray, gamma: np.ndarray, eps: float, pos0: int = 0, pos=None, sections=None,
                 theta: float = 10000.0, style: str = "half") -> np.ndarray:
    """Per-head RMSNorm of q or k followed by the rotary embedding, float64.

    [HY3] section "计算分解": after the merged QKV projection the query and key
    heads are normalised and rotated before attention (the page's "Q和V" is
    read as Q and K: the rotation applies to q and k, section
    消除旋转位置编码冗余cast算子).  One axis with positions pos0 + t when pos is
    None, else the multi-axis form of rope_apply_mx.
    """
    xn = rms_norm(x, gamma, eps)
    if pos is None:
        return rope_apply(xn, pos0, theta, style)
    return rope_apply_mx(xn, pos, sections, theta, style)


# ---------------------------------------------------------------------------
# 2-D spatial tiles of the VAE  [HY3, VAE并行优化]
# ---------------------------------------------------------------------------


def tile_bounds(Hh: int, Ww: int, pr: int, pc: int, p: int) -> tuple[int, int, int, int]:
    """Block (r0, r1, c0, c1) of process p when an Hh x Ww grid is cut into pr x pc blocks.

    [HY3, VAE并行优化] cuts the image along height and width into blocks, one
    per process; how the cut falls is not stated.  Reading: processes are
    numbered row-major over the block grid (p = i*pc + j) and each axis is cut
    like the token ranges of [MH3, 机制一]: rows [Hh*i//pr, Hh*(i+1)//pr),
    columns [Ww*j//pc, Ww*(j+1)//pc).
    """
    Hh, Ww, pr, pc, p = int(Hh), int(Ww), int(pr), int(pc), int(p)
    if pr < 1 or pc < 1 or not (0 <= p < pr * pc) or Hh < 0 or Ww < 0:
        raise ValueError("need pr, pc >= 1, 0 <= p < pr*pc, Hh, Ww >= 0")
    i, j = divmod(p, pc)
    r0, r1 = shard_bounds(Hh, pr, i)
    c0, c1 = shard_bounds(Ww, pc, j)
    return r0, r1, c0, c1


def tile_pack(raster: np.ndarray, pr: int, pc: int) -> np.ndarray:
    """Cut a channels-last raster [Hh, Ww, C] into its pr*pc blocks and lay them
    out one after another in process order, each block row-major: [sum h_p*w_p, C].

    This is the split of the input over the processes ([HY3, VAE并行优化], first
    step) and, block after block, the AllGatherV receive buffer of the K and V
    blocks ([MH3, 后端 A] with one block per process).
    """
    raster = np.asarray(raster)
    Hh, Ww = raster.shape[0], raster.shape[1]
    parts = []
    for p in range(pr * pc):
        r0, r1, c0, c1 = tile_bounds(Hh, Ww, pr, pc, p)
        parts.append(raster[r0:r1, c0:c1].reshape((r1 - r0) * (c1 - c0), *raster.shape[2:]))
    return np.concatenate(parts, axis=0)


def tile_unpack(flat: np.ndarray, Hh: int, Ww: int, pr: int, pc: int) -> np.ndarray:
    """Inverse of tile_pack: put each process's block back at its spatial position.

    The second stage of the two-stage gather of [HY3, VAE并行优化] (the first
    stage is the AllGatherV that concatenates the blocks in process order).
    """
    flat = np.asarray(flat)
    out = np.zeros((Hh, Ww) + flat.shape[1:], dtype=flat.dtype)
    a = 0
    for p in range(pr * pc):
        r0, r1, c0, c1 = tile_bounds(Hh, Ww, pr, pc, p)
        n = (r1 - r0) * (c1 - c0)
        out[r0:r1, c0:c1] = flat[a:a + n].reshape((r1 - r0), (c1 - c0), *flat.shape[1:])
        a += n
    if a != flat.shape[0]:
        raise ValueError("flat does not hold exactly the pr*pc blocks")
    return out


def av_positions(T: int, Hh: int, Ww: int, n_audio: int, a: int, b: int) -> np.ndarray:
    """Axis positions [b - a, 3] of tokens [a, b) of a packed video + audio sequence.

    Video tokens come first, frame-major then row-major (token i < T*Hh*Ww is
    frame i // (Hh*Ww), row (i // Ww) % Hh, column i % Ww); the n_audio audio
    tokens follow and take a 1-D position, their index among the audio tokens,
    on the first axis (0 on the others).  Reading of the packed layout
    (video then audio in one index) stated in the design notes.
    """
    V = T * Hh * Ww
    if not (0 <= a <= b <= V + n_audio):
        raise ValueError("token range outside the sequence")
    out = np.zeros((b - a, 3), dtype=np.int64)
    for k, i in enumerate(range(a, b)):
        if i < V:
            out[k] = (i // (Hh * Ww), (i // Ww) % Hh, i % Ww)
        else:
            out[k, 0] = i - V
    return out


# ---------------------------------------------------------------------------
# Attention of local queries against the full sequence  [MH3, 机制一; HY3]
# ---------------------------------------------------------------------------


def _attend_head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, row_block: int):
    """softmax(scale * qh kh^T) vh and the natural-log LSE for one head, float64.

    Query rows are independent, so they are taken row_block at a time only to
    bound memory; every row is the plain definition.
    """
    sq = qh.shape[0]
    o = np.empty((sq, vh.shape[1]), dtype=np.float64)
    lse = np.empty(sq, dtype=np.float64)
    for i0 in range(0, sq, row_block):
        i1 = min(sq, i0 + row_block)
        logits = (qh[i0:i1] @ kh.T) * np.float64(scale)            # [rows, skv]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        z = e.sum(axis=1, keepdims=True)
        o[i0:i1] = (e / z) @ vh
        lse[i0:i1] = (m + np.log(z))[:, 0]
    return o, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None,
              row_block: int = 1024):
    """O[i,h,:] = sum_j softmax_j(scale <q_ih, k_jh>) v_jh, unmasked  [MH3, 机制一].

    q [sq, H, d] are the rank's local (rotated) queries, k and v [skv, H, d] the
    full gathered sequence.  scale defaults to 1/sqrt(d) [HY3].  Returns
    (O [sq, H, d], LSE [H, sq]) in float64, LSE = log sum_j exp(scale <q, k_j>).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sq, H, d = q.shape
    if k.shape[1:] != (H, d) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((sq, H, d), dtype=np.float64)
    lse = np.empty((H, sq), dtype=np.float64)
    for h in range(H):
        o[:, h, :], lse[h] = _attend_head(q[:, h, :], k[:, h, :], v[:, h, :], scale, row_block)
    return o, lse


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None,
                   widen=None):
    """attention() for a few query rows against a (possibly huge) K/V.

    Identical definition; K and V are widened to float64 one head at a time so
    that full-size sequences fit in host memory.  `widen` maps a raw [skv, d]
    head slice to float64 (default: np.asarray(..., float64)); callers holding
    bf16 bit patterns pass a widening function from the input generator.
    """
    if widen is None:
        def widen(a):
            return np.asarray(a, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    n, H, d = q_rows.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((n, H, d), dtype=np.float64)
    lse = np.empty((H, n), dtype=np.float64)
    for h in range(H):
        kh = widen(k[:, h, :])
        vh = widen(v[:, h, :])
        o[:, h, :], lse[h] = _attend_head(q_rows[:, h, :], kh, vh, scale, row_block=256)
    return o, lse

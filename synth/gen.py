"""Seeded, chunked N(0,1) generation of token-major [S, H, d] tensors.

Every chunk of CHUNK tokens of tensor t (0 = Q, 1 = K, 2 = V) draws from its
own numpy PCG64 stream seeded by SeedSequence(seed, spawn_key=(t, chunk)), so a
tensor is the same whether it is generated whole, in pieces or on several
threads.  bf16 workloads round the fp32 draws to bf16 once, round-to-nearest-
even, and both the oracle and the GPU path read those exact bf16 values.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 4096  # tokens per independent random stream


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite normal draws; NaN is not handled specially.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _chunk_rng(seed: int, tensor_id: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(tensor_id, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def gen_tensor(seed: int, tensor_id: int, S: int, H: int, d: int, dtype: str,
               tok0: int = 0, tok1: int | None = None, threads: int | None = None) -> np.ndarray:
    """Tokens [tok0, tok1) of tensor `tensor_id` of a [S, H, d] workload tensor.

    Returns float32 for dtype "f32" and uint16 bf16 bit patterns for "bf16".
    tok0 and tok1 may cut through chunks; the values do not depend on them.
    """
    if tok1 is None:
        tok1 = S
    if not (0 <= tok0 <= tok1 <= S):
        raise ValueError("token range out of bounds")
    out_dtype = np.float32 if dtype == "f32" else np.uint16
    out = np.empty((tok1 - tok0, H, d), dtype=out_dtype)
    c0, c1 = tok0 // CHUNK, (tok1 + CHUNK - 1) // CHUNK

    def work(c):
        rng = _chunk_rng(seed, tensor_id, c)
        n = min(CHUNK, S - c * CHUNK)
        vals = rng.standard_normal((n, H, d), dtype=np.float32)
        a, b = max(tok0, c * CHUNK), min(tok1, c * CHUNK + n)
        sl = vals[a - c * CHUNK: b - c * CHUNK]
        out[a - tok0: b - tok0] = sl if dtype == "f32" else f32_to_bf16_bits(sl)

    nthreads = threads or min(32, os.cpu_count() or 1)
    if c1 - c0 <= 1 or nthreads == 1:
        for c in range(c0, c1):
            work(c)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(c0, c1)))
    return out


def gen_gamma(seed: int, d: int) -> np.ndarray:
    """A float32 RMSNorm weight [d]: 1 + 0.1 * N(0, 1), the spread of a trained
    norm weight around its initial value of one (synthetic: no checkpoint)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(7, d))))
    return (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)


def gen_qkv(wl, scale_q: float = 1.0, threads: int | None = None):
    """Full [S, H, d] Q, K, V of a workload (see gen_tensor for the dtype).

    scale_q multiplies the (already rounded) Q; it is meant for powers of two
    (the "peaky" variant uses Q x 4), which are exact in bf16.
    """
    q = gen_tensor(wl.seed, 0, wl.S, wl.H, wl.d, wl.dtype, threads=threads)
    k = gen_tensor(wl.seed, 1, wl.S, wl.H, wl.d, wl.dtype, threads=threads)
    v = gen_tensor(wl.seed, 2, wl.S, wl.H, wl.d, wl.dtype, threads=threads)
    if scale_q != 1.0:
        if wl.dtype == "f32":
            q = q * np.float32(scale_q)
        else:
            q = f32_to_bf16_bits(bf16_bits_to_f32(q) * np.float32(scale_q))
    return q, k, v


def sample_rows(n_rows: int, count: int, seed: int, tile: int = 128) -> np.ndarray:
    """Sorted distinct row indices in [0, n_rows) for sampled checks.

    Always includes the first and last rows and rows on both sides of multiples
    of `tile` (where GPU tiles start and end), topped up with uniform draws.
    """
    rows = {0, n_rows - 1}
    for t in (tile, 2 * tile, (n_rows // tile) * tile):
        for r in (t - 1, t, t + 1):
            if 0 <= r < n_rows:
                rows.add(r)
    rng = np.random.default_rng(seed)
    while len(rows) < min(count, n_rows):
        rows.add(int(rng.integers(0, n_rows)))
    return np.array(sorted(rows), dtype=np.int64)

"""Workload descriptions for one rank's share of packed-token sequence-parallel
DiT self-attention.

The pages (MiniMax-H3-Comfy-NPU, "mechanism one") split one packed audio+video
token sequence of length S over W ranks and run attention of each rank's local
queries against the full key/value sequence.  They give no model dimensions;
the head count, head size and token counts below describe synthetic stand-ins
for the pages' 480P and 768P (1344x768, 24 fps, 5 s and 15 s) video workloads:
video latent tokens (width x height per latent frame x latent frames) followed
by the audio tokens appended to the same packed index.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    S: int                 # packed sequence length (video tokens + audio tokens)
    W: int                 # simulated rank count
    ranks: tuple           # ranks whose local share is exercised
    H: int                 # attention heads
    d: int                 # head size
    dtype: str             # "f32" or "bf16": storage and MFMA operand type
    seed: int
    theta: float = 10000.0  # RoPE base
    note: str = ""
    video: tuple = field(default=())  # (w, h, frames) of the video latent grid
    audio: int = 0                    # audio tokens appended after the video


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", S=1001, W=4, ranks=(1,), H=2, d=64, dtype="f32", seed=1,
        note="tiny fp32 case: rank 1 holds [250,500) of 1001 tokens"),
    "uneven_bf16": Workload(
        "uneven_bf16", S=16383, W=4, ranks=(0, 1, 2, 3), H=16, d=128, dtype="bf16", seed=2,
        note="uneven shards 4095/4096/4096/4096, every rank in turn"),
    "p480_w1": Workload(
        "p480_w1", S=25640, W=1, ranks=(0,), H=24, d=128, dtype="bf16", seed=3,
        video=(53, 30, 16), audio=200,
        note="480P-like: 53x30 latent tokens x 16 frames + 200 audio tokens, one rank"),
    "p768_5s_w4": Workload(
        "p768_5s_w4", S=125117, W=4, ranks=(3,), H=24, d=128, dtype="bf16", seed=4,
        video=(84, 48, 31), audio=125,
        note="768P/5 s-like: 84x48 latent tokens x 31 frames + 125 audio tokens, rank 3"),
    "p768_15s_w4": Workload(
        "p768_15s_w4", S=367287, W=4, ranks=(0,), H=24, d=128, dtype="bf16", seed=5,
        video=(84, 48, 91), audio=375,
        note="768P/15 s-like: 84x48 latent tokens x 91 frames + 375 audio tokens, rank 0"),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None

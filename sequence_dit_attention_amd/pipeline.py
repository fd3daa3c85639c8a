"""One rank's share of packed-token sequence-parallel DiT attention on one GPU.

The sequence of library calls that one rank makes, as the pages lay it out
(MiniMax-H3-Comfy-NPU, sections 机制一 and 机制二/后端 A):
  1. RoPE on the rank's local Q and K slice at absolute positions,
  2. AllGatherV of K and V: every rank's shard packed into a flat buffer by
     counts/displacements, then narrow/view/concat back to [S, H, d],
  3. attention of the local Q against the full K/V,
  4. the final AllGatherV of the per-rank outputs along the sequence.
On one GPU the W ranks' shards are W separate device buffers; the other
ranks' K shards are rotated once at set-up (each rank rotates its own), and
their outputs are stand-in buffers of the right shape (their attention would
run on their own GPUs).  Only library calls run here: no computation in
Python, no synchronisation.
"""
from __future__ import annotations

import math

import torch

from . import api


class RankShare:
    def __init__(self, S: int, W: int, r: int, H: int, d: int, dtype: torch.dtype,
                 theta: float = 10000.0, device="cuda", style: str = "half"):
        self.S, self.W, self.r, self.H, self.d = S, W, r, H, d
        self.dtype, self.theta, self.style, self.device = dtype, theta, style, torch.device(device)
        self.bounds = [api.sp_shard_bounds(S, W, i) for i in range(W)]
        self.lens = [b - a for a, b in self.bounds]
        self.inner = H * d
        self.counts, self.displs = api.sp_allgatherv_layout(S, W, 1, self.inner)
        self.scale = 1.0 / math.sqrt(d)
        a, b = self.bounds[r]
        self.a, self.b = a, b
        e = dict(dtype=dtype, device=self.device)
        self.q_rot = torch.empty(b - a, H, d, **e)
        self.k_rot = [torch.empty(n, H, d, **e) for n in self.lens]
        self.flat_k = torch.empty(S * self.inner, **e)
        self.flat_v = torch.empty(S * self.inner, **e)
        self.k_full = torch.empty(S, H, d, **e)
        self.v_full = torch.empty(S, H, d, **e)
        self.o_shards = [torch.zeros(n, H, d, **e) for n in self.lens]
        self.flat_o = torch.empty(S * self.inner, **e)
        self.o_full = torch.empty(S, H, d, **e)
        self.lse = torch.empty(H, b - a, dtype=torch.float32, device=self.device)
        self.q = self.k = self.v = None

    def set_inputs(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """Full-sequence raw Q, K, V [S, H, d] on the device; rank shards are row slices."""
        for t in (q, k, v):
            if t.shape != (self.S, self.H, self.d) or t.dtype != self.dtype or not t.is_contiguous():
                raise ValueError("inputs must be contiguous [S, H, d] of the share's dtype")
        self.q, self.k, self.v = q, k, v
        self.v_shards = [v[a:b] for a, b in self.bounds]
        for i, (a, b) in enumerate(self.bounds):  # other ranks rotate their own K
            if i != self.r:
                api.rope_apply(k[a:b], a, self.theta, self.style, out=self.k_rot[i])

    # -- the rank's hot path ------------------------------------------------------
    def rope(self) -> None:
        a, b = self.a, self.b
        api.rope_apply(self.q[a:b], a, self.theta, self.style, out=self.q_rot)
        api.rope_apply(self.k[a:b], a, self.theta, self.style, out=self.k_rot[self.r])

    def gather_kv_pack(self) -> None:
        api.varlen_pack([t.view(-1) for t in self.k_rot], self.counts, self.displs, self.flat_k)
        api.varlen_pack([t.reshape(-1) for t in self.v_shards], self.counts, self.displs, self.flat_v)

    def gather_kv_unpack(self) -> None:
        api.varlen_unpack(self.flat_k, self.displs, self.lens, 1, self.inner, self.k_full)
        api.varlen_unpack(self.flat_v, self.displs, self.lens, 1, self.inner, self.v_full)

    def gather_kv(self) -> None:
        self.gather_kv_pack()
        self.gather_kv_unpack()

    def attend(self) -> None:
        api.shard_attn_fwd(self.q_rot, self.k_full, self.v_full, out=self.o_shards[self.r],
                           lse=self.lse, scale=self.scale)

    def attend_gather_free(self) -> None:
        """Attention reading K/V from the rank shards in place (no pack/unpack)."""
        api.shard_attn_fwd_gv(self.q_rot, self.k_rot, self.v_shards, out=self.o_shards[self.r],
                              lse=self.lse, scale=self.scale)

    def concat_out(self) -> None:
        api.varlen_pack([t.view(-1) for t in self.o_shards], self.counts, self.displs, self.flat_o)
        api.varlen_unpack(self.flat_o, self.displs, self.lens, 1, self.inner, self.o_full)

    def step(self) -> None:
        self.rope()
        self.gather_kv()
        self.attend()
        self.concat_out()

    def step_gather_free(self) -> None:
        """The same share without the K/V gather: attention reads the shards directly."""
        self.rope()
        self.attend_gather_free()
        self.concat_out()

    # -- algorithmic work of one step -------------------------------------------------
    def attn_flops(self) -> int:
        return 4 * (self.b - self.a) * self.S * self.H * self.d

    def pack_kv_bytes(self) -> int:
        """Read + write bytes of the K and V pack (one AllGatherV of each)."""
        return 2 * 2 * self.S * self.inner * self.flat_k.element_size()


class VaeBlockShare:
    """Process p's share of the VAE's attention under the spatial block split.

    Page NPU HunyuanImage-3.0模型推理优化实践, section VAE并行优化: the feature
    map is cut along height and width into pr x pc blocks, one per process;
    attention gathers the K and V of all blocks; the outputs are gathered back
    in two stages and put at their spatial positions.  Per step:
      1. gather of the K and V blocks in process order (tile_pack_n of the
         two channels-last rasters, one batch of copies: the AllGatherV
         receive buffers),
      2. attention of process p's block queries against all gathered keys,
         one head over the C channels, keys cut into nsplit ranges,
         written straight into p's slot of the flat output,
      3. second stage of the output gather: the flat blocks back into the
         raster (tile_unpack); the other processes' output blocks are
         stand-ins, as on a real run they come from their own GPUs.
    Process p's query block is prepared at set-up (on a real run the 1x1
    projections produce it locally).
    """

    def __init__(self, Hh: int, Ww: int, C: int, pr: int, pc: int, p: int, nsplit: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda"):
        self.Hh, self.Ww, self.C, self.pr, self.pc, self.p, self.nsplit = Hh, Ww, C, pr, pc, p, nsplit
        self.n = Hh * Ww
        self.blocks = [api.sp_tile_bounds(Hh, Ww, pr, pc, i) for i in range(pr * pc)]
        sizes = [(r1 - r0) * (c1 - c0) for r0, r1, c0, c1 in self.blocks]
        self.off = sum(sizes[:p])
        self.m = sizes[p]
        e = dict(dtype=dtype, device=torch.device(device))
        self.k_flat = torch.empty(self.n, C, **e)
        self.v_flat = torch.empty(self.n, C, **e)
        self.o_flat = torch.zeros(self.n, C, **e)
        self.o = torch.empty(Hh, Ww, C, **e)
        self.q_block = torch.empty(self.m, C, **e)
        self.workspace = torch.empty(api.split_workspace_bytes(self.m, 1, C, nsplit), dtype=torch.uint8,
                                     device=torch.device(device))
        self.q = self.k = self.v = None

    def set_inputs(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        """Channels-last rasters [Hh, Ww, C]; process p's query block is cut out once here."""
        for t in (q, k, v):
            if t.shape != (self.Hh, self.Ww, self.C) or not t.is_contiguous():
                raise ValueError("inputs must be contiguous [Hh, Ww, C]")
        self.q, self.k, self.v = q, k, v
        flat = api.tile_pack(q, self.pr, self.pc)
        self.q_block.copy_(flat[self.off:self.off + self.m])

    def gather_kv(self) -> None:
        api.tile_pack_n([self.k, self.v], self.pr, self.pc, [self.k_flat, self.v_flat])

    def attend(self) -> None:
        C = self.C
        api.shard_attn_fwd_split(self.q_block.view(self.m, 1, C), self.k_flat.view(self.n, 1, C),
                                 self.v_flat.view(self.n, 1, C), self.nsplit,
                                 out=self.o_flat[self.off:self.off + self.m].view(self.m, 1, C),
                                 workspace=self.workspace)

    def place_out(self) -> None:
        api.tile_unpack(self.o_flat, self.Hh, self.Ww, self.pr, self.pc, self.o)

    def step(self) -> None:
        self.gather_kv()
        self.attend()
        self.place_out()

    def capture(self) -> torch.cuda.CUDAGraph:
        """The step recorded as a HIP graph.  The share is four short launches
        around one attention launch, so issuing it from the host leaves the
        GPU idle between them; a replay issues all of them at once.  Nothing in
        the step allocates, synchronises or clears memory.  Each replay reads
        whatever the input rasters hold at that time (their addresses are
        recorded, so the rasters and this object must stay alive)."""
        if self.k is None:
            raise RuntimeError("set_inputs first")
        side = torch.cuda.Stream(device=self.k.device)  # default priority
        side.wait_stream(torch.cuda.current_stream(self.k.device))
        with torch.cuda.stream(side):
            self.step()  # first use of every launch outside the capture
        torch.cuda.current_stream(self.k.device).wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        return g

    def attn_flops(self) -> int:
        return 4 * self.m * self.n * self.C

    def copy_bytes(self) -> int:
        """Read + write bytes of the K and V gathers and of the output placement."""
        return 3 * 2 * self.n * self.C * self.k_flat.element_size()

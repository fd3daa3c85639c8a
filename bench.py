#!/usr/bin/env python3
"""Benchmark of one rank's share of packed-token sequence-parallel DiT attention.

One step = the whole hot path of one rank on one MI355X: RoPE of the local Q
and K slice, AllGatherV of K and V (pack into the flat buffer + unpack), the
attention of the local Q shard against the full K/V, and the AllGatherV of
the per-rank outputs.  Default workload: the 768P/15 s-like sequence
(S = 367,287 packed tokens, W = 4 simulated ranks, rank 0 holds 91,821 query
tokens, 24 heads x 128, bf16).  Inputs are resident in HBM before timing.

Prints ONE JSON line.  `value` = attention FLOP of a step / wall time of the
whole step (TFLOP/s); per-kernel times come from HIP events recorded on the
stream the kernels run on (torch's current stream) over the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard-attention TFLOP/s (% bf16 MFMA peak) + varlen pack GB/s (% HBM), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
ATTN_SRC = os.path.join(ROOT, "sequence_dit_attention_amd", "csrc", "attn_d128.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_d128_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(wl_name: str):
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary,
    or None when it is missing or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash() or t.get("workload") != wl_name:
        return None
    return t.get("hbm_bytes_per_launch")


def host_info() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, CPUs this
    process may use, and the BLAS threads numpy's oracle actually runs with."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = None
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable, "blas_threads": blas}


def _oracle_share(wl, r, q64, k64, v64):
    """The oracle's whole share of rank r in float64: RoPE of its Q and K slice,
    AllGatherV pack + unpack of K and V, attention of its queries against the
    full K/V, pack + unpack of the W outputs (the other ranks' K rotated and
    outputs stood in before timing, as on the GPU).  Returns seconds."""
    import numpy as np

    import oracle

    bounds = oracle.all_shard_bounds(wl.S, wl.W)
    inner = wl.H * wl.d
    lens = [b - a for a, b in bounds]
    k_rot = [oracle.rope_apply(k64[a:b], a, wl.theta) for a, b in bounds]
    v_sh = [v64[a:b] for a, b in bounds]
    o_sh = [np.zeros((n, wl.H, wl.d)) for n in lens]
    counts, displs = oracle.allgatherv_layout(wl.S, wl.W, 1, inner)
    a, b = bounds[r]
    t0 = time.perf_counter()
    qr = oracle.rope_apply(q64[a:b], a, wl.theta)
    k_rot[r] = oracle.rope_apply(k64[a:b], a, wl.theta)
    k_full = oracle.varlen_unpack(oracle.varlen_pack(k_rot, counts, displs, np.zeros(sum(counts))), displs, lens, 1,
                                  inner).reshape(wl.S, wl.H, wl.d)
    v_full = oracle.varlen_unpack(oracle.varlen_pack(v_sh, counts, displs, np.zeros(sum(counts))), displs, lens, 1,
                                  inner).reshape(wl.S, wl.H, wl.d)
    o_sh[r] = oracle.attention(qr, k_full, v_full)[0]
    oracle.varlen_unpack(oracle.varlen_pack(o_sh, counts, displs, np.zeros(sum(counts))), displs, lens, 1, inner)
    return time.perf_counter() - t0


def _gpu_share_ms(wl, r, qd, kd, vd, reps: int = 5) -> float:
    """Event-timed whole share of rank r on the GPU (median of reps)."""
    import torch

    from sequence_dit_attention_amd.pipeline import RankShare

    share = RankShare(wl.S, wl.W, r, wl.H, wl.d, qd.dtype, wl.theta, qd.device)
    share.set_inputs(qd, kd, vd)
    share.step()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        share.step()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return sorted(times)[len(times) // 2]


def cpu_baseline(wl, q, k, v, a, b, rows: int, gpu_attn_ms: float, gpu_pack_ms: float, gpu_rope_ms: float):
    """The float64 oracle on the host, beside the GPU numbers of the same run.

    Headline (`value`): the oracle's attention on a bounded sample of the
    benchmark workload -- `rows` query rows of the rank's shard (first and last
    rows, both sides of 128-row tile edges, the rest drawn at random) x all
    heads against the full K/V -- in TFLOP/s, extrapolated to the shard.
    `rows_detail` adds the oracle's whole rank share, timed in full, of the tiny
    float32 workload and of the uneven bf16 workload (all four ranks of each),
    each beside the GPU's event-timed share, and the oracle's K pack and RoPE
    at the benchmark size.  Widening bf16 to float64 is set-up, not timed."""
    import numpy as np
    import torch

    import oracle
    from synth import bf16_bits_to_f32, gen_qkv, get_workload, sample_rows

    info = host_info()
    idx = a + sample_rows(b - a, rows, seed=17)
    qrows = bf16_bits_to_f32(q[idx]).astype(np.float64)
    spent = 0.0
    for h in range(wl.H):
        kh = bf16_bits_to_f32(k[:, h:h + 1, :]).astype(np.float64)
        vh = bf16_bits_to_f32(v[:, h:h + 1, :]).astype(np.float64)
        t0 = time.perf_counter()
        oracle.attention(qrows[:, h:h + 1, :], kh, vh)
        spent += time.perf_counter() - t0
    n = len(idx)
    flops = 4.0 * n * wl.S * wl.H * wl.d
    cpu_tflops = flops / spent / 1e12
    shard_s = spent * (b - a) / n
    detail = [{"workload": wl.name, "what": f"attention of the rank-{wl.ranks[0]} shard ({b - a} queries x {wl.H} "
                                           f"heads x {wl.S} keys)",
               "kind": f"extrapolated from {n} rows", "cpu_s": shard_s, "gpu_ms": gpu_attn_ms,
               "gpu_over_cpu": shard_s * 1e3 / gpu_attn_ms}]

    # The oracle's whole share, in full, on the two workloads small enough for it.
    def widen(x, dt):
        return (bf16_bits_to_f32(x) if dt == "bf16" else x).astype(np.float64)

    def dev(x, dt):
        if dt == "f32":
            return torch.from_numpy(np.ascontiguousarray(x)).cuda()
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    for name in ("tiny_f32", "uneven_bf16"):
        w = get_workload(name)
        wq, wk, wv = gen_qkv(w)
        q64, k64, v64 = widen(wq, w.dtype), widen(wk, w.dtype), widen(wv, w.dtype)
        ranks = list(range(w.W))   # every rank of the workload, one after another
        cpu_s = sum(_oracle_share(w, r, q64, k64, v64) for r in ranks)
        qd, kd, vd = dev(wq, w.dtype), dev(wk, w.dtype), dev(wv, w.dtype)
        gpu_ms = sum(_gpu_share_ms(w, r, qd, kd, vd) for r in ranks)
        log(f"CPU oracle, {name}: {cpu_s:.1f} s for ranks {ranks} (GPU {gpu_ms:.3f} ms)")
        detail.append({"workload": name, "what": f"whole share (RoPE, K/V pack + unpack, attention, output "
                                                  f"concat) of ranks {ranks}, summed",
                       "kind": "full", "cpu_s": cpu_s, "gpu_ms": gpu_ms, "gpu_over_cpu": cpu_s * 1e3 / gpu_ms})

    # Data movement at the benchmark size: the oracle's AllGatherV pack of the
    # four K shards (the whole tensor, bf16 bit patterns) and its RoPE of 2,048
    # tokens of the rank's Q slice, in algorithmic GB/s of the bf16 data.
    bounds = [oracle.shard_bounds(wl.S, wl.W, r) for r in range(wl.W)]
    inner = wl.H * wl.d
    counts, displs = oracle.allgatherv_layout(wl.S, wl.W, 1, inner)
    sends = [np.ascontiguousarray(k[x:y]).reshape(-1) for x, y in bounds]
    flat = np.empty(wl.S * inner, dtype=k.dtype)
    t0 = time.perf_counter()
    oracle.varlen_pack(sends, counts, displs, flat)
    t_pack = time.perf_counter() - t0
    nr = min(2048, b - a)
    qs = bf16_bits_to_f32(q[a:a + nr]).astype(np.float64)
    t0 = time.perf_counter()
    oracle.rope_apply(qs, a, wl.theta)
    t_rope = time.perf_counter() - t0
    pack_b = 2.0 * wl.S * inner * k.itemsize
    rope_b = 2.0 * nr * inner * 2
    gpu_pack_gbs = 2 * pack_b / (gpu_pack_ms * 1e-3) / 1e9   # the GPU step packs K and V
    gpu_rope_gbs = 2 * 2.0 * (b - a) * inner * 2 / (gpu_rope_ms * 1e-3) / 1e9   # RoPE of Q and K
    detail.append({"workload": wl.name, "what": f"AllGatherV pack of the {wl.W} K shards ({pack_b / 2e9:.2f} GB)",
                   "kind": "full", "cpu_gbs": pack_b / t_pack / 1e9, "gpu_gbs": gpu_pack_gbs,
                   "gpu_over_cpu": gpu_pack_gbs / (pack_b / t_pack / 1e9)})
    detail.append({"workload": wl.name, "what": f"RoPE of {nr} tokens x {wl.H} heads of the rank's Q slice",
                   "kind": "sample", "cpu_gbs": rope_b / t_rope / 1e9, "gpu_gbs": gpu_rope_gbs,
                   "gpu_over_cpu": gpu_rope_gbs / (rope_b / t_rope / 1e9)})
    gpu_tflops = flops / n * (b - a) / (gpu_attn_ms * 1e-3) / 1e12
    return {"value": cpu_tflops, "unit": "TFLOP/s", "cores": info["blas_threads"] or info["usable_cpus"],
            "kind": "oracle",
            "sample": f"{n} query rows x {wl.H} heads of the rank-{wl.ranks[0]} shard against the full {wl.S}-token "
                      f"K/V (fp64 numpy oracle attention, {spent:.1f} s)",
            "host": info, "gpu_over_cpu": gpu_tflops / cpu_tflops, "rows_detail": detail}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="p768_15s_w4")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="query rows in the CPU-oracle sample, about 15-20 s of host work (0: skip)")
    ap.add_argument("--vae-steps", type=int, default=20, help="timed steps of the VAE block-split share (0: skip)")
    ap.add_argument("--vae-eager-only", action="store_true",
                    help="time the VAE share's eager steps only (no graph replay), e.g. under counter collection")
    ap.add_argument("--calib-copy-gib", type=float, default=0.0,
                    help="before timing, one plain elementwise copy (torch neg) of this many GiB of bf16, the known-size "
                         "kernel the HBM counters of a profile are calibrated on (0: none)")
    ap.add_argument("--gf-steps", type=int, default=2,
                    help="steps of the gather-free variant timed after the headline steps (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (--gpus {args.gpus} "
              "requested). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sequence_dit_attention_amd import api
    from sequence_dit_attention_amd.pipeline import RankShare
    from synth import gen_gamma, gen_qkv, gen_tensor, get_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wl = get_workload(args.workload)
    if wl.dtype != "bf16":
        print("bench.py times the bf16 workloads", file=sys.stderr)
        return 1
    r = wl.ranks[0]
    dev = torch.device("cuda:0")
    t0 = time.time()
    log(f"workload {wl.name}: S={wl.S} W={wl.W} rank={r} H={wl.H} d={wl.d}; generating inputs")
    q, k, v = gen_qkv(wl)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    share = RankShare(wl.S, wl.W, r, wl.H, wl.d, torch.bfloat16, wl.theta, dev)
    share.set_inputs(up(q), up(k), up(v))
    torch.cuda.synchronize()
    log(f"inputs resident after {time.time() - t0:.1f}s; warmup {args.warmup} steps")

    for _ in range(args.warmup):
        share.step()
    torch.cuda.synchronize()

    calib = None
    if args.calib_copy_gib > 0:
        n = int(args.calib_copy_gib * (1 << 30)) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(src, out=dst)
        e1.record()
        torch.cuda.synchronize()
        calib = {"kernel": "torch neg (vectorized elementwise)", "bytes_read": 2 * n, "bytes_written": 2 * n,
                 "ms": e0.elapsed_time(e1)}
        del src, dst
        log(f"calibration copy: {4 * n / 2**30:.2f} GiB moved in {calib['ms']:.3f} ms")

    stages = ["rope", "pack_kv", "unpack_kv", "attn", "concat_out"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        e = ev[i]
        e[0].record()
        share.rope()
        e[1].record()
        share.gather_kv_pack()
        e[2].record()
        share.gather_kv_unpack()
        e[3].record()
        share.attend()
        e[4].record()
        share.concat_out()
        e[5].record()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    per = {s: sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)) / args.steps
           for j, s in enumerate(stages)}
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms); "
        + ", ".join(f"{s} {t:.3f} ms" for s, t in per.items()))

    # The attention call alone, back to back (one event pair around the calls,
    # the queue ahead of the GPU): on short workloads the per-stage events of a
    # step also hold the host's launch gap before the call.
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nb = max(args.steps, 3)
    b0.record()
    for _ in range(nb):
        share.attend()
    b1.record()
    torch.cuda.synchronize()
    attn_call_ms = b0.elapsed_time(b1) / nb

    # The gather-free variant of the same share (K/V read from the rank shards by
    # the attention kernel, no pack/unpack); reported beside the headline step.
    gf = None
    if args.gf_steps > 0:
        share.step_gather_free()
        torch.cuda.synchronize()
        g = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.gf_steps)]
        for i in range(args.gf_steps):
            g[i][0].record()
            share.rope()
            g[i][1].record()
            share.attend_gather_free()
            g[i][2].record()
            share.concat_out()
            g[i][3].record()
        torch.cuda.synchronize()
        gms = [sum(g[i][j].elapsed_time(g[i][j + 1]) for i in range(args.gf_steps)) / args.gf_steps for j in range(3)]
        gf = {"ms_per_step": sum(gms), "rope_ms": gms[0], "attn_gv_ms": gms[1], "concat_out_ms": gms[2],
              "attn_gv_tflops": share.attn_flops() / (gms[1] * 1e-3) / 1e12}
        log(f"gather-free step: {sum(gms):.3f} ms (attention on the shards {gms[1]:.3f} ms)")

    # Multi-axis RoPE of the rank's Q slice with the packed video+audio positions of
    # the 768P/15 s grid (reported beside the headline step; not part of it).
    rmx = None
    grid = {"p768_15s_w4": (91, 48, 84, 375), "p768_5s_w4": (31, 48, 84, 125)}.get(wl.name)
    if grid is not None:
        T, Hh, Ww, A = grid
        V = T * Hh * Ww
        pos = api.sp_av_positions(T, Hh, Ww, A, share.a, share.b).to(share.q_rot.device)
        nv = max(0, min(share.b, V) - share.a)
        sec_video = (wl.d // 2 - 2 * (wl.d // 6), wl.d // 6, wl.d // 6)
        xq = torch.empty_like(share.q_rot)

        def rope_mx():
            if nv:
                api.rope_apply_mx(share.q[share.a:share.a + nv], pos[:nv], sec_video, wl.theta, out=xq[:nv])
            if nv < share.b - share.a:
                api.rope_apply_mx(share.q[share.a + nv:share.b], pos[nv:], (wl.d // 2, 0, 0), wl.theta,
                                  out=xq[nv:])
        rope_mx()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            rope_mx()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        rmx = {"q_ms": ms, "gbs": 2 * xq.numel() * xq.element_size() / (ms * 1e-3) / 1e9,
               "sections_video": sec_video, "grid": {"T": T, "H": Hh, "W": Ww, "audio": A}}

    # Per-head RMSNorm fused with RoPE on the rank's Q slice at its absolute 1-D
    # positions (the step's RoPE with the q/k norm folded in; reported beside it).
    gamma = torch.from_numpy(gen_gamma(wl.seed, wl.d)).to(share.q_rot.device)
    xn = torch.empty_like(share.q_rot)
    qsl = share.q[share.a:share.b]
    api.qk_norm_rope(qsl, gamma, 1e-6, share.a, theta=wl.theta, out=xn)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        api.qk_norm_rope(qsl, gamma, 1e-6, share.a, theta=wl.theta, out=xn)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    qn_gbs = 2 * xn.numel() * xn.element_size() / (ms * 1e-3) / 1e9
    qnr = {"q_ms": ms, "gbs": qn_gbs, "frac_hbm_peak": qn_gbs / PEAK_HBM_GBS, "eps": 1e-6}

    # The VAE's attention under the spatial block split: process 0 of a 128 x 128
    # latent feature map with 512 channels cut into 2 x 2 blocks (reported
    # beside the headline step; a second workload, not part of it).
    vae = None
    if args.vae_steps > 0:
        from sequence_dit_attention_amd.pipeline import VaeBlockShare
        vs = VaeBlockShare(128, 128, 512, 2, 2, 0, nsplit=8)
        gq, gk, gv = (gen_tensor(wl.seed + 100, t, vs.n, 1, vs.C, "bf16") for t in range(3))
        dev_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16).view(128, 128, 512)
        vs.set_inputs(dev_bf16(gq), dev_bf16(gk), dev_bf16(gv))
        vs.step()
        torch.cuda.synchronize()
        eager_o = vs.o.clone()
        # Eager steps, one event per phase (host launch gaps included).
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.vae_steps)]
        for i in range(args.vae_steps):
            ev[i][0].record()
            vs.gather_kv()
            ev[i][1].record()
            vs.attend()
            ev[i][2].record()
            vs.place_out()
            ev[i][3].record()
        torch.cuda.synchronize()
        vms = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.vae_steps)) / args.vae_steps
               for j in range(3)]
        # The attention call alone (split attention + merge), back to back: one
        # event pair around the calls, so the queue stays ahead of the GPU.
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(args.vae_steps):
            vs.attend()
        b1.record()
        torch.cuda.synchronize()
        call_ms = b0.elapsed_time(b1) / args.vae_steps
        call_tf = vs.attn_flops() / (call_ms * 1e-3) / 1e12
        # The same step replayed as a HIP graph (all five launches issued at once).
        graph_ms, replay_same = None, None
        if not args.vae_eager_only:
            graph = vs.capture()
            graph.replay()
            torch.cuda.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record()
            for _ in range(args.vae_steps):
                graph.replay()
            g1.record()
            torch.cuda.synchronize()
            graph_ms = g0.elapsed_time(g1) / args.vae_steps
            replay_same = bool(torch.equal(vs.o.view(torch.int16), eager_o.view(torch.int16)))
        va_tf = vs.attn_flops() / (vms[1] * 1e-3) / 1e12
        vae = {"workload": "vae_128x128_c512_blocks2x2_p0", "sq": vs.m, "skv": vs.n, "d": vs.C, "nsplit": vs.nsplit,
               "ms_per_step": graph_ms if graph_ms is not None else sum(vms),
               "launch": "eager" if graph_ms is None else "hip_graph", "graph_equals_eager": replay_same,
               "eager_ms_per_step": sum(vms), "gather_kv_ms": vms[0], "attn_ms": vms[1], "place_out_ms": vms[2],
               "attn_tflops": va_tf, "attn_frac_mfma_peak": va_tf / PEAK_BF16_TFLOPS,
               "attn_call_ms": call_ms, "attn_call_tflops": call_tf, "attn_call_frac_mfma_peak": call_tf / PEAK_BF16_TFLOPS,
               "copy_gbs": vs.copy_bytes() / ((vms[0] + vms[2]) * 1e-3) / 1e9}
        if replay_same is False:
            raise RuntimeError("VAE share: graph replay differs from the eager step")
        log(f"VAE block share: {vae['ms_per_step']:.3f} ms per step ({vae['launch']}), {sum(vms):.3f} ms eager "
            f"(attention {vms[1]:.3f} ms, {va_tf:.0f} TFLOP/s); attention call back to back {call_ms * 1e3:.1f} us "
            f"({call_tf:.0f} TFLOP/s)")

    flops = share.attn_flops()
    attn_tflops = flops / (per["attn"] * 1e-3) / 1e12
    pack_bytes = share.pack_kv_bytes()
    pack_gbs = pack_bytes / (per["pack_kv"] * 1e-3) / 1e9
    unpack_gbs = pack_bytes / (per["unpack_kv"] * 1e-3) / 1e9
    traffic = traffic_from_profiles(wl.name)
    out = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "S": wl.S, "W": wl.W, "rank": r, "sq": share.b - share.a,
                   "H": wl.H, "d": wl.d, "theta": wl.theta},
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic},
        "kernels": {
            "attn_ms": per["attn"], "attn_tflops": attn_tflops, "attn_frac_mfma_peak": attn_tflops / PEAK_BF16_TFLOPS,
            "attn_call_ms": attn_call_ms, "attn_call_frac_mfma_peak": flops / (attn_call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "pack_kv_ms": per["pack_kv"], "pack_kv_gbs": pack_gbs, "pack_frac_hbm_peak": pack_gbs / PEAK_HBM_GBS,
            "unpack_kv_ms": per["unpack_kv"], "unpack_kv_gbs": unpack_gbs,
            "rope_ms": per["rope"], "concat_out_ms": per["concat_out"],
            "attn_kernel_sha256_16": kernel_hash(),
        },
        "gather_free": gf,
        "rope_multi_axis": rmx,
        "qk_norm_rope": qnr,
        "vae_block_attention": vae,
    }
    if calib is not None:
        out["calib_copy"] = calib
    if args.cpu_rows > 0:
        log(f"CPU oracle baseline on {args.cpu_rows} rows")
        out["cpu_baseline"] = cpu_baseline(wl, q, k, v, share.a, share.b, args.cpu_rows, per["attn"],
                                           per["pack_kv"], per["rope"])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

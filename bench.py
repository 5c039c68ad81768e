#!/usr/bin/env python3
"""Benchmark of the VSA forward on one MI355X.

One step is one pass of the whole forward over the large video-DiT workload
(B=1, H=56, D=128, S=15488 = 242 blocks of 64, top-49, gated): pool + coarse
attention + top-k routing, then block-sparse attention with the combine fused
into its epilogue, issued through the C ABI stage entry points exactly as
vsa_forward issues them, on PyTorch's current HIP stream with inputs resident
in HBM.  HIP events between the stages give each kernel's average duration
over the timed steps.  Outside the timed steps the stand-alone combine kernel
is timed with L2 and MALL flushed (its HBM rate; median of 20 launches, each
after reading a 1 GiB buffer) and the sparse kernel without the fused combine
is timed for comparison.

Prints one JSON line.  ``value`` is effective TFLOP/s of the whole step with
the pages' benchmark convention 4*B*H*nQ*k*64*64*D (padded blocks counted as
full; with ``--block-size 128`` or ``256`` the same count over the 64-token
sub-blocks of the selected VSA blocks).  ``roofline`` is for the dominant kernel (the sparse attention, MFMA
bound).  ``cpu_baseline`` times the fp64 oracle on this host's cores on a
bounded sample of the same workload (whole heads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VSA fwd effective TFLOP/s & % bf16 MFMA peak; combine HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_large_traffic.json")
SPARSE_SRC = os.path.join(ROOT, "video_sparse_attention_amd", "csrc", "sparse_attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large",
                    choices=["large", "varlen_many", "video", "train", "pages_bench_49k"],
                    help="large (the default line), varlen_many, video: the large shape as an "
                         "11 x 32 x 44 latent in 4 x 4 x 4 tiles, gathered from and scattered to "
                         "raster order, train: the large shape's forward plus backward, or "
                         "pages_bench_49k: B=1 H=16 D=128 S=49152, top-64 of 768 blocks, ungated")
    ap.add_argument("--block-size", type=int, default=64, choices=[64, 128, 256],
                    help="VSA block size for the large workload (128 / 256: top-k about 20%% of the blocks)")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="wall-time budget of the oracle sample (whole heads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-stages", action="store_true",
                    help="time the fp64 oracle per stage on every workload (host only) and exit")
    ap.add_argument("--combine-only", choices=["read", "write", "stream"], default=None,
                    help="time only the stand-alone combine kernel on the large workload, 40 launches, "
                         "each after a flush of L2 and MALL that reads (or writes) a 1 GiB buffer, or "
                         "(stream) back to back over four output buffers in turn, and exit (one mode per "
                         "process, so that a kernel trace of the run holds that mode's launches only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy kernel (reference for the HBM "
                         "byte counters) three times and exit")
    return ap.parse_args()


def copy_calibration():
    """A plain elementwise copy of known size: 1 GiB read, 1 GiB written per launch."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": 4 * n,
                      "copy_calibration_bytes_written_per_launch": 4 * n}), flush=True)


def combine_only(mode: str, launches: int = 40):
    """The stand-alone combine on the large workload, each launch after a
    flush of L2 and MALL: reading a 1 GiB buffer (no dirty line is left) or
    writing it (the MALL's write-back of the flush buffer then lands in the
    combine's window); or back to back over four outputs in turn ("stream").
    Prints the median duration and HBM rate."""
    import torch

    import synth
    import video_sparse_attention_amd as vsa
    dev = torch.device("cuda:0")
    inp = synth.workload("large")
    B, H, Sq, Skv, D = inp.shape
    prob = vsa.dense_problem(B, H, Sq, Skv, D, inp.topk)
    q, k, v, gate = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gate))
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    ws = vsa.alloc_workspace(prob, dev)
    vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, ws)
    out = torch.empty_like(q)
    vsa.vsa_sparse_attn_from_indices(prob, q, k, v, idx, num, out)
    times = []
    if mode == "stream":
        # four 222 MB outputs in turn (888 MB, above the 256 MB MALL): in the
        # steady state every launch's reads miss the caches and its writes
        # evict the dirty lines of earlier launches, so the write-backs fall
        # inside the launches
        outs = [out] + [out.clone() for _ in range(3)]
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        for i in range(launches):
            evs[i][0].record()
            vsa.vsa_combine(prob, out_c, gate, outs[i % 4])
            evs[i][1].record()
        torch.cuda.synchronize()
        times = [a.elapsed_time(b) for a, b in evs[8:]]
    else:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(launches):
            if mode == "read":
                flush.sum()
            else:
                flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            vsa.vsa_combine(prob, out_c, gate, out)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
    med = sorted(times)[len(times) // 2]
    nbytes = 2 * 2 * B * H * Sq * D + 2 * B * H * Sq + 4 * B * H * (-(-Sq // 64)) * D
    print(json.dumps({"combine_flush": mode, "launches": launches, "median_ms": round(med, 4),
                      "bytes": nbytes, "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
                      "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}), flush=True)


def kernel_hash(path=SPARSE_SRC) -> str:
    """Hash of the sparse kernel's source and the headers it includes."""
    h = hashlib.sha256()
    d = os.path.dirname(path)
    for p in (path, os.path.join(d, "attn_common.hpp"), os.path.join(d, "attn_layout.hpp"),
              os.path.join(d, "vsa_internal.hpp")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(launch_algo_bytes: float):
    """HBM bytes per launch of the sparse kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def pair_count(idx, num, Sq: int, Skv: int, block: int) -> int:
    """(64-token query block, 64-token KV block) pairs the sparse attention
    visits: every selected VSA block of ``block`` tokens stands for its
    64-token sub-blocks, for each 64-token query block of the VSA query block
    (for block = 64 this is B*H*nQ*k)."""
    import numpy as np
    r = block // 64
    idx, num = np.asarray(idx, dtype=np.int64), np.asarray(num, dtype=np.int64)
    nq64, nkv64 = -(-Sq // 64), -(-Skv // 64)
    nqb = idx.shape[-2]
    qsub = np.minimum(r, nq64 - r * np.arange(nqb))  # 64-token query blocks per VSA block
    used = np.arange(idx.shape[-1]) < num[..., None]
    ksub = np.clip(nkv64 - r * idx, 0, r) * used
    return int((ksub.sum(axis=-1) * qsub).sum())


def cpu_baseline(inp, budget_s: float, block: int = 64):
    """Time the fp64 oracle on whole heads of the workload until the budget is used."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    to64 = lambda t: t.to(torch.float64).numpy()
    B, H, Sq, Skv, D = inp.shape
    done, t_total, pairs = 0, 0.0, 0
    for h in range(H):
        sl = slice(h, h + 1)
        q, k, v = to64(inp.q[:, sl]), to64(inp.k[:, sl]), to64(inp.v[:, sl])
        g = None if inp.gate is None else to64(inp.gate[:, sl])
        t0 = time.perf_counter()
        r = oracle.vsa_forward(q, k, v, inp.topk, g, block=block)
        t_total += time.perf_counter() - t0
        pairs += pair_count(r["q2k_idx"], r["q2k_num"], Sq, Skv, block)
        done += 1
        if t_total >= budget_s:
            break
    flops = 4.0 * pairs * 64 * 64 * D
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {H} heads of the same workload, whole forward per head "
                      f"(pool, coarse, top-k, sparse, combine) in fp64 NumPy; "
                      f"{t_total:.1f} s; rate scaled by the same effective-FLOP formula"}


def _oracle_stage_seconds(oracle, q, k, v, gate, topk):
    """Wall seconds of the oracle's stages on one head of one sequence
    ([S, D] float64 arrays): pool + coarse + top-k, sparse, combine."""
    qs, ks = oracle.block_sizes(q.shape[0]), oracle.block_sizes(k.shape[0])
    t0 = time.perf_counter()
    qc, kc, vc = oracle.pool(q, qs), oracle.pool(k, ks), oracle.pool(v, ks)
    dots, out_c = oracle.coarse(qc, kc, vc)
    sel = [oracle.select_topk(dots[i], topk)[0] for i in range(len(qs))]
    t1 = time.perf_counter()
    rows = [oracle.sparse_block(q[64 * i: 64 * i + n], k, v, ks, sel[i]) for i, n in enumerate(qs)]
    t2 = time.perf_counter()
    for i, n in enumerate(qs):
        oracle.combine(out_c[i], rows[i], None if gate is None else gate[64 * i: 64 * i + n])
    t3 = time.perf_counter()
    return t1 - t0, t2 - t1, t3 - t2


def oracle_stages(budget_s: float):
    """Per-stage wall time of the fp64 oracle on the host cores for every
    workload: whole workloads for the three small ones (also with one BLAS
    thread), a bounded sample of heads (and sequences) for the large ones,
    scaled to the whole workload and labelled so."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import synth
    f64 = lambda t: t.float().double().numpy()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    lines = []
    for name in ("tiny", "dense_equiv", "varlen_small", "large", "varlen_many"):
        inp = synth.workload(name)
        units = []  # (q, k, v, gate, topk) per (sequence, head)
        if isinstance(inp, synth.DenseInputs):
            B, H = inp.shape[0], inp.shape[1]
            for b in range(B):
                for h in range(H):
                    g = None if inp.gate is None else f64(inp.gate[b, h])
                    units.append((inp.q[b, h], inp.k[b, h], inp.v[b, h], g, inp.topk))
        else:
            for h in range(inp.heads):
                for s, per in enumerate(inp.per_seq):
                    g = None if per["gate"] is None else f64(per["gate"][h])
                    units.append((per["q"][h], per["k"][h], per["v"][h], g, inp.topk[s]))
        small = name in ("tiny", "dense_equiv", "varlen_small")
        for nthreads in ((threads, 1) if small else (threads,)):
            with threadpool_limits(nthreads):
                tot = np.zeros(3)
                done = 0
                for (q, k, v, g, topk) in units:
                    tot += _oracle_stage_seconds(oracle, f64(q), f64(k), f64(v), g, topk)
                    done += 1
                    if not small and tot.sum() >= budget_s:
                        break
            scale = len(units) / done
            lines.append({"workload": name, "threads": nthreads, "units": len(units), "timed_units": done,
                          "extrapolated": done < len(units),
                          "seconds": {"pool_coarse_topk": round(tot[0] * scale, 4),
                                      "sparse": round(tot[1] * scale, 4),
                                      "combine": round(tot[2] * scale, 4)}})
            print(json.dumps(lines[-1]), flush=True)
    return lines


def video_bench(args, torch, synth, vsa):
    """The large shape as a video latent (11 x 32 x 44 tokens, 4 x 4 x 4 tiles,
    partial along t): one step = gather q, k, v and the gate into tile order,
    coarse stage, sparse attention with the fused combine, scatter of the
    output back to raster order."""
    dev = torch.device("cuda:0")
    grid, tile, H, D = (11, 32, 44), (4, 4, 4), 56, 128
    S = grid[0] * grid[1] * grid[2]
    n_tiles = -(-grid[0] // 4) * -(-grid[1] // 4) * -(-grid[2] // 4)
    topk = -(-n_tiles // 5)
    inp = synth.dense_inputs(1, H, S, D, topk, seed=1006, gated=True)
    q, k, v, gate = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gate))
    meta = vsa.vsa_build_tile_metadata(1, grid, topk, tile, device=dev)
    prob = meta.problem(H, D)
    slots = 64 * n_tiles
    gq, gk, gv = (torch.empty(H, slots, D, dtype=torch.bfloat16, device=dev) for _ in range(3))
    gg = torch.empty(H, slots, dtype=torch.bfloat16, device=dev)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    out_t = torch.empty(H, slots, D, dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    ws = vsa.alloc_workspace(prob, dev)

    def step(ev=None):
        if ev: ev[0].record()
        for src, dst in ((q, gq), (k, gk), (v, gv), (gate, gg)):
            vsa.tile_gather(src, grid, tile, out=dst)
        if ev: ev[1].record()
        vsa.vsa_coarse_topk(prob, gq, gk, gv, out_c, idx, num, ws)
        if ev: ev[2].record()
        vsa.vsa_sparse_attn_combine(prob, gq, gk, gv, idx, num, out_c, gg, out_t)
        if ev: ev[3].record()
        vsa.tile_scatter(out_t, grid, 1, tile, out=out)
        if ev: ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("gather", "coarse", "sparse", "scatter")
    avg = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, n in enumerate(names)}
    ms_per_step = wall * 1e3 / args.steps
    flops = 4.0 * H * n_tiles * topk * 64 * 64 * D
    sparse_tf = flops / (avg["sparse"] * 1e-3) / 1e12
    gather_bytes = 3 * (2 * H * S * D + 2 * H * slots * D) + 2 * H * S + 2 * H * slots
    scatter_bytes = 2 * H * S * D * 2
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"video latent {grid[0]}x{grid[1]}x{grid[2]} = {S} tokens in 4x4x4 tiles "
                               f"({n_tiles} tiles, partial along t), H={H} D={D}, top-{topk}, token gate; "
                               "gather + forward + scatter",
                   "heads": H, "head_dim": D, "grid": list(grid), "tile": list(tile), "topk": topk,
                   "gate": "token"},
        "roofline": {"bound": "mfma", "kernel": "sparse_attn_kernel<128, 1>", "achieved": round(sparse_tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(sparse_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(avg["sparse"], 4), "flops_per_launch": flops},
        "kernels": {"tile_gather_ms": round(avg["gather"], 4),
                    "tile_gather_GBps": round(gather_bytes / (avg["gather"] * 1e-3) / 1e9, 1),
                    "coarse_topk_stage_ms": round(avg["coarse"], 4),
                    "sparse_attn_combine_ms": round(avg["sparse"], 4),
                    "tile_scatter_ms": round(avg["scatter"], 4),
                    "tile_scatter_GBps": round(scatter_bytes / (avg["scatter"] * 1e-3) / 1e9, 1)},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def train_bench(args, torch, synth, vsa):
    """Training step on the large shape (B=1, H=56, D=128, S=15488, top-49,
    per-token gate): coarse/top-k, the training forward (sparse attention
    with the fused combine, also writing out_s and lse) and the backward
    (vsa_backward_pooled: the block means of q, k and v come from the coarse
    stage's workspace, as in the autograd wrapper) for a fixed output gradient.  Effective FLOPs: the forward's
    4 B H nQ k 64^2 D plus 2.5 times that for the backward (dV, dP, dQ, dK and
    the recomputed scores: five block products where the forward has two)."""
    dev = torch.device("cuda:0")
    inp = synth.workload("large")
    B, H, Sq, Skv, D = inp.shape
    prob = vsa.dense_problem(B, H, Sq, Skv, D, inp.topk)
    nq = -(-Sq // 64)
    kk = min(inp.topk, -(-Skv // 64))
    fwd_flops = 4.0 * B * H * nq * kk * 64 * 64 * D
    bwd_flops = 2.5 * fwd_flops
    q, k, v, gate = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.gate))
    dout = synth.output_grad(inp.q.shape, 1100).to(dev)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    out, out_s = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(vsa.lse_shape(prob), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty_like(gate)
    ws = vsa.alloc_workspace(prob, dev)
    bws = vsa.alloc_backward_workspace(prob, dev)

    def step(ev=None):
        if ev: ev[0].record()
        vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, ws)
        if ev: ev[1].record()
        vsa.vsa_sparse_attn_combine_train(prob, q, k, v, idx, num, out_c, gate, out, out_s, lse)
        if ev: ev[2].record()
        vsa.vsa_backward(prob, q, k, v, idx, num, out_c, gate, out_s, lse, dout, dq, dk, dv, dg, bws,
                         forward_workspace=ws)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("coarse", "forward", "backward")
    avg = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, n in enumerate(names)}
    ms_per_step = wall * 1e3 / args.steps
    bwd_tf = bwd_flops / (avg["backward"] * 1e-3) / 1e12
    res = {
        "metric": "VSA training step (fwd+bwd) effective TFLOP/s",
        "value": round((fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"large video-DiT shape B={B} H={H} D={D} S={Sq}, top-{inp.topk}, token gate; "
                               "coarse + training forward + backward",
                   "batch": B, "heads": H, "head_dim": D, "seq_len": Sq, "topk": inp.topk, "gate": "token"},
        "kernels": {"coarse_topk_stage_ms": round(avg["coarse"], 4),
                    "forward_train_ms": round(avg["forward"], 4),
                    "forward_train_TFLOPs": round(fwd_flops / (avg["forward"] * 1e-3) / 1e12, 2),
                    "backward_ms": round(avg["backward"], 4),
                    "backward_TFLOPs": round(bwd_tf, 2),
                    "backward_frac_bf16_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the forward "
              "is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.combine_only:
        combine_only(args.combine_only)
        return
    if args.oracle_stages:
        oracle_stages(args.cpu_budget_s)
        return

    import torch

    import synth
    import video_sparse_attention_amd as vsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "video":
        video_bench(args, torch, synth, vsa)
        return
    if args.workload == "train":
        train_bench(args, torch, synth, vsa)
        return
    inp = synth.workload(args.workload)
    block = args.block_size
    if block != 64 and args.workload not in ("large", "varlen_many"):
        print("--block-size applies to the large and varlen_many workloads only", file=sys.stderr)
        sys.exit(2)

    flops = None
    if isinstance(inp, synth.DenseInputs):
        B, H, Sq, Skv, D = inp.shape
        nqb = -(-Sq // block)
        if block != 64:
            inp.topk = math.ceil(0.20 * -(-Skv // block))  # about 20 % of the VSA blocks
        prob = vsa.dense_problem(B, H, Sq, Skv, D, inp.topk, block)
        q_tokens = B * H * Sq
        n_qblocks = B * H * nqb
        n_kvblocks = B * H * -(-Skv // block)
        gated = inp.gate is not None
        what = "large video-DiT shape" if args.workload == "large" else "the pages' benchmark-command shape"
        cfg = {"workload": f"{what} B={B} H={H} D={D} S={Sq} ({nqb} blocks of {block}), "
                           f"top-{inp.topk}, " + ("per-token-per-head sigmoid gate" if gated else "ungated"),
               "batch": B, "heads": H, "head_dim": D, "seq_len": Sq, "block": block,
               "topk": inp.topk, "gate": "token" if gated else "none"}
    else:
        if block != 64:  # the same sequences in VSA blocks of 128 / 256 slots, top-k 20 % of them
            inp = synth.workload(args.workload, block=block)
        meta = vsa.vsa_build_metadata(inp.seqlens_q, inp.seqlens_kv, inp.topk, device=dev, block_size=block)
        H, D = inp.heads, inp.head_dim
        prob = meta.problem(H, D)
        tk = meta.topk.tolist()
        nqs = [-(-s // block) for s in inp.seqlens_q]
        # every sequence is a whole number of VSA blocks here: each selected
        # block stands for block / 64 full 64-token KV blocks, for each of the
        # block / 64 query blocks of a VSA query block
        r = block // 64
        flops = 4.0 * H * sum(n * k * r * r for n, k in zip(nqs, tk)) * 64 * 64 * D
        q_tokens = H * sum(inp.seqlens_q)
        n_qblocks = H * sum(nqs)
        n_kvblocks = H * sum(-(-s // block) for s in inp.seqlens_kv)
        cfg = {"workload": f"{len(nqs)} packed sequences, Q blocks {nqs} of {block} tokens, "
                           f"KV = Q + {512 // block} blocks, H={H} D={D}, top-k {tk}, gated",
               "heads": H, "head_dim": D, "block": block, "topk": tk, "gate": "token"}

    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    gate = None if inp.gate is None else inp.gate.to(dev)
    cs, isz, ns = vsa.block_shapes(prob)
    out_c = torch.empty(cs, dtype=torch.float32, device=dev)
    idx = torch.empty(isz, dtype=torch.int32, device=dev)
    num = torch.empty(ns, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = vsa.alloc_workspace(prob, dev)

    def step(ev=None):
        if ev: ev[0].record()
        vsa.vsa_coarse_topk(prob, q, k, v, out_c, idx, num, ws)
        if ev: ev[1].record()
        vsa.vsa_sparse_attn_combine(prob, q, k, v, idx, num, out_c, gate, out)
        if ev: ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if flops is None:  # effective flops of the routing the kernels produce (identical every step)
        flops = 4.0 * pair_count(idx.cpu().numpy(), num.cpu().numpy(), Sq, Skv, block) * 64 * 64 * D

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    st = {"coarse": 0.0, "sparse": 0.0}
    for e in evs:
        st["coarse"] += e[0].elapsed_time(e[1])
        st["sparse"] += e[1].elapsed_time(e[2])
    avg = {key: val / args.steps for key, val in st.items()}  # ms
    ms_per_step = wall * 1e3 / args.steps

    # Outside the timed steps: the stand-alone combine kernel (the pages'
    # separate combine) with L2 and MALL flushed before each launch, and the
    # sparse kernel without the fused combine.  The flush reads a 1 GiB
    # buffer: afterwards neither cache holds any of the combine's data and no
    # dirty line of earlier writes is left to be written back during the
    # timed launch.  The same launch after a flush that WRITES 1 GiB is also
    # reported: there the MALL's write-back of 256 MB of the flush buffer's
    # dirty lines lands inside the combine's window.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    comb_ms, comb_dirty_ms, unf_ms = [], [], []
    for rep in range(40):
        if rep % 2 == 0:
            flush.sum()
        else:
            flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        vsa.vsa_combine(prob, out_c, gate, out)
        e1.record()
        torch.cuda.synchronize()
        (comb_ms if rep % 2 == 0 else comb_dirty_ms).append(e0.elapsed_time(e1))
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        vsa.vsa_sparse_attn_from_indices(prob, q, k, v, idx, num, out)
        e1.record()
        torch.cuda.synchronize()
        unf_ms.append(e0.elapsed_time(e1))
    del flush
    comb = sorted(comb_ms)[len(comb_ms) // 2]
    comb_dirty = sorted(comb_dirty_ms)[len(comb_dirty_ms) // 2]
    unf = sorted(unf_ms)[len(unf_ms) // 2]

    # algorithmic bytes: the combine reads and writes out once, reads the gate and out_c
    gate_bytes = 0 if gate is None else 2 * q_tokens
    comb_bytes = 2 * 2 * q_tokens * D + gate_bytes + 4 * n_qblocks * D
    coarse_bytes = 2 * (q.numel() + 2 * k.numel()) + 8 * D * (n_qblocks + 2 * n_kvblocks)
    sparse_tf = flops / (avg["sparse"] * 1e-3) / 1e12
    traffic = measured_traffic(None) if (args.workload == "large" and block == 64) else None
    kname = "sparse_attn_kernel<128, 1, 1>" if gate is not None else "sparse_attn_kernel<128, 0, 1>"
    if block != 64:
        kname = kname.replace(", 1>", ", 2>")  # one workgroup per pair of 64-token query blocks

    res = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": cfg,
        "roofline": {
            "bound": "mfma",
            "kernel": kname + " (block-sparse attention with the combine fused)",
            "achieved": round(sparse_tf, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(sparse_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(avg["sparse"], 4),
            "flops_per_launch": flops,
        },
        "kernels": {
            "coarse_topk_stage_ms": round(avg["coarse"], 4),
            "coarse_topk_stage_GBps": round(coarse_bytes / (avg["coarse"] * 1e-3) / 1e9, 1),
            "sparse_attn_combine_ms": round(avg["sparse"], 4),
            "sparse_attn_combine_TFLOPs": round(sparse_tf, 2),
            "sparse_attn_unfused_ms": round(unf, 4),
            "combine_standalone_cold_ms": round(comb, 4),
            "combine_standalone_GBps": round(comb_bytes / (comb * 1e-3) / 1e9, 1),
            "combine_standalone_frac_hbm": round(comb_bytes / (comb * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "combine_after_write_flush_ms": round(comb_dirty, 4),
            "combine_after_write_flush_GBps": round(comb_bytes / (comb_dirty * 1e-3) / 1e9, 1),
            "combine_bytes": comb_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and isinstance(inp, synth.DenseInputs):
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s, block)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

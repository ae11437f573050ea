#!/usr/bin/env python3
"""Benchmark of the FlashBlock attention step on one MI355X.

One bench step is one block of S denoising steps of one attention layer, all
batch streams and heads: the refresh step runs the split-KV prefix pass, the
split combine into the fp32 cache, and the fused in-block attention + LSE
merge; the other steps run only the fused in-block + merge kernel.  Inputs
(prefix KV cache, every step's block Q/K/V) are resident in HBM before the
timed region; consecutive bench steps rotate over three copies of the prefix
KV cache (like consecutive layers), so no pass finds the prefix in the 256 MB
Infinity Cache.

value = query tokens per second in cached mode with refresh period r
      = B * Lb * S * n_blocks / (time of one bench step).
The same line reports full recompute (the standard per-step attention over the
whole KV cache), the cached-vs-full speedup, per-step latencies, the
cached-vs-recompute drift, the prefix kernel against the HBM roofline, and the
fp64 oracle timed on the host cores as a baseline.

The default workload is the long-context GQA text layer (32 query / 8 KV
heads, head_dim 128, 64-token block, 128K-token prefix, 8 steps, r = 8).  The
roofline object covers the prefix pass: the split-KV kernel (K1) and the split
combine (K2) together, timed back to back on the launch stream; K1 alone is
reported beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--r R]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn-step latency & query-tok/s, cached vs full recompute; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
N_LAYERS = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


LIBRARY_SOURCES = ("fb_kernels.hip", "fb_api.cpp", "fb_internal.h")


def library_source_sha(root=None):
    """First 16 hex digits of the sha256 over the library's sources: the kernels,
    and the host planner and shared header that pick each pass's configuration.
    None if one is missing."""
    here = root or os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for name in LIBRARY_SOURCES:
        path = os.path.join(here, "cached_attention_amd", "csrc", name)
        if not os.path.exists(path):
            return None
        h.update(name.encode() + b"\0" + open(path, "rb").read() + b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload, pass_name="prefix"):
    """HBM bytes per launch of one pass from profiles/hbm_traffic.md, or None.

    The table has one row per kernel of a pass (the prefix pass: the split-KV
    kernel and the split combine), with the hash of the library sources the
    counters were taken with (library_source_sha); rows only count while the
    sources still hash the same.  Returns the sum over the pass's rows.
    """
    here = os.path.dirname(os.path.abspath(__file__))
    table = os.path.join(here, "profiles", "hbm_traffic.md")
    sha = library_source_sha(here)
    if not os.path.exists(table) or sha is None:
        return None
    total, rows = 0.0, 0
    for line in open(table):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] == workload and cells[1] == pass_name and cells[2] == sha:
            total += float(cells[6])
            rows += 1
    return total if rows else None


def smi_snapshot():
    """Socket power and clocks of GPU 0 from `amd-smi metric` (a child process), or None."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    try:
        out = subprocess.run([exe, "metric", "-g", "0", "--power", "--clock", "--json"], capture_output=True,
                             text=True, timeout=30).stdout
        d = json.loads(out[out.index("{"):])
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = g["clock"]
        gfx = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_") and isinstance(clk[k], dict)]
        return {"socket_power_w": g["power"]["socket_power"]["value"], "gfx_clk_mhz": gfx,
                "gfx_clk_max_mhz": clk["gfx_0"]["max_clk"]["value"], "mem_clk_mhz": clk["mem_0"]["clk"]["value"]}
    except Exception:
        return None


def snapshot_under_load(fn, sync, seconds=3.0, lead=1.0):
    """amd-smi snapshot started `lead` seconds into a run of fn back to back
    (untimed), which lasts at least `seconds` and until the snapshot returns."""
    import threading
    res = {}
    t = threading.Thread(target=lambda: res.update(snap=smi_snapshot()))
    t0 = time.perf_counter()
    started = False
    while not started or t.is_alive() or time.perf_counter() < t0 + seconds:
        for _ in range(10):
            fn()
        sync()
        if not started and time.perf_counter() >= t0 + lead:
            t.start()
            started = True
    t.join()
    return res.get("snap")


def algorithmic(w, lens, sparse_tokens=None):
    """Algorithmic bytes / flops of the prefix pass and of the in-block + merge pass."""
    e = 2 if w.dtype == "bf16" else 4
    tok = sum(lens) if sparse_tokens is None else sparse_tokens
    prefix_bytes = (2 * tok * w.hkv * w.head_dim * e + w.batch * w.block_len * w.hq * w.head_dim * e
                    + w.batch * w.hq * w.block_len * (w.head_dim + 1) * 4)
    prefix_flops = 4 * w.hq * w.block_len * w.head_dim * tok
    block_bytes = (w.batch * w.block_len * w.head_dim * e * (w.hq + 2 * w.hkv)
                   + w.batch * w.hq * w.block_len * (w.head_dim + 1) * 4
                   + w.batch * w.block_len * w.hq * w.head_dim * e)
    block_flops = 4 * w.batch * w.hq * w.block_len ** 2 * w.head_dim
    return prefix_bytes, prefix_flops, block_bytes, block_flops


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def cpu_baseline(w, prefix, blocks, r, budget_s=12.0, variant="fixed", k_sel=0, tau=0, eps=0.0, gamma=0.0):
    """The fp64 oracle (as it stands) on the same workload's first block, in
    the variant the GPU runs (fixed-period cached, sparse with the oracle's own
    chunk selection at the block's first step, or an adaptive reuse policy), on
    the host cores; repeated until ~budget_s of CPU work.  Full recompute is
    sampled as the block's first step alone (every full step costs the same),
    scaled to the block's steps."""
    import oracle
    scale = 1.0 / math.sqrt(w.head_dim)
    blk = blocks[0]

    def one_block():
        if variant == "sparse":
            chunks = oracle.select_chunks(blk.q[0], prefix.k, prefix.offsets, k_sel, 64)
            oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, scale, r=r, chunks=chunks)
        elif variant in ("tau", "gamma"):
            oracle.run_block_policy(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, scale, variant,
                                    tau=tau, eps=eps, gamma=gamma)
        else:
            oracle.run_block(prefix.k, prefix.v, prefix.offsets, blk.q, blk.k, blk.v, scale, r=r)

    t0 = time.perf_counter()
    runs = 0
    while True:
        one_block()
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 100:
            break
    per_block = el / runs
    t1 = time.perf_counter()
    oracle.full_step(blk.q[0], blk.k[0], blk.v[0], prefix.k, prefix.v, prefix.offsets, scale)
    full_step_s = time.perf_counter() - t1
    tok = w.batch * w.block_len * w.steps
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {
        "value": tok / per_block,
        "unit": "query-tok/s",
        "cores": blas_threads(),
        "cpu_count": os.cpu_count(),
        "sched_affinity": affinity,
        "threads": {"blas": blas_threads(), "elementwise": 1,
                    "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
                    "OPENBLAS_NUM_THREADS": os.environ.get("OPENBLAS_NUM_THREADS")},
        "kind": "oracle",
        "sample": f"{runs} x first block of {w.name} ({w.steps} steps, {variant}, r={r}, all streams and heads), "
                  f"numpy fp64, {el:.1f} s; full recompute: the block's first step ({full_step_s:.1f} s) "
                  f"x {w.steps} steps; cores = BLAS threads, elementwise work single-threaded",
        "ms_per_block": per_block * 1e3,
        "full_recompute": {"value": tok / (full_step_s * w.steps), "unit": "query-tok/s",
                           "ms_per_block": full_step_s * w.steps * 1e3},
        "speedup_vs_full": full_step_s * w.steps / per_block,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30, help="timed bench steps (blocks)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="text_gqa_128k")
    ap.add_argument("--r", type=int, default=8)
    ap.add_argument("--kv-layout", choices=("head", "token", "interleave"), default="head",
                    help="prefix KV cache layout: head-major [Hkv][T][D], token-major [T][Hkv][D], or head-major "
                         "with each token's K and V rows adjacent [Hkv][T][2][D]")
    ap.add_argument("--sparse", action="store_true",
                    help="chunk-sparse variant: cached residual of the unselected 64-token chunks plus a fresh "
                         "partial over the selected ones (workloads with a sparse keep fraction)")
    ap.add_argument("--density", type=float, default=0.0,
                    help="sparse variant: fraction of 64-token chunks kept (default: the workload's, 10%%)")
    ap.add_argument("--chunk-select", choices=("topk", "random"), default="topk",
                    help="sparse variant: chunks chosen on the GPU from each block's first-step queries "
                         "(pooled chunk keys, max query score, top-k), or a fixed seeded random stand-in")
    ap.add_argument("--policy", choices=("fixed", "tau", "gamma"), default="fixed",
                    help="refresh policy: fixed period r, or adaptive reuse on decoding-style block steps "
                         "(tau: updated-token threshold; gamma: per-head query similarity)")
    ap.add_argument("--tau", type=int, default=0, help="tau policy: recompute iff >= tau tokens updated "
                    "(default: a quarter of the block)")
    ap.add_argument("--eps", type=float, default=0.25, help="tau policy: a token is updated if its K or V "
                    "changed by more than eps")
    ap.add_argument("--gamma", type=float, default=0.99, help="gamma policy: a head reuses its cache iff "
                    "its query similarity exceeds gamma")
    ap.add_argument("--prefix-len", type=int, default=0,
                    help="override the workload's prefix length (tokens per stream), e.g. a 128K -> 800K sweep")
    ap.add_argument("--graph", action="store_true",
                    help="time whole bench steps as replays of captured HIP graphs (one per KV-cache copy), so "
                         "the host's launch overhead stays out; per-step latencies stay eager")
    ap.add_argument("--sustain-s", type=float, default=1.5,
                    help="seconds of alternating prefix-pass batches (K1 alone, K1 + K2) behind the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gpu-state", action="store_true",
                    help="skip the amd-smi power and clock snapshots (and the extra full-recompute steps "
                         "that run under the second one), e.g. under a profiler")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (to scale FETCH_SIZE / WRITE_SIZE "
                         "counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU (asked for {max(args.gpus, world)}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from cached_attention_amd import flashblock as fbl
    from cached_attention_amd import workloads as wl
    from cached_attention_amd.session import AttentionStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    fbl.lib()   # fails loudly when the HIP library is not built
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return 0
    w = wl.WORKLOADS[args.workload]
    if args.prefix_len > 0:
        w = dataclasses.replace(w, name=f"{w.name}@{args.prefix_len}", prefix_len=args.prefix_len)
    if args.density > 0:
        if not 0 < args.density <= 1 or not args.sparse:
            print("--density takes a fraction in (0, 1] with --sparse", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, name=f"{w.name}~{args.density:g}", sparse_keep=args.density)
    r = args.r
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    log(f"[bench] workload {w.name}: B={w.batch} Hq={w.hq} Hkv={w.hkv} D={w.head_dim} Lb={w.block_len} "
        f"Lp={w.prefix_len} S={w.steps} blocks={w.n_blocks} r={r}")
    t_gen = time.perf_counter()
    if args.policy == "fixed":
        prefix, blocks = wl.make_inputs(w)
    else:   # decoding-style steps: abrupt reveals (tau) or per-head drift (gamma)
        if args.sparse:
            print("adaptive reuse policies run on the dense prefix", file=sys.stderr)
            return 2
        rng = np.random.default_rng(w.seed)
        prefix = wl.make_prefix(w, rng)
        blocks = [wl.make_block_steps_decoding(w, rng, 0.9 if args.policy == "gamma" else 0.0,
                                               reveal=args.policy == "tau") for _ in range(w.n_blocks)]
        if args.tau <= 0:
            args.tau = max(1, w.block_len // 4)
    log(f"[bench] inputs drawn in {time.perf_counter() - t_gen:.1f} s")

    # per-block prefix: blocks after the first see the earlier blocks' final K/V appended
    block_prefix = []
    kp_np, vp_np, off = prefix.k, prefix.v, prefix.offsets
    for j, blk in enumerate(blocks):
        block_prefix.append((kp_np, vp_np, off))
        if j + 1 < len(blocks):
            ks, vs = [], []
            new_off = np.zeros_like(off)
            for b in range(w.batch):
                t0, t1 = int(off[b]), int(off[b + 1])
                ks += [kp_np[t0:t1], blk.k[-1][b]]
                vs += [vp_np[t0:t1], blk.v[-1][b]]
                new_off[b + 1] = new_off[b] + (t1 - t0) + w.block_len
            kp_np, vp_np, off = np.concatenate(ks), np.concatenate(vs), new_off

    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", tdt)
    head_major = args.kv_layout == "head"
    # head-major keeps each KV head's keys contiguous: a 64-key tile is one 16 KB run
    dev_kv = (lambda x: dev(np.transpose(x, (1, 0, 2)))) if head_major else dev

    def interleaved(kp, vp):
        """[Hkv][T][2][D]: each token's K and V rows adjacent; K and V are strided views."""
        il = dev(np.stack([np.transpose(kp, (1, 0, 2)), np.transpose(vp, (1, 0, 2))], axis=2))
        return il[:, :, 0, :], il[:, :, 1, :]

    layers = []   # N_LAYERS copies of each block's prefix
    pre_strides = []
    for j in range(len(blocks)):
        kp, vp, _ = block_prefix[j]
        t_tot = kp.shape[0]
        if args.kv_layout == "interleave":
            pre_strides.append((2 * w.head_dim, 2 * t_tot * w.head_dim))
            layers.append([interleaved(kp, vp) for _ in range(N_LAYERS)])
            continue
        pre_strides.append((w.head_dim, t_tot * w.head_dim) if head_major else (w.hkv * w.head_dim, w.head_dim))
        k0, v0 = dev_kv(kp), dev_kv(vp)
        layers.append([(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(N_LAYERS - 1)])
    steps_dev = [[(dev(b.q[s]), dev(b.k[s]), dev(b.v[s])) for s in range(w.steps)] for b in blocks]
    chunks = None
    if args.sparse:
        if w.sparse_keep <= 0:
            print(f"workload {w.name} has no sparse variant", file=sys.stderr)
            return 2
        lens0 = [int(prefix.offsets[b + 1] - prefix.offsets[b]) for b in range(w.batch)]
        chunks = torch.from_numpy(wl.make_chunk_selection(w, lens0))
    states = [AttentionStep(w.dtype, w.batch, w.hq, w.hkv, w.head_dim, w.block_len, block_prefix[j][2],
                            pre_strides=pre_strides[j], chunks=chunks)
              for j in range(len(blocks))]
    topk = args.sparse and args.chunk_select == "topk"
    k_sel = int(chunks.shape[-1]) if args.sparse else 0
    if topk:
        # pooled chunk keys are per-layer state like the KV cache: full chunks of
        # the append-only prefix never change, so a block pools only the chunks
        # from the first one its predecessor's append touched (block 0: the
        # steady state after the previous block's append)
        blk_lens = [[int(o[b + 1] - o[b]) for b in range(w.batch)] for (_, _, o) in block_prefix]
        cap = max(-(-l // 64) for l in blk_lens[-1])
        first = [max(0, min(blk_lens[0]) - w.block_len) // 64] + [min(blk_lens[j - 1]) // 64
                                                                   for j in range(1, len(blocks))]
        pooled = [torch.empty(w.batch, cap, w.hkv, w.head_dim, device="cuda") for _ in range(N_LAYERS)]
        scores_buf = torch.empty(w.batch, w.hkv, cap, device="cuda")
        for layer in range(N_LAYERS):
            fbl.fb_pool_chunk_keys(states[0].desc, layers[0][layer][0], 64, cap, 0, pooled[layer])
        sel_ws = torch.empty(fbl.fb_select_chunks_ws(states[0].desc, 64), dtype=torch.uint8, device="cuda")

    def select(j, q, layer):
        """Top-k chunks of block j from its first-step queries, into the state's chunk list."""
        fbl.fb_pool_chunk_keys(states[j].desc, layers[j][layer][0], 64, cap, first[j], pooled[layer])
        fbl.fb_select_chunks_pooled(states[j].desc, q, pooled[layer], 64, cap, k_sel, scores_buf, states[j].chunks)

    torch.cuda.synchronize()

    counter = [0]

    def bench_step(mode, rr, layer=None):
        if layer is None:
            layer = counter[0] % N_LAYERS
            counter[0] += 1
        for j, st in enumerate(states):
            kp, vp = layers[j][layer]
            for s in range(w.steps):
                q, k, v = steps_dev[j][s]
                if topk and s == 0:
                    select(j, q, layer)
                if mode == "cached" and args.policy != "fixed":
                    _, kprev, vprev = steps_dev[j][max(s - 1, 0)]
                    st.step_policy(q, k, v, kprev, vprev, kp, vp, s, args.policy, args.tau, args.eps, args.gamma,
                                   want_lse=False)
                else:
                    st.step(q, k, v, kp, vp, s, rr, mode, want_lse=False)

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n   # ms

    def sustained(fns, seconds, batch=10):
        """Average device time per call (ms) of each fn, measured in alternating
        batches of `batch` back-to-back calls for about `seconds`; each batch
        between two HIP events on the launch stream, the first quarter dropped."""
        times = [[] for _ in fns]
        pending = []
        t_end = time.perf_counter() + seconds
        i = 0
        while time.perf_counter() < t_end or i < 8 * len(fns):
            k = i % len(fns)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(batch):
                fns[k]()
            e1.record()
            pending.append((k, e0, e1))
            i += 1
            if len(pending) >= 16:   # keep the host within a few batches of the GPU
                torch.cuda.synchronize()
                for kk, a, b in pending:
                    times[kk].append(a.elapsed_time(b) / batch)
                pending = []
        torch.cuda.synchronize()
        for kk, a, b in pending:
            times[kk].append(a.elapsed_time(b) / batch)
        return [float(np.mean(t[len(t) // 4:])) for t in times]

    def timed_graph(fn, n, reps=10):
        """Device time per call of fn (ms): n back-to-back calls captured in one
        graph, replayed reps times, so host launch overhead stays out of short
        kernels.  The library only launches kernels (no memset, no allocation)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        ms = timed(g.replay, reps) / n
        del g
        return ms

    def graph_steps(mode, rr):
        """One captured graph per KV-cache copy of a whole bench step; replays
        rotate over them like the eager steps.  Every launch of the library is a
        kernel (no memset, no allocation, no host synchronisation)."""
        graphs = []
        for layer in range(N_LAYERS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                bench_step(mode, rr, layer)
            graphs.append(g)
        turn = [0]

        def replay():
            graphs[turn[0] % N_LAYERS].replay()
            turn[0] += 1
        return replay

    gpu_idle = None if args.no_gpu_state else smi_snapshot()
    # ---- whole bench steps: cached (r) and full recompute ----
    for _ in range(args.warmup):
        bench_step("cached", r)
    cached_step = graph_steps("cached", r) if args.graph else (lambda: bench_step("cached", r))
    for _ in range(2 if args.graph else 0):
        cached_step()
    ms_cached = timed(cached_step, args.steps)
    for _ in range(max(1, args.warmup // 2)):
        bench_step("full", 1)
    full_step = graph_steps("full", 1) if args.graph else (lambda: bench_step("full", 1))
    for _ in range(2 if args.graph else 0):
        full_step()
    ms_full = timed(full_step, args.steps)
    q_tokens = w.batch * w.block_len * w.steps * len(blocks)
    gpu_load = (None if args.no_gpu_state
                else snapshot_under_load(lambda: bench_step("full", 1), torch.cuda.synchronize))

    # ---- per-step latency: refresh vs reuse steps (first block) ----
    st0 = states[0]
    lat = {"refresh": [], "reuse": []}
    n_rep = max(20, args.steps // 2)   # >= 20 refresh steps (one per block pass)
    recomputed = []   # policy mode: fraction of (stream, KV head) partials recomputed per step
    for rep in range(n_rep):
        kp, vp = layers[0][rep % N_LAYERS]
        for s in range(w.steps):
            q, k, v = steps_dev[0][s]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if topk and s == 0:
                select(0, q, rep % N_LAYERS)
            if args.policy == "fixed":
                refreshed = st0.step(q, k, v, kp, vp, s, r, "cached", want_lse=False)
            else:
                _, kprev, vprev = steps_dev[0][max(s - 1, 0)]
                st0.step_policy(q, k, v, kprev, vprev, kp, vp, s, args.policy, args.tau, args.eps, args.gamma,
                                want_lse=False)
            e1.record()
            torch.cuda.synchronize()
            if args.policy != "fixed":
                frac = float(st0.mask.float().mean())
                refreshed = frac > 0
                if rep == 0:
                    recomputed.append(frac)
            lat["refresh" if refreshed else "reuse"].append(e0.elapsed_time(e1) * 1e3)
    med = lambda xs: float(np.median(xs)) if xs else None
    pct = lambda xs, q: float(np.percentile(xs, q)) if xs else None

    # ---- the dominant pass alone: split-KV prefix kernel (fb_prefix_partials,
    # K1) + split combine into the fp32 cache (fb_prefix_combine, K2) ----
    q0 = steps_dev[0][0][0]
    n_k = max(20, args.steps)
    rot = [0]

    sel = None
    if args.sparse:   # the prefix work of every step: the selected chunks
        sel = fbl.Sparse(st0.chunks, int(st0.chunks.shape[-1]), 64, fbl.FB_CHUNKS_SELECTED)

    def prefix_kernel():
        kp, vp = layers[0][rot[0] % N_LAYERS]
        rot[0] += 1
        fbl.fb_prefix_partials(st0.desc, q0, kp, vp, sel, st0.ws, st0.ws_bytes)

    def combine():
        fbl.fb_prefix_combine(st0.desc, sel, None, None, st0.o_ext, st0.lse_ext, st0.ws, st0.ws_bytes)

    def prefix_pass():
        prefix_kernel()
        combine()

    for _ in range(3):
        prefix_pass()
    # K1 alone and K1 + K2 in alternating batches, so both see the same clock:
    # a long pass drives the board to its power cap, where the GFX clock
    # settles well below its peak within a few ms.  The first quarter of the
    # batches (clock still moving) is dropped.
    ms_prefix_kernel, ms_prefix_pass = sustained([prefix_kernel, prefix_pass], seconds=args.sustain_s)
    ms_combine = timed_graph(combine, n_k)
    qb, kb, vb = steps_dev[0][1]
    ms_block = timed_graph(lambda: fbl.fb_block_attn(st0.desc, qb, kb, vb, st0.o_ext, st0.lse_ext, st0.o), n_k)
    ms_select = ms_select_full = None
    if topk:
        sel_rot = [0]

        def select_rot():
            select(0, q0, sel_rot[0] % N_LAYERS)
            sel_rot[0] += 1

        ms_select = timed(select_rot, n_k)
        ms_select_full = timed(lambda: fbl.fb_select_chunks(st0.desc, q0, layers[0][0][0], 64, k_sel, st0.chunks,
                                                            sel_ws, sel_ws.numel()), n_k)
    # one refresh step (s = 0) and one reuse step (s = 1) of the first stream
    # set, each replayed from a graph: device time without host launch gaps.
    # A gamma step rewrites its reference queries, so a replayed step 1 would
    # not repeat itself; it is not timed this way.
    step_graph = None
    if args.policy != "gamma":
        kp1, vp1 = layers[0][0]

        def one_step(s):
            q, k, v = steps_dev[0][s]
            if args.policy == "fixed":
                st0.step(q, k, v, kp1, vp1, s, r, "cached", want_lse=False)
            else:
                _, kprev, vprev = steps_dev[0][max(s - 1, 0)]
                st0.step_policy(q, k, v, kprev, vprev, kp1, vp1, s, args.policy, args.tau, args.eps, args.gamma,
                                want_lse=False)

        if w.steps > 1 and r > 1:
            step_graph = {"refresh_step": timed_graph(lambda: one_step(0), n_k) * 1e3}
            if topk:
                select(0, steps_dev[0][0][0], 0)
            one_step(0)
            step_graph["reuse_step"] = timed_graph(lambda: one_step(1), n_k) * 1e3
            if args.policy != "fixed":
                torch.cuda.synchronize()
                step_graph["reuse_step_recompute_fraction"] = float(st0.mask.float().mean())
    tiny = torch.zeros(8, 128, device="cuda")
    tiny_l = torch.zeros(8, device="cuda")
    ms_floor = timed(lambda: fbl.fb_merge(4, 128, tiny, tiny_l, tiny, tiny_l, tiny, tiny_l), 200)

    # ---- drift: cached (r) vs full recompute, same inputs, first block ----
    kp, vp = layers[0][0]
    drift = []
    full_o = []
    for s in range(w.steps):
        q, k, v = steps_dev[0][s]
        st0.step(q, k, v, kp, vp, s, 1, "full", want_lse=False)
        full_o.append(st0.o.float().clone())
    for s in range(w.steps):
        q, k, v = steps_dev[0][s]
        if topk and s == 0:
            select(0, q, 0)
        if args.policy == "fixed":
            st0.step(q, k, v, kp, vp, s, r, "cached", want_lse=False)
        else:
            _, kprev, vprev = steps_dev[0][max(s - 1, 0)]
            st0.step_policy(q, k, v, kprev, vprev, kp, vp, s, args.policy, args.tau, args.eps, args.gamma,
                            want_lse=False)
        drift.append(float((st0.o.float() - full_o[s]).abs().max()))

    sparse_only_drift = None
    if args.sparse:   # context: the selected chunks alone, without the cached residual
        o_sel = torch.empty_like(st0.o_ext)
        l_sel = torch.empty_like(st0.lse_ext)
        o_so = torch.empty_like(st0.o)
        sparse_only_drift = []
        for s in range(w.steps):
            q, k, v = steps_dev[0][s]
            fbl.fb_prefix_attn(st0.desc, q, kp, vp, sel, o_sel, l_sel, st0.ws, st0.ws_bytes)
            fbl.fb_block_attn(st0.desc, q, k, v, o_sel, l_sel, o_so)
            sparse_only_drift.append(float((o_so.float() - full_o[s]).abs().max()))

    lens = block_prefix[0][2]
    lens = [int(lens[b + 1] - lens[b]) for b in range(w.batch)]
    sparse_tokens = None
    if args.sparse:
        sparse_tokens = sum(min(64 * k_sel, l) for l in lens)   # selected keys per KV head, all streams
    pb, pf, bb, bf = algorithmic(w, lens, sparse_tokens)
    # the pass (K1 + K2) is what the roofline reports; K1 alone sits beside it
    prefix_gbs = pb / (ms_prefix_pass * 1e-3) / 1e9
    prefix_tflops = pf / (ms_prefix_pass * 1e-3) / 1e12
    k1_gbs = pb / (ms_prefix_kernel * 1e-3) / 1e9
    k1_tflops = pf / (ms_prefix_kernel * 1e-3) / 1e12

    # the dominant pass's roofline: HBM below the ridge point, MFMA above it
    mfma_bound = pf / pb > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": prefix_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": prefix_tflops / MFMA_BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": prefix_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": prefix_gbs / HBM_PEAK_GBS}
    traffic_key = f"{w.name}~sparse" if args.sparse else w.name
    traffic = measured_traffic(traffic_key) if args.kv_layout == "head" and args.chunk_select == "topk" else None
    roof.update({
        "traffic": traffic,
        "traffic_source": ("profiles/hbm_traffic.md (rocprofv3 FETCH_SIZE + WRITE_SIZE per dispatch, "
                           "copy-calibrated, K1 + K2, same library source)") if traffic is not None else None,
        "kernel": ("prefix pass: attn_bf16 split-KV partials (fb_prefix_partials" +
                   (", selected chunks" if args.sparse else "") + ") + combine_kernel (fb_prefix_combine)"),
        "us_per_launch": ms_prefix_pass * 1e3,
        "timing": (f"HIP events on the launch stream around batches of 10 back-to-back passes, K1 alone and "
                   f"K1 + K2 alternating for {args.sustain_s:g} s after the timed steps; first quarter dropped"),
        "algorithmic_bytes_per_launch": pb,
        "algorithmic_flops_per_launch": pf,
        "hbm_gbs": prefix_gbs, "hbm_frac": prefix_gbs / HBM_PEAK_GBS,
        "mfma_tflops": prefix_tflops, "mfma_frac": prefix_tflops / MFMA_BF16_PEAK_TFLOPS,
        "k1_only": {"kernel": "attn_bf16 split-KV partials (fb_prefix_partials)", "us": ms_prefix_kernel * 1e3,
                    "hbm_gbs": k1_gbs, "hbm_frac": k1_gbs / HBM_PEAK_GBS,
                    "mfma_tflops": k1_tflops, "mfma_frac": k1_tflops / MFMA_BF16_PEAK_TFLOPS},
    })

    result = {
        "metric": METRIC,
        "value": q_tokens / (ms_cached * 1e-3),
        "unit": "query-tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_cached,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded N(0,1) draws, bf16-rounded, block random walk)" if args.policy == "fixed" else
                 "synthetic (seeded N(0,1) draws, bf16-rounded, decoding-style block steps: "
                 + ("uneven token reveals)" if args.policy == "tau" else "per-head drift spread 0.9)")),
        "config": {
            "workload": w.name, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "head_dim": w.head_dim,
            "block_len": w.block_len, "prefix_len": lens if w.batch > 1 else lens[0],
            "denoise_steps": w.steps, "blocks": len(blocks), "refresh_period": r,
            "kv_layout": {"head": "head-major [Hkv][T][D]", "token": "token-major [T][Hkv][D]",
                          "interleave": "per-token K/V interleave [Hkv][T][2][D]"}[args.kv_layout],
            "sparse": ({"chunks_kept": k_sel, "chunk_len": 64, "residual": "cached at refresh steps",
                        "selection": ("top-k on the GPU at each block's first step (inside the step); pooled "
                                      "chunk keys kept per layer, the block's new chunks pooled in the step" if topk
                                      else "seeded random stand-in (fixed)")} if args.sparse else None),
            "step": "one block of denoise_steps attention steps, one layer",
            "launch": "graph replay" if args.graph else "eager",
            "policy": ({"name": "fixed", "refresh_period": r} if args.policy == "fixed" else
                       {"name": args.policy, "tau": args.tau, "eps": args.eps} if args.policy == "tau" else
                       {"name": "gamma", "gamma": args.gamma}),
        },
        "recompute_fraction_per_step": recomputed if args.policy != "fixed" else None,
        "full_recompute": {"value": q_tokens / (ms_full * 1e-3), "unit": "query-tok/s", "ms_per_step": ms_full},
        "speedup_vs_full": ms_full / ms_cached,
        "step_latency_us": {"refresh_median": med(lat["refresh"]), "refresh_p10": pct(lat["refresh"], 10),
                            "refresh_p90": pct(lat["refresh"], 90), "reuse_median": med(lat["reuse"]),
                            "reuse_p10": pct(lat["reuse"], 10), "reuse_p90": pct(lat["reuse"], 90),
                            "samples": {"refresh": len(lat["refresh"]), "reuse": len(lat["reuse"])},
                            "launch_floor": ms_floor * 1e3},
        "step_graph_us": step_graph,
        "block_pass": {"us": ms_block * 1e3, "timing": "graph of back-to-back launches, replayed",
                       "algorithmic_bytes": bb, "algorithmic_flops": bf,
                       "gbs": bb / (ms_block * 1e-3) / 1e9, "tflops": bf / (ms_block * 1e-3) / 1e12,
                       "mfma_frac": bf / (ms_block * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "kernels_us": {"prefix_splitkv": ms_prefix_kernel * 1e3, "split_combine": ms_combine * 1e3,
                       "prefix_pass_k1_k2": ms_prefix_pass * 1e3,
                       "block_attn_merge": ms_block * 1e3,
                       "select_chunks": ms_select * 1e3 if ms_select is not None else None,
                       "select_chunks_full_pool": ms_select_full * 1e3 if ms_select_full is not None else None},
        "drift_max_abs": max(drift),
        "drift_per_step": drift,
        "sparse_only_drift_max_abs": max(sparse_only_drift) if sparse_only_drift else None,
        "roofline": roof,
        "gpu_state": (None if args.no_gpu_state else
                      {"idle_before_timing": gpu_idle, "under_full_recompute_steps_after_timing": gpu_load,
                       "source": "amd-smi metric -g 0 --power --clock"}),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host ...")
        variant = "sparse" if args.sparse else args.policy
        result["cpu_baseline"] = cpu_baseline(w, wl.Prefix(*block_prefix[0]), blocks, r, variant=variant,
                                              k_sel=k_sel, tau=args.tau, eps=args.eps, gamma=args.gamma)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

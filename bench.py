#!/usr/bin/env python3
"""Benchmark of one CSA2 Full-mode decode layer step on one MI355X.

Step (per timed iteration, all on one stream, inputs resident in HBM):
  quantise-and-write the new token's main-KV entry (NVFP4), indexer-K entry (MXFP4) and
  sliding-window entry (FP8) of every sequence; quantise the indexer Q (MXFP4); score every
  visible entry (FP4 matrix cores); Top-512; sparse attention over the 512 entries plus the
  128-token window.  Metric: query tokens per second per layer.

Default workload: batched decode, 64 queries, 131,072 compressed entries per sequence (128K
tokens at m=1), 64 heads, 16 indexer heads.  `--ctx1m` adds the 1M-entry decode (8 queries)
as a second measurement.  The CPU baseline times the fp64 oracle on a bounded sample.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MAIN_ENTRY_B = 288      # 256 B E2M1 codes + 32 E4M3 scales
INDEX_ENTRY_B = 68      # 64 B E2M1 codes + 4 E8M0 scales


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def build_gpu_state(wl, torch, C):
    """Seeded latents -> HBM caches through the library's own quantiser (setup, untimed)."""
    from fp4_kv_cache_layer_amd.layer import Caches, Csa2Step
    from synth.workloads import DIM, IDX_DIM
    dev = "cuda"
    caches = Caches.empty(wl.n_seq, wl.seq_cap, (0,), wl.swa_cap)
    caches.swa_base.fill_(wl.swa_base)
    chunk = 1 << 16
    t0 = time.time()
    for b in range(wl.n_seq):
        for r0 in range(0, wl.seq_cap, chunk):
            n = min(chunk, wl.seq_cap - r0)
            lat = torch.from_numpy(wl.main_latents(b, r0, n)).to(dev)
            C.csa2_quantize_kv(lat, C.FMT_NVFP4, caches.kv_codes[b, r0:r0 + n], caches.kv_scales[b, r0:r0 + n])
            ik = torch.from_numpy(wl.index_k_latents(b, r0, n)).to(dev)
            C.csa2_quantize_kv(ik, C.FMT_MXFP4, caches.ik_codes[b, r0:r0 + n], caches.ik_scales[b, r0:r0 + n])
        t = int(wl.q_pos[wl.q_seq == b].max())
        p0 = max(0, t - wl.swa_cap + 1)
        sw = wl.swa_latents(0, b, p0, t - p0 + 1)
        rows = torch.from_numpy(((np.arange(p0, t + 1) - wl.swa_base) % wl.swa_cap).astype(np.int64)).to(dev)
        C.csa2_quantize_kv(torch.from_numpy(sw).to(dev), C.FMT_FP8, caches.swa[0][b], None, rows)
        if b % 16 == 15:
            log(f"  caches: {b + 1}/{wl.n_seq} sequences ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    st = {}
    q_seq = torch.from_numpy(wl.q_seq.astype(np.int32)).to(dev)
    st["q_seq"], st["n_vis"] = q_seq, torch.from_numpy(wl.n_vis).to(dev)
    st["q_pos"], st["rs"] = torch.from_numpy(wl.q_pos).to(dev), torch.from_numpy(wl.replay_start).to(dev)
    st["q_idx"] = torch.from_numpy(wl.index_q(0)).to(dev)
    st["w"] = torch.from_numpy(wl.index_w(0)).to(dev)
    st["qa"] = torch.from_numpy(wl.attn_q_bits(0).view(np.int16)).to(dev).view(torch.bfloat16)
    # the newest token of every sequence: its entry latents, written inside the step
    first_new = int(wl.new_entries[0])
    new_main = np.stack([wl.main_latents(int(b), first_new, 1)[0] for b in wl.q_seq])
    new_ik = np.stack([wl.index_k_latents(int(b), first_new, 1)[0] for b in wl.q_seq])
    new_swa = np.stack([wl.swa_latents(0, int(b), int(t), 1)[0] for b, t in zip(wl.q_seq, wl.q_pos)])
    st["new_main"], st["new_ik"] = torch.from_numpy(new_main).to(dev), torch.from_numpy(new_ik).to(dev)
    st["new_swa"] = torch.from_numpy(new_swa).to(dev)
    st["dst_entry"] = torch.from_numpy((wl.q_seq.astype(np.int64) * wl.seq_cap + first_new)).to(dev)
    st["dst_swa"] = torch.from_numpy(wl.q_seq.astype(np.int64) * wl.swa_cap +
                                     (wl.q_pos - wl.swa_base) % wl.swa_cap).to(dev)
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap)
    return caches, st, step


def bound_calls(wl, caches, st, step, C):
    """The step's calls, validated and marshalled once: list of (phase, callable)."""
    kvc = caches.kv_codes.view(-1, caches.kv_codes.shape[2])
    kvs = caches.kv_scales.view(-1, caches.kv_scales.shape[2])
    ikc = caches.ik_codes.view(-1, caches.ik_codes.shape[2])
    iks = caches.ik_scales.view(-1, caches.ik_scales.shape[2])
    swa = caches.swa[0].view(-1, caches.swa[0].shape[2])
    return [
        ("quant_main", C.csa2_quantize_kv(st["new_main"], C.FMT_NVFP4, kvc, kvs, st["dst_entry"], _bind=True)),
        ("quant_index_k", C.csa2_quantize_kv(st["new_ik"], C.FMT_MXFP4, ikc, iks, st["dst_entry"], _bind=True)),
        ("quant_swa", C.csa2_quantize_kv(st["new_swa"], C.FMT_FP8, swa, None, st["dst_swa"], _bind=True)),
        ("quant_index_q", step.quantize_index_q(st["q_idx"], bind=True)),
        ("index_topk", step.index_topk(caches, st["w"], st["q_seq"], st["n_vis"], bind=True)),
        ("attn", step.attend(caches, 0, st["qa"], st["q_seq"], st["q_pos"], st["rs"], bind=True)),
    ]


def time_isolated(fn, iters, torch):
    """Mean GPU time of `iters` back-to-back launches of one bound call (HIP events on the
    launch stream; meaningful for kernels much longer than the host launch cost)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def capture_step(wl, caches, st, step, C, torch):
    """Record the step's calls into one HIP graph and check replays against an eager run."""
    for _, fn in bound_calls(wl, caches, st, step, C):
        fn()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.idx, step.count, step.out, step.lse)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _, fn in bound_calls(wl, caches, st, step, C):   # bound to the capture stream
            fn()
    for rep in range(3):
        for t in (step.idx, step.count, step.out, step.lse):  # eager work between replays
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip((step.idx, step.count, step.out, step.lse), ref):
            if not torch.equal(t, r):
                raise RuntimeError(f"graph replay {rep} differs from the eager step")
    return graph


def time_graph(graph, steps, warmup, torch):
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - wall0


def score_bytes(wl) -> int:
    """Algorithmic HBM bytes of one scoring launch: every visible indexer-K entry (68 B) of
    every query, plus each query's MXFP4 indexer Q and head weights."""
    per_q_fixed = wl.idx_heads * (64 + 4 + 4)
    return int(wl.n_vis.sum()) * INDEX_ENTRY_B + wl.n_q * per_q_fixed


def step_bytes(wl) -> int:
    """Algorithmic HBM bytes of one Full layer step (what must cross HBM at least once)."""
    k, W = 512, 128
    per_q = (k * MAIN_ENTRY_B + W * 512 + wl.heads * 512 * (2 + 4) + k * 4)   # gather, window, Q bf16, out f32, idx
    return score_bytes(wl) + wl.n_q * per_q


def cpu_baseline(wl, n_sample: int, reps: int):
    """The fp64 oracle, as it stands, on `n_sample` queries of the same workload."""
    from oracle import csa2_oracle as O
    from synth import bf16_bits_to_f32
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:
        threads = 1
    sm = 1.0 / math.sqrt(512)
    prepared = []
    for qi in range(n_sample):
        b = int(wl.q_seq[qi])
        nv, t, s = int(wl.n_vis[qi]), int(wl.q_pos[qi]), int(wl.replay_start[qi])
        ik_c, ik_s = O.quantize_mxfp4(wl.index_k_latents(b, 0, nv))
        qc, qs = O.quantize_mxfp4(wl.index_q(0, qi, 1)[0])
        w = wl.index_w(0, qi, 1)[0]
        qa = bf16_bits_to_f32(wl.attn_q_bits(0, qi, 1)[0]).astype(np.float64)
        kv_c = np.zeros((nv, 256), np.uint8)
        kv_s = np.zeros((nv, 32), np.uint8)
        probe = O.PackedCaches(kv_c, kv_s, ik_c, ik_s)
        pos, sc = O.full_scores(qc, qs, w, probe, nv)
        need = O.topk_positions(sc, pos, 512)
        need = need[need >= 0]
        for p in need:  # the main-KV rows this query reads (the packed cache is an input)
            kv_c[p], kv_s[p] = (a[0] for a in O.quantize_nvfp4(wl.main_latents(b, int(p), 1)))
        p0 = max(0, t - wl.swa_cap + 1)
        ring = np.zeros((wl.swa_cap, 512), np.float32)
        ring[(np.arange(p0, t + 1) - wl.swa_base) % wl.swa_cap] = wl.swa_latents(0, b, p0, t - p0 + 1)
        swa = {0: (O.quantize_fp8(ring), wl.swa_base, wl.swa_cap)}
        prepared.append((qc, qs, w, qa, kv_c, kv_s, ik_c, ik_s, swa, t, s, nv))
    t0 = time.perf_counter()
    for _ in range(reps):
        for (qc, qs, w, qa, kv_c, kv_s, ik_c, ik_s, swa, t, s, nv) in prepared:
            caches = O.PackedCaches(kv_c, kv_s, ik_c, ik_s, swa)   # fresh: dequantises the cache again
            O.layer_step("full", q_codes=qc, q_scales=qs, w=w, caches=caches, layer=0, q_attn=qa, t=t, s=s,
                         n_vis=nv, sm_scale=sm)
    el = time.perf_counter() - t0
    return {"value": n_sample * reps / el, "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_sample} of {wl.n_q} queries (their own {wl.seq_cap}-entry sequences), each Full layer "
                      f"step (dequantise indexer-K cache, score, Top-512, dequantise 512+window rows, attention) "
                      f"run {reps}x; {el:.1f}s; numpy fp64, BLAS threads = cores"}


def run_workload(name, steps, warmup, torch, C):
    from synth import workloads
    wl = workloads.config(name)
    log(f"workload {name}: {wl.description}")
    caches, st, step = build_gpu_state(wl, torch, C)
    graph = capture_step(wl, caches, st, step, C, torch)
    ms, wall = time_graph(graph, steps, warmup, torch)
    calls = dict(bound_calls(wl, caches, st, step, C))
    phase = {name: time_isolated(fn, 20, torch) for name, fn in calls.items()}
    return wl, ms, phase, wall


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--ctx1m", action="store_true", help="also measure the 1M-entry decode workload")
    ap.add_argument("--cpu-sample", type=int, default=4)
    ap.add_argument("--cpu-reps", type=int, default=48)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the CSA2 step is built and measured on a single MI355X "
              "(sequences would shard across GPUs with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp4_kv_cache_layer_amd import csa2 as C
    C.csa2_init()
    torch.cuda.set_device(0)

    wl, ms, phase, wall = run_workload(args.workload, args.steps, args.warmup, torch, C)
    value = wl.n_q / (ms / 1000.0)
    sb = score_bytes(wl)
    achieved = sb / (phase["index_topk"] / 1000.0) / 1e9
    log(f"step {ms * 1000:.1f} us (graph replay); isolated launches (us): " +
        ", ".join(f"{k}={v * 1000:.1f}" for k, v in phase.items()))
    log(f"index_topk {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of HBM peak)")
    result = {
        "metric": "CSA2 decode query-tokens/s per layer at 128K & 1M ctx; % HBM peak",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4 scoring (mxfp4 x mxfp4 -> fp32), bf16/fp16 attention -> fp32",
        "data": "synthetic (seeded counter-based generator; no datasets or weights)",
        "config": {"workload": f"{wl.name}: {wl.description}", "queries": wl.n_q, "context_entries": wl.seq_cap,
                   "m": wl.m, "heads": wl.heads, "index_heads": wl.idx_heads, "topk": 512, "window": 128},
        "timing": "HIP events around graph replays of the whole step (one graph launch per step)",
        "isolated_launch_us": {k: round(v * 1000, 2) for k, v in phase.items()},
        "hbm_frac_step": round(step_bytes(wl) / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "csa2_index_topk (k_score_select + last selection level)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": sb, "traffic": None},
    }
    if args.ctx1m:
        wl4, ms4, phase4, _ = run_workload("c4", args.steps, args.warmup, torch, C)
        sb4 = score_bytes(wl4)
        result["ctx_1m"] = {"workload": f"{wl4.name}: Full layer only, {wl4.n_q} queries x {wl4.seq_cap} entries",
                            "value": round(wl4.n_q / (ms4 / 1000.0), 1), "ms_per_step": round(ms4, 5),
                            "isolated_launch_us": {k: round(v * 1000, 2) for k, v in phase4.items()},
                            "index_topk_frac_hbm": round(sb4 / (phase4["index_topk"] / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

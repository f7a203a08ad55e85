#!/usr/bin/env python3
"""Benchmark of the CSA2 layer step on one MI355X.

A layer step (inputs resident in HBM): append the new token's cache
entries (Full layers: main KV in NVFP4 and indexer K in MXFP4; every layer: its FP8
window entry), quantise the layer's indexer Q (MXFP4), score the candidates on the FP4
matrix cores and keep the Top-512 (Full: every visible entry; Reindex: the same cache
with the layer's own indexer Q, inside the pool when there is one), and attend over the
512 entries plus the 128-token window.  A Reuse layer only appends its window entry and
attends with the borrowed index set.  A step's quantisations run as one launch.

Headline: the Full decode step of 64 queries x 131,072 entries (128K tokens at m=1), 64
heads, 16 indexer heads; metric query tokens per second per layer.  Also reported (unless
--no-modes): every mode of the 128K layer group (Full, 3 Reuse, Reindex; 32 queries) and
of the 1M group (Full + pool, 4 Reindex inside the pool; 8 queries), each group as one
graph, the m = 2 prefill chunk, an encoder group (Full + 5 Reuse) over that chunk after a
window-state miss, multi-token decode, the headline step with the NVFP4-style indexer
(E4M3 per 16 channels), and the whole decoder step (its 20 CSA2 layers as one graph) at
128K and 1M.  The CPU baseline times the fp64 oracle on a bounded sample of the headline step.
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
TOPK, WINDOW, BLOCK, MAX_BLOCKS = 512, 128, 8, 2048


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class LayerBench:
    """GPU state of one workload's layer group: caches built from the seeded latents by the
    library's own quantiser (setup, untimed), per-layer query inputs, the new token's
    latents, and a Csa2Step.  A layer step = appending the new token's cache entries, then
    the layer's own calls (Full: main KV + indexer K + its window entry; Reuse / Reindex:
    its window entry only, since they share the Full layer's global KV).  With a window miss
    (`swa_miss`: the prefix's window state is not cached) the rings start empty and every
    layer writes the window entries of all its query rows, replay rows included."""

    def __init__(self, wl, torch, C, group: int = 1, index_fmt: str = "mxfp4", attn_select: bool = True,
                 fused: bool = True):
        from fp4_kv_cache_layer_amd.layer import INDEX_FORMATS, Caches, Csa2Step, plan_group
        self.wl, self.torch, self.C = wl, torch, C
        self.ik_fmt, self.ik_group = INDEX_FORMATS[index_fmt]
        n_layers = len(wl.layers)
        dev = "cuda"
        caches = Caches.empty(wl.n_seq, wl.seq_cap, range(n_layers), wl.swa_cap, index_fmt=index_fmt)
        caches.swa_base.fill_(wl.swa_base)
        chunk = 1 << 16
        t0 = time.time()
        for b in range(wl.n_seq):
            for r0 in range(0, wl.seq_cap, chunk):
                n = min(chunk, wl.seq_cap - r0)
                main = wl.main_latents(b, r0, n)
                lat = torch.from_numpy(main).to(dev)
                C.csa2_quantize_kv(lat, C.FMT_NVFP4, caches.kv_codes[b, r0:r0 + n], caches.kv_scales[b, r0:r0 + n])
                ik = torch.from_numpy(wl.index_k_latents(b, r0, n, main=main)).to(dev)
                C.csa2_quantize_kv(ik, self.ik_fmt, caches.ik_codes[b, r0:r0 + n], caches.ik_scales[b, r0:r0 + n])
            t = int(wl.q_pos[wl.q_seq == b].max())
            p0 = max(0, t - wl.swa_cap + 1)
            rows = torch.from_numpy(((np.arange(p0, t + 1) - wl.swa_base) % wl.swa_cap).astype(np.int64)).to(dev)
            for L in range(n_layers) if not wl.extra.get("swa_miss") else ():
                sw = wl.swa_latents(L, b, p0, t - p0 + 1)
                C.csa2_quantize_kv(torch.from_numpy(sw).to(dev), C.FMT_FP8, caches.swa[L][b], None, rows)
            if b % 16 == 15 or b == wl.n_seq - 1:
                log(f"  caches: {b + 1}/{wl.n_seq} sequences ({time.time() - t0:.1f}s)")
        torch.cuda.synchronize()
        self.caches = caches
        self.q_seq = torch.from_numpy(wl.q_seq.astype(np.int32)).to(dev)
        self.n_vis = torch.from_numpy(wl.n_vis).to(dev)
        self.q_pos = torch.from_numpy(wl.q_pos).to(dev)
        self.rs = torch.from_numpy(wl.replay_start).to(dev)
        self.inputs = []
        for L in range(n_layers):
            q_idx = torch.from_numpy(wl.index_q(L)).to(dev)
            w = torch.from_numpy(wl.index_w(L)).to(dev)
            qa = torch.from_numpy(wl.attn_q_bits(L).view(np.int16)).to(dev).view(torch.bfloat16)
            self.inputs.append((q_idx, w, qa))
        # every queried sequence's new entries [first_new, first_new + n_new) (decode: its
        # newest token; multi-token decode: its tokens; prefill: the chunk's entries), and the
        # window rows of the new tokens (of every query row when the window state missed;
        # otherwise the replay rows' window entries are cached)
        first_new, n_new = int(wl.new_entries[0]), int(wl.new_entries[1])
        seqs = np.unique(wl.q_seq).astype(np.int64)
        ent_seq = np.repeat(seqs, n_new)
        ent_row = np.tile(first_new + np.arange(n_new, dtype=np.int64), seqs.size)
        new_tok = wl.q_pos >= (-1 if wl.extra.get("swa_miss") else first_new * wl.m)
        tok_seq, tok_pos = wl.q_seq[new_tok].astype(np.int64), wl.q_pos[new_tok]
        self.new_main = torch.from_numpy(np.stack([wl.main_latents(int(b), int(r), 1)[0]
                                                   for b, r in zip(ent_seq, ent_row)])).to(dev)
        self.new_ik = torch.from_numpy(np.stack([wl.index_k_latents(int(b), int(r), 1)[0]
                                                 for b, r in zip(ent_seq, ent_row)])).to(dev)
        self.new_swa = [torch.from_numpy(np.stack([wl.swa_latents(L, int(b), int(t), 1)[0]
                                                   for b, t in zip(tok_seq, tok_pos)])).to(dev)
                        for L in range(n_layers)]
        # one new token per queried sequence and every row is one of them (decode): the
        # attention call appends the row's window entry itself
        self.fuse_window = bool(np.unique(wl.q_seq).size == wl.n_q and new_tok.all()
                                and not wl.extra.get("swa_miss"))
        self.dst_entry = torch.from_numpy(ent_seq * wl.seq_cap + ent_row).to(dev)
        # single-token decode (each query its own sequence, one new entry each): a Full layer's
        # scoring call writes the new main-KV and indexer-K rows itself and quantises the
        # indexer Q itself, and the attention call appends the window entry, so the layer
        # step makes no quantise launch
        self.fold_append = bool(self.fuse_window and n_new == 1 and index_fmt == "mxfp4" and group == 1 and fused)
        if self.fold_append:
            self.app = (torch.full((wl.n_q,), first_new, dtype=torch.int64, device=dev),
                        torch.from_numpy(np.stack([wl.main_latents(int(b), first_new, 1)[0] for b in wl.q_seq])).to(dev),
                        torch.from_numpy(np.stack([wl.index_k_latents(int(b), first_new, 1)[0]
                                                   for b in wl.q_seq])).to(dev))
        self.dst_swa = torch.from_numpy(tok_seq * wl.swa_cap + (tok_pos - wl.swa_base) % wl.swa_cap).to(dev)
        self.step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap, group=group, index_fmt=index_fmt,
                             attn_select=attn_select, fused=fused)
        self.plan = plan_group(wl.layers, fused=fused, group=group, index_fmt=index_fmt,
                               attn_select=self.step.attn_select, pool_select=self.step.pool_select,
                               group_select=self.step.group_select, q_in_call=self.step.q_in_call)
        torch.cuda.synchronize()   # the setup's copies and launches end here

    def calls(self, L: int):
        """Layer L's step as {phase: bound call} bound to the current stream, in order."""
        C, c, st = self.C, self.caches, self.step
        mode = self.wl.layers[L]
        flat = lambda t: t.view(-1, t.shape[2])
        out = {}
        # the step's quantisations in one launch: the new entries (Full layers: main KV and
        # indexer K; every layer: its window entry) and the layer's indexer Q
        jobs = []
        fold = self.fold_append and mode.startswith("full")   # appends and Q inside the scoring call
        app = self.app if fold else None
        if mode.startswith("full") and not fold:
            jobs += [(self.new_main, C.FMT_NVFP4, flat(c.kv_codes), flat(c.kv_scales), self.dst_entry),
                     (self.new_ik, self.ik_fmt, flat(c.ik_codes), flat(c.ik_scales), self.dst_entry)]
        if not self.fuse_window:
            jobs.append((self.new_swa[L], C.FMT_FP8, flat(c.swa[L]), None, self.dst_swa))
        q_idx, w, qa = self.inputs[L]
        names = self.plan[L]
        if "quantize_index_q" in names and not fold:
            n_q, h, d = q_idx.shape
            jobs.append((q_idx.view(n_q * h, d), self.ik_fmt, st.qi_codes.view(n_q * h, d // 2),
                         st.qi_scales.view(n_q * h, d // self.ik_group), None))
        if jobs:
            out["quantize"] = C.csa2_quantize_kv_multi(jobs, _bind=True)
        nw = self.new_swa[L] if self.fuse_window else None
        # calls named "..._q" (and a Full layer's scoring call with the appends) read the
        # unquantised indexer Q and quantise it themselves
        qq = q_idx if fold or any(n.endswith("_q") and n != "quantize_index_q" for n in names) else None
        if mode == "full_pool":
            out["index_topk_pool"] = st.index_topk_build_pool(c, w, self.q_seq, self.n_vis, bind=True, q=qq,
                                                              append=app)
        elif "index_topk_grouped" in names:   # grouped rows scored and selected, no score array
            out["index_topk_grouped"] = st.index_topk_grouped(c, w, self.q_seq, self.n_vis, bind=True)
        elif "score_grouped" in names:
            out["score"] = st.score_grouped(c, w, self.q_seq, self.n_vis, bind=True)
            out["select"] = st.select(self.n_vis, bind=True)
        elif "index_segments" in names or "index_segments_q" in names:
            out["index_segments"] = st.index_segments(c, w, self.q_seq, self.n_vis, bind=True, q=qq, append=app)
        elif "score_pool_q" in names:   # pool slot scores from the unquantised Q; Top-K in attention
            out["score"] = st.score_q(c, q_idx, w, self.q_seq, self.n_vis, in_pool=True, bind=True)
        elif "attend_pool_topk" in names:   # pool slot scores; the Top-K is selected in attention
            out["score"] = st.score(c, w, self.q_seq, self.n_vis, in_pool=True, bind=True)
        elif mode != "reuse":
            out["index_topk"] = st.index_topk(c, w, self.q_seq, self.n_vis, mode == "reindex_pool", bind=True, q=qq,
                                              append=app)
        if "attend_topk" in names:   # the last Top-K level runs inside the attention call
            out["attn"] = st.attend_topk(c, L, qa, self.q_seq, self.q_pos, self.rs, bind=True, new_win=nw)
        elif "attend_pool_topk" in names:
            out["attn"] = st.attend_pool_topk(c, L, qa, self.q_seq, self.n_vis, self.q_pos, self.rs, bind=True,
                                              new_win=nw)
        else:
            out["attn"] = st.attend(c, L, qa, self.q_seq, self.q_pos, self.rs, bind=True, new_win=nw)
        return out

    def segments_call(self, L: int):
        """Layer L's scoring pass alone (csa2_index_segments: the one k_score_select launch of
        csa2_index_topk, same grid and arguments), bound to the current stream; None where the
        layer does not score every visible entry or its survivors exceed one selection."""
        mode, st = self.wl.layers[L], self.step
        if mode not in ("full", "reindex") or not 1 <= self.C.csa2_segment_keys(self.wl.seq_cap, st.k) <= 8192:
            return None
        return st.index_segments(self.caches, self.inputs[L][1], self.q_seq, self.n_vis, bind=True,
                                 q=self.inputs[L][0] if st.q_in_call else None)

    def record(self, layers):
        """Issues the steps of `layers` on the current stream.  (Forking the appends onto
        parallel graph branches was measured slower: the joins cost more than the overlap.)"""
        for L in layers:
            for fn in self.calls(L).values():
                fn()

    def capture(self, layers):
        """One HIP graph of the steps of `layers`; three replays are checked bitwise against
        an eager run of the same calls."""
        torch = self.torch
        # a Reuse layer reads the index set the previous scoring layer left: only the
        # attention outputs are outputs there
        scoring = any(self.wl.layers[L] != "reuse" for L in layers)
        outs = ((self.step.idx, self.step.count) if scoring else ()) + (self.step.out, self.step.lse)
        self.record(layers)
        torch.cuda.synchronize()
        ref = [t.clone() for t in outs]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.record(layers)
        for rep in range(3):
            for t in outs:  # eager work between replays
                t.zero_()
            graph.replay()
            torch.cuda.synchronize()
            for t, r in zip(outs, ref):
                if not torch.equal(t, r):
                    raise RuntimeError(f"graph replay {rep} of layers {layers} differs from the eager run")
        return graph


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


def time_call_graph(make, calls, replays, torch):
    """Mean GPU time of one call, from HIP events (on the launch stream) around `replays`
    replays of a graph holding `calls` back-to-back launches of it: the kernels' own
    durations and the gaps between them, without the host's launch cost.  `make()` binds
    the call to the current stream, so it is called inside the capture."""
    make()()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn = make()
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (replays * calls)


def steps_per_graph(steps: int) -> int:
    """Layer steps captured in one graph: consecutive layers of a decode step replay as one
    graph, so the per-launch cost of the runtime is paid once per group, not per layer.
    The largest divisor of `steps` up to 8, so that exactly `steps` steps are timed."""
    return max(d for d in range(1, 9) if steps % d == 0)


def time_graph(graph, replays, warmup, torch, per_replay=1):
    """Mean time per step of `replays` graph replays, each running `per_replay` steps."""
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * per_replay), time.perf_counter() - wall0


def score_bytes(wl, mode: str, index_fmt: str = "mxfp4") -> int:
    """Algorithmic HBM bytes of one scoring pass: every candidate's indexer-K entry (68 B in
    MXFP4, 72 B in NVFP4; all visible entries, or the 16,384 pool positions) plus each
    query's indexer Q and head weights."""
    if mode == "reuse":
        return 0
    n_sc = 8 if index_fmt == "nvfp4" else 4
    cand = np.minimum(wl.n_vis, MAX_BLOCKS * BLOCK) if mode == "reindex_pool" else wl.n_vis
    return int(cand.sum()) * (64 + n_sc) + wl.n_q * wl.idx_heads * (64 + n_sc + 4)


def step_bytes(wl, mode: str, index_fmt: str = "mxfp4") -> int:
    """Algorithmic HBM bytes of one layer step: what must cross HBM at least once
    (scoring input; the gathered main-KV entries, window, Q, output, LSE and index set of
    attention; the pool ids where a pool is written or read)."""
    k, W = TOPK, WINDOW
    attn = k * MAIN_ENTRY_B + W * 512 + wl.heads * 512 * (2 + 4) + wl.heads * 4 + k * 4
    pool = MAX_BLOCKS * 4 if mode in ("full_pool", "reindex_pool") else 0
    return score_bytes(wl, mode, index_fmt) + wl.n_q * (attn + pool)


MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16 matrix-core peak


def attn_flops(wl) -> int:
    """Algorithmic FLOPs of one attention launch: S = Q K^T and O = P V over the Top-512
    entries plus the 128 window keys, 2 FLOP per multiply-add, for every head and query."""
    return wl.n_q * 4 * wl.heads * (TOPK + WINDOW) * 512


def attn_bytes(wl) -> int:
    """Algorithmic HBM bytes of one attention launch: the gathered main-KV entries (288 B),
    the window keys (512 B), Q (bf16), the fp32 output and LSE and the index set."""
    return wl.n_q * (TOPK * MAIN_ENTRY_B + WINDOW * 512 + wl.heads * 512 * (2 + 4) + wl.heads * 4 + TOPK * 4)


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
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:
        pass
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
            "cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n_sample} of {wl.n_q} queries (their own {wl.seq_cap}-entry sequences), each Full layer "
                      f"step (dequantise indexer-K cache, score, Top-512, dequantise 512+window rows, attention) "
                      f"run {reps}x; {el:.1f}s; numpy fp64, BLAS threads = cores"}


def measure_layers(name, steps, warmup, torch, C, layers_to_time, group: int = 1, index_fmt: str = "mxfp4",
                   attn_select: bool = True, fused: bool = True):
    """Graph-replay time of each listed layer's step (`steps` steps in graphs of
    steps_per_graph(steps) consecutive steps of that layer) and of the whole group (one
    group per graph); isolated launch times of the first listed layer's calls."""
    from synth import workloads
    wl = workloads.config(name)
    log(f"workload {name}: {wl.description}")
    label = f"workload {name}" + (f" group {group}" if group > 1 else "") + \
        (f" index {index_fmt}" if index_fmt != "mxfp4" else "") + ("" if attn_select else " last level kernel")
    with torch.cuda.nvtx.range(label):
        return _measure_layers(wl, steps, warmup, torch, C, layers_to_time, group, index_fmt, attn_select, fused)


def _measure_layers(wl, steps, warmup, torch, C, layers_to_time, group, index_fmt, attn_select, fused):
    with torch.cuda.nvtx.range("setup"):
        lb = LayerBench(wl, torch, C, group, index_fmt, attn_select, fused)
    res = {"wl": wl, "layers": {}}
    G = steps_per_graph(steps)
    res["per_graph"] = G
    for L in layers_to_time:
        g = lb.capture([L] * G)
        ms, wall = time_graph(g, steps // G, max(warmup // G, 1), torch, per_replay=G)
        res["layers"][L] = {"mode": wl.layers[L], "ms": ms, "wall": wall}
        del g
    if len(wl.layers) > 1:
        g = lb.capture(list(range(len(wl.layers))))
        ms, _ = time_graph(g, steps, warmup, torch)
        res["group_ms"] = ms
        del g
    L0 = layers_to_time[0]
    calls0 = lb.calls(L0)
    res["isolated"] = {n: time_isolated(fn, 20, torch) for n, fn in calls0.items()}
    res["graph_call"] = {n: time_call_graph(lambda n=n: lb.calls(L0)[n], 8, max(steps // 8, 3), torch)
                         for n in calls0}
    if "index_segments" not in calls0 and lb.segments_call(L0) is not None:
        # the dominant kernel on its own, for its roofline
        res["graph_call"]["scoring_kernel"] = time_call_graph(lambda: lb.segments_call(L0), 8, max(steps // 8, 3),
                                                              torch)
    del lb, calls0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def measure_group(name, steps, warmup, torch, C, group: int = 1):
    """Graph-replay time of a workload's whole layer group (each layer with its own appends)
    captured as one graph: a decoder step, or an encoder group over a prefill chunk."""
    from synth import workloads
    wl = workloads.config(name)
    log(f"workload {name}: {wl.description}")
    with torch.cuda.nvtx.range(f"workload {name}"):
        with torch.cuda.nvtx.range("setup"):
            lb = LayerBench(wl, torch, C, group)
        g = lb.capture(list(range(len(wl.layers))))
        ms, _ = time_graph(g, steps, warmup, torch)
        del g, lb
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return wl, ms


def decoder_entry(wl, ms) -> dict:
    n = len(wl.layers)
    return {"layers": n, "structure": "Full + pool, 3 Reuse, 4 x (Reindex in the pool, 3 Reuse)",
            "queries": wl.n_q, "context_entries": wl.seq_cap,
            "us_per_decode_step": round(ms * 1e3, 2), "us_per_layer": round(ms * 1e3 / n, 2),
            "query_tokens_per_s": round(wl.n_q / (ms / 1e3), 1)}


PREFILL_GROUP = 8   # rows of a prefill chunk scored per pass over the sequence's indexer K

TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_score_select_c2_128k_traffic.md")
TRAFFIC_SOURCES = ("fp4_kv_cache_layer_amd/csrc/score.hip", "fp4_kv_cache_layer_amd/csrc/select.h",
                   "fp4_kv_cache_layer_amd/csrc/device.h", "fp4_kv_cache_layer_amd/csrc/topk.hip",
                   "fp4_kv_cache_layer_amd/build.py")
COPY_BYTES = 1 << 30   # the calibration copy: 1 GiB read + 1 GiB written


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per k_score_select launch (the roofline's kernel) from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE runs, scaled by the calibration copy), or None when the
    summary is missing or the kernel sources changed since it was taken."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    vals = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("digest:", "traffic_bytes:")))
    if vals.get("digest", "").strip() != sources_digest():
        return None
    return int(vals["traffic_bytes"].strip())


def pmc_run(torch, C, name="c2"):
    """Workload of the counter runs: one plain 1 GiB device copy (the calibration of
    FETCH_SIZE / WRITE_SIZE), then each call of the workload's Full layer three times (the
    64 x 128K decode step, or the m = 2 prefill chunk scored in groups of 8 rows)."""
    from synth import workloads
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    lb = LayerBench(workloads.config(name), torch, C, group=PREFILL_GROUP if name == "c5" else 1)
    for name, fn in lb.calls(0).items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        log(f"pmc: {name} done")


def mode_entry(wl, mode, ms):
    b = step_bytes(wl, mode)
    return {"query_tokens_per_s": round(wl.n_q / (ms / 1e3), 1), "us_per_layer_step": round(ms * 1e3, 2),
            "hbm_frac": round(b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": b}


MFMA_FP4_PEAK_TFLOPS = 10100.0   # dense FP4 matrix-core peak


def score_flops(wl) -> int:
    """Algorithmic FLOPs of one scoring pass over every visible entry: a 128-channel dot
    product per indexer head (2 FLOP per multiply-add) for each query row and entry."""
    return int(wl.n_vis.astype(np.int64).sum()) * wl.idx_heads * 128 * 2


def mfma_entry(flops, ms, peak) -> dict:
    tf = flops / (ms / 1e3) / 1e12
    return {"us": round(ms * 1e3, 1), "flops": int(flops), "tflops": round(tf, 1), "mfma_peak_tflops": peak,
            "mfma_frac": round(tf / peak, 4)}


def run_group_128k(args, torch, C):
    r3 = measure_layers("c3", args.steps, args.warmup, torch, C, [0, 1, 4])
    out = {f"{v['mode']}_128k": mode_entry(r3["wl"], v["mode"], v["ms"]) for v in r3["layers"].values()}
    n3 = len(r3["wl"].layers)
    out["group_128k"] = {"layers": list(r3["wl"].layers), "us_per_group": round(r3["group_ms"] * 1e3, 2),
                         "query_tokens_per_s_per_layer": round(r3["wl"].n_q * n3 / (r3["group_ms"] / 1e3), 1)}
    return out


def run_group_1m(args, torch, C):
    r4 = measure_layers("c4", args.steps, args.warmup, torch, C, [0, 1])
    out = {f"{v['mode']}_1m": mode_entry(r4["wl"], v["mode"], v["ms"]) for v in r4["layers"].values()}
    n4 = len(r4["wl"].layers)
    out["group_1m"] = {"layers": list(r4["wl"].layers), "us_per_group": round(r4["group_ms"] * 1e3, 2),
                       "query_tokens_per_s_per_layer": round(r4["wl"].n_q * n4 / (r4["group_ms"] / 1e3), 1)}
    return out


def run_prefill_chunk(args, torch, C):
    # the chunk's rows all belong to one sequence: scored and selected in groups of 8 over
    # one pass of K
    r5 = measure_layers("c5", max(args.steps // 5, 3), max(args.warmup // 5, 1), torch, C, [0], group=PREFILL_GROUP)
    wl5, ms5, g5 = r5["wl"], r5["layers"][0]["ms"], r5["graph_call"]
    rows = int(wl5.extra["counted_rows"])
    return {"prefill_chunk_m2": {
        "query_rows": wl5.n_q, "counted_new_tokens": rows, "scoring_group": PREFILL_GROUP,
        "us_per_chunk": round(ms5 * 1e3, 1), "new_tokens_per_s": round(rows / (ms5 / 1e3), 1),
        "graph_call_us": {k: round(v * 1e3, 1) for k, v in g5.items()},
        "scoring": dict(kernel="k_score_topk_grouped (csa2_index_topk_grouped: FP4 scores and Top-512 of 8 rows "
                               "per pass over the sequence's indexer K; no score array)",
                        **mfma_entry(score_flops(wl5), g5["index_topk_grouped"], MFMA_FP4_PEAK_TFLOPS)),
        "attention": dict(kernel="k_attn_rows (csa2_sparse_attn, 512 entries + window per row, one workgroup per row)",
                          **mfma_entry(attn_flops(wl5), g5["attn"], MFMA_F16_PEAK_TFLOPS)),
        "isolated_launch_us": {k: round(v * 1000, 1) for k, v in r5["isolated"].items()}}}


def run_encoder_group(args, torch, C):
    re_ = measure_layers("enc_group", max(args.steps // 5, 3), max(args.warmup // 5, 1), torch, C, [0, 1],
                         group=PREFILL_GROUP)
    wle, mse, ge = re_["wl"], re_["group_ms"], re_["graph_call"]
    rows = int(wle.extra["counted_rows"])
    return {"encoder_group_prefill_m2": {
        "layers": len(wle.layers), "structure": "Full + 5 Reuse, window state missed (replay rows rewrite it)",
        "query_rows": wle.n_q, "counted_new_tokens": rows, "us_per_chunk": round(mse * 1e3, 1),
        "us_per_layer": round(mse * 1e3 / len(wle.layers), 1), "new_tokens_per_s": round(rows / (mse / 1e3), 1),
        "scoring_group": PREFILL_GROUP,
        "us_full_layer": round(re_["layers"][0]["ms"] * 1e3, 1), "us_reuse_layer": round(re_["layers"][1]["ms"] * 1e3, 1),
        "full_layer_graph_call_us": {k: round(v * 1e3, 1) for k, v in ge.items()},
        "scoring": mfma_entry(score_flops(wle), ge["index_topk_grouped"], MFMA_FP4_PEAK_TFLOPS),
        "attention": mfma_entry(attn_flops(wle), ge["attn"], MFMA_F16_PEAK_TFLOPS)}}


def run_multi_token_decode(args, torch, C):
    # 4 tokens of each of 16 sequences; the Full layer's scoring with each sequence's 4 rows
    # in one pass over its K (group 4) and per row (group 1)
    mt = {}
    for g in (1, 4):
        rm = measure_layers("mtd_128k", args.steps, args.warmup, torch, C, [0], group=g)
        mt[g] = (rm["wl"], rm["layers"][0]["ms"], rm["isolated"])
    wlm = mt[1][0]
    return {"multi_token_decode_128k": {
        "sequences": wlm.n_seq, "tokens_per_seq": int(wlm.extra["tokens_per_seq"]), "query_rows": wlm.n_q,
        "us_per_layer_step": round(mt[1][1] * 1e3, 2), "query_tokens_per_s": round(wlm.n_q / (mt[1][1] / 1e3), 1),
        "us_per_layer_step_grouped_scoring": round(mt[4][1] * 1e3, 2),
        "isolated_launch_us": {k: round(v * 1e3, 1) for k, v in mt[1][2].items()},
        "isolated_launch_us_grouped": {k: round(v * 1e3, 1) for k, v in mt[4][2].items()}}}


def run_last_level_kernel(args, torch, C):
    # the headline step with the last Top-K level as a launch of its own
    rs_ = measure_layers("c2", args.steps, args.warmup, torch, C, [0], attn_select=False)
    g_ = rs_["graph_call"]
    return {"full_128k_last_level_kernel": {
        "calls": "csa2_index_topk (k_score_select + the last Top-K level), then csa2_sparse_attn",
        "us_per_layer_step": round(rs_["layers"][0]["ms"] * 1e3, 2),
        "query_tokens_per_s": round(rs_["wl"].n_q / (rs_["layers"][0]["ms"] / 1e3), 1),
        "graph_call_us": {k: round(v * 1e3, 2) for k, v in g_.items()},
        "index_topk_gb_per_s": round(score_bytes(rs_["wl"], "full") / (g_["index_topk"] / 1e3) / 1e9, 1)}}


def run_nvfp4_indexer(args, torch, C):
    rn = measure_layers("c2", args.steps, args.warmup, torch, C, [0], index_fmt="nvfp4")
    wln, msn, isn, gcn = rn["wl"], rn["layers"][0]["ms"], rn["isolated"], rn["graph_call"]
    bn = score_bytes(wln, "full", "nvfp4")
    scn = "index_segments" if "index_segments" in gcn else "index_topk"
    gbs = bn / (gcn[scn] / 1e3) / 1e9
    return {"full_128k_nvfp4_indexer": {
        "index_format": "E2M1 + E4M3 per 16 (72 B per indexer-K entry), fp16 MFMA scoring",
        "us_per_layer_step": round(msn * 1e3, 2), "query_tokens_per_s": round(wln.n_q / (msn / 1e3), 1),
        "scoring_call": f"csa2_{scn} (fmt CSA2_FMT_NVFP4)", "scoring_us": round(gcn[scn] * 1e3, 2),
        "scoring_gb_per_s": round(gbs, 1), "scoring_hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "scoring_bytes": bn,
        "scoring_kernel_us": round(gcn["scoring_kernel"] * 1e3, 2) if "scoring_kernel" in gcn else None,
        "isolated_launch_us": {k: round(v * 1e3, 2) for k, v in isn.items()}}}


def run_decoders(args, torch, C):
    out = {}
    for name, key in (("dec_128k", "decoder_128k"), ("dec_1m", "decoder_1m")):
        wld, msd = measure_group(name, args.steps, args.warmup, torch, C)
        out[key] = decoder_entry(wld, msd)
    return out


# the reported modes, each measured in its own runner (`--only NAME` runs one, for profiling)
MODE_RUNNERS = {"group_128k": run_group_128k, "group_1m": run_group_1m, "prefill_chunk": run_prefill_chunk,
                "encoder_group": run_encoder_group, "multi_token_decode": run_multi_token_decode,
                "last_level_kernel": run_last_level_kernel, "nvfp4_indexer": run_nvfp4_indexer,
                "decoders": run_decoders}


def device_copy_gbs(torch, reps: int = 10) -> dict:
    """Two plain streaming kernels of torch on 1 GiB, timed with HIP events: a device-to-device
    copy (read + write counted) and row sums of the buffer as a [2^18, 4096] fp32 matrix (a
    read stream; it writes 1 MiB; of torch's reductions this layout reads fastest here): the
    HBM rates ordinary streaming kernels reach on this GPU, beside the 8 TB/s spec.  The
    scoring kernel only reads, so the read stream is its practical reference."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    rows = src.view(torch.float32).view(-1, 4096)
    dst.copy_(src)
    rows.sum(dim=1)
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    copy = 2 * COPY_BYTES / timed(lambda: dst.copy_(src)) / 1e9
    read = COPY_BYTES / timed(lambda: rows.sum(dim=1)) / 1e9
    del src, dst, rows
    torch.cuda.empty_cache()
    return {"gb_per_s": round(copy, 1), "bytes_per_copy": 2 * COPY_BYTES, "frac_of_spec": round(copy / HBM_PEAK_GBS, 4),
            "read_gb_per_s": round(read, 1), "read_frac_of_spec": round(read / HBM_PEAK_GBS, 4),
            "timing": f"HIP events around {reps} back-to-back 1 GiB copies (read + write counted) and {reps} "
                      f"row sums of the same 1 GiB as a [2^18, 4096] fp32 matrix (read stream)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-modes", action="store_true", help="skip the per-mode 128K group and 1M pool group")
    ap.add_argument("--cpu-sample", type=int, default=4)
    ap.add_argument("--cpu-reps", type=int, default=48)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--pmc-run", nargs="?", const="c2", choices=("c2", "c5"),
                    help="only run the workload of a counter run and exit: the calibration copy and the "
                         "64 x 128K Full step's calls (c2, the default), or the m = 2 prefill chunk's calls (c5)")
    ap.add_argument("--only", choices=tuple(MODE_RUNNERS),
                    help="only measure this mode (no headline line: for per-workload kernel traces)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the CSA2 step is built and measured on a single MI355X "
              "(sequences would shard across GPUs with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from fp4_kv_cache_layer_amd import csa2 as C
    C.csa2_init()
    torch.cuda.set_device(0)
    if args.pmc_run:
        pmc_run(torch, C, args.pmc_run)
        return
    if args.only:
        modes = MODE_RUNNERS[args.only](args, torch, C)
        print(json.dumps({"only": args.only, "modes": modes}), flush=True)
        return

    head = measure_layers("c2", args.steps, args.warmup, torch, C, [0])
    wl = head["wl"]
    ms = head["layers"][0]["ms"]
    phase = head["isolated"]
    gcall = head["graph_call"]
    value = wl.n_q / (ms / 1000.0)
    sb = score_bytes(wl, "full")
    # the dominant kernel, k_score_select (FP4 scores of every visible entry and the first
    # Top-K level): the step's scoring call csa2_index_segments launches just that kernel
    # (the last Top-K level runs inside the attention call)
    score_call = "index_segments"
    achieved = sb / (gcall[score_call] / 1000.0) / 1e9
    at_ms = gcall["attn"]
    at_tflops = attn_flops(wl) / (at_ms / 1e3) / 1e12
    at_gbs = attn_bytes(wl) / (at_ms / 1e3) / 1e9
    log(f"step {ms * 1000:.1f} us (graph replay); isolated launches (us): " +
        ", ".join(f"{k}={v * 1000:.1f}" for k, v in phase.items()) + "; per call in graphs (us): " +
        ", ".join(f"{k}={v * 1000:.1f}" for k, v in gcall.items()))
    log(f"k_score_select {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of HBM peak); attention "
        f"{at_tflops:.1f} TFLOP/s ({at_tflops / MFMA_F16_PEAK_TFLOPS:.2%} of fp16 MFMA peak), {at_gbs:.0f} GB/s")
    with torch.cuda.nvtx.range("device copy"):
        copy = device_copy_gbs(torch)
    log(f"device copy {copy['gb_per_s']:.0f} GB/s, read stream {copy['read_gb_per_s']:.0f} GB/s")
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
                   "m": wl.m, "heads": wl.heads, "index_heads": wl.idx_heads, "topk": TOPK, "window": WINDOW},
        "timing": f"HIP events around graph replays; each replay runs {head['per_graph']} consecutive layer "
                  f"steps (a decode step replays its layers as one graph), {args.steps} steps in total",
        "isolated_launch_us": {k: round(v * 1000, 2) for k, v in phase.items()},
        "graph_call_us": {k: round(v * 1000, 2) for k, v in gcall.items()},
        "hbm_frac_step": round(step_bytes(wl, "full") / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm",
                     "kernel": "k_score_select (csa2_index_segments: FP4 scoring of every visible entry + the "
                               "first Top-K level, one launch; the last level runs in the attention call)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "bytes_per_launch": sb,
                     "traffic": measured_traffic(),
                     "frac_of_measured_copy": round(achieved / copy["gb_per_s"], 4),
                     "frac_of_measured_read": round(achieved / copy["read_gb_per_s"], 4),
                     "timing": "HIP events around graph replays of 8 back-to-back csa2_index_segments calls"},
        "attention": {"kernel": "csa2_sparse_attn_topk (k_attn_fc: the last Top-K level, then attention)",
                      "us": round(at_ms * 1e3, 2),
                      "flops_per_launch": attn_flops(wl), "tflops": round(at_tflops, 2),
                      "mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS, "mfma_frac": round(at_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                      "bytes_per_launch": attn_bytes(wl), "gb_per_s": round(at_gbs, 1),
                      "hbm_frac": round(at_gbs / HBM_PEAK_GBS, 4),
                      "timing": "HIP events around graph replays of 8 back-to-back csa2_sparse_attn_topk calls "
                                "(the selection of the last Top-K level included)"},
        "device_copy": copy,
    }
    if not args.no_modes:
        modes = {}
        for name in MODE_RUNNERS:
            modes.update(MODE_RUNNERS[name](args, torch, C))
        result["modes"] = modes
        for k, v in modes.items():
            log(f"  {k}: {v}")
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

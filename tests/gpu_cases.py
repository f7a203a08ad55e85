"""Shared helpers of the GPU parity tests and the smoke check.

Both sides start from the same seeded latents (synth): the HIP path quantises them
with csa2_quantize_kv into device caches, the oracle quantises them with its own
quantiser; the caches are compared byte for byte, then each side runs the layer on
its own copy.
"""
from __future__ import annotations

import functools
import math
import threading

import numpy as np
import torch

from oracle import csa2_oracle as O
from synth import bf16_bits_to_f32, workloads
from synth.workloads import DIM, IDX_DIM, Workload

ROWS_PER_UPLOAD = 1 << 16


def C():
    from fp4_kv_cache_layer_amd import csa2
    return csa2


def swa_ring_latents(wl: Workload, layer: int, seq: int) -> np.ndarray:
    """Latents of the window ring of one sequence: row (p - base) mod cap holds token p,
    for the cap most recent tokens up to the sequence's last query position."""
    sel = wl.q_seq == seq
    hi = int(wl.q_pos[sel].max()) if sel.any() else 0
    cap = wl.swa_cap
    p0 = max(0, hi - cap + 1)
    lat = wl.swa_latents(layer, seq, p0, hi - p0 + 1)
    ring = np.zeros((cap, DIM), np.float32)
    rows = np.mod(np.arange(p0, hi + 1) - wl.swa_base, cap)
    ring[rows] = lat
    return ring


class Case:
    """A workload's inputs on both sides."""

    def __init__(self, wl: Workload, swa_layers=(0,), index_fmt: str = "mxfp4", interleaved: bool = False):
        self.wl = wl
        self.swa_layers = tuple(swa_layers)
        self.index_fmt = index_fmt
        self.interleaved = interleaved   # main KV as one 288-byte record per entry

    # ---------- HIP side ----------
    def gpu_caches(self, window_empty: bool = False):
        """The sequences' caches built by the library's quantiser from the seeded latents;
        window_empty leaves the window rings zero (a prefix-cache miss: the layer steps
        write them)."""
        from fp4_kv_cache_layer_amd.layer import Caches
        wl, C_ = self.wl, C()
        caches = Caches.empty(wl.n_seq, wl.seq_cap, self.swa_layers, wl.swa_cap, index_fmt=self.index_fmt,
                              interleaved=self.interleaved)
        ik_fmt = C_.FMT_NVFP4 if self.index_fmt == "nvfp4" else C_.FMT_MXFP4
        caches.swa_base.fill_(wl.swa_base)
        for b in range(wl.n_seq):
            for r0 in range(0, wl.seq_cap, ROWS_PER_UPLOAD):
                n = min(ROWS_PER_UPLOAD, wl.seq_cap - r0)
                main = wl.main_latents(b, r0, n)
                lat = torch.from_numpy(main).cuda()
                C_.csa2_quantize_kv(lat, C_.FMT_NVFP4, caches.kv_codes[b, r0:r0 + n], caches.kv_scales[b, r0:r0 + n])
                ik = torch.from_numpy(wl.index_k_latents(b, r0, n, main=main)).cuda()
                C_.csa2_quantize_kv(ik, ik_fmt, caches.ik_codes[b, r0:r0 + n], caches.ik_scales[b, r0:r0 + n])
            for L in self.swa_layers if not window_empty else ():
                ring = torch.from_numpy(swa_ring_latents(wl, L, b)).cuda()
                C_.csa2_quantize_kv(ring, C_.FMT_FP8, caches.swa[L][b])
        torch.cuda.synchronize()
        return caches

    def gpu_query_inputs(self, layer: int):
        wl = self.wl
        d = dict(device="cuda")
        q_idx = torch.from_numpy(wl.index_q(layer)).to(**d)
        w = torch.from_numpy(wl.index_w(layer)).to(**d)
        qa = torch.from_numpy(wl.attn_q_bits(layer).view(np.int16)).to(**d).view(torch.bfloat16)
        return q_idx, w, qa

    def gpu_meta(self):
        wl = self.wl
        d = dict(device="cuda")
        return (torch.from_numpy(wl.q_seq.astype(np.int32)).to(**d), torch.from_numpy(wl.n_vis).to(**d),
                torch.from_numpy(wl.q_pos).to(**d), torch.from_numpy(wl.replay_start).to(**d))

    # ---------- oracle side ----------
    def oracle_caches(self, seq: int, n_rows: int | None = None) -> O.PackedCaches:
        wl = self.wl
        n = wl.seq_cap if n_rows is None else n_rows
        kv_c, kv_s = O.quantize_nvfp4(wl.main_latents(seq, 0, n))
        ik_c, ik_s = O.quantize_indexer(wl.index_k_latents(seq, 0, n), self.index_fmt)
        swa = {L: (O.quantize_fp8(swa_ring_latents(wl, L, seq)), wl.swa_base, wl.swa_cap) for L in self.swa_layers}
        return O.PackedCaches(kv_c, kv_s, ik_c, ik_s, swa, self.index_fmt)

    def oracle_query(self, layer: int, qi: int):
        wl = self.wl
        qc, qs = O.quantize_indexer(wl.index_q(layer, qi, 1)[0], self.index_fmt)
        w = wl.index_w(layer, qi, 1)[0]
        qa = bf16_bits_to_f32(wl.attn_q_bits(layer, qi, 1)[0]).astype(np.float64)
        return qc, qs, w, qa


# ---------- acceptance rules ----------

def topk_accept(gpu_idx: np.ndarray, gpu_count: int, positions: np.ndarray, oracle_scores: np.ndarray, k: int):
    """The rule for a GPU Top-K set: size min(k, n), no duplicates, every index a candidate,
    and every chosen index's oracle score >= the oracle's k-th score - 1e-4 |k-th score|."""
    n = positions.size
    want = min(k, n)
    assert gpu_count == want, (gpu_count, want)
    sel = gpu_idx[:gpu_count].astype(np.int64)
    assert np.all(gpu_idx[gpu_count:] == -1)
    assert np.all(np.diff(sel) > 0), "not ascending / duplicates"
    lookup = dict(zip(positions.tolist(), oracle_scores.tolist()))
    assert all(int(p) in lookup for p in sel), "index outside the candidate set"
    if want == 0:
        return 0
    kth = np.sort(oracle_scores)[::-1][want - 1]
    got = np.array([lookup[int(p)] for p in sel])
    bad = got < kth - 1e-4 * abs(kth)
    assert not bad.any(), f"{bad.sum()} chosen indices below the k-th oracle score"
    oracle_set = set(O.topk_positions(oracle_scores, positions, k)[:want].tolist())
    return len(oracle_set - set(sel.tolist()))   # informational: set difference size


def attn_close(out_gpu: np.ndarray, out_ref: np.ndarray, tol: float = 2e-3) -> float:
    err = np.abs(out_gpu.astype(np.float64) - out_ref).max() / np.abs(out_ref).max()
    assert err <= tol, f"attention max-abs error {err:.3g} (normalised) > {tol}"
    return float(err)


def attn_close_bf16(out_bf16: np.ndarray, ref: np.ndarray, tol: float = 2e-3):
    """The bf16 output bar: every element within the fp32 bar (tol x max|ref|) plus one bf16
    ulp of the reference element."""
    ref = np.asarray(ref, np.float64)
    mag = np.abs(ref)
    ulp = np.where(mag > 0, np.ldexp(1.0, np.floor(np.log2(np.where(mag > 0, mag, 1.0))).astype(np.int64) - 7), 0.0)
    err = np.abs(out_bf16.astype(np.float64) - ref)
    bound = tol * mag.max() + ulp
    assert np.all(err <= bound), f"bf16 output: {(err > bound).sum()} elements beyond fp32 bar + 1 ulp"


def smoke_check() -> dict:
    """One Full-mode step of the tiny decode workload on cuda:0 against the oracle."""
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config("c1")
    case = Case(wl)
    caches = case.gpu_caches()
    q_idx, w, qa = case.gpu_query_inputs(0)
    q_seq, n_vis, q_pos, rs = case.gpu_meta()
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap)
    step.full(caches, 0, q_idx, w, qa, q_seq, n_vis, q_pos, rs)
    torch.cuda.synchronize()
    oc = case.oracle_caches(0)
    assert np.array_equal(caches.kv_codes[0].cpu().numpy(), oc.kv_codes)
    assert np.array_equal(caches.ik_codes[0].cpu().numpy(), oc.ik_codes)
    qc, qs, wq, qa_np = case.oracle_query(0, 0)
    n = int(wl.n_vis[0])
    pos, sc = O.full_scores(qc, qs, wq, oc, n)
    idx = step.idx[0].cpu().numpy()
    cnt = int(step.count[0].item())
    miss = topk_accept(idx, cnt, pos, sc, wl.extra.get("k", 512))
    main = oc.main_rows(idx[:cnt])
    swa = oc.swa_rows(0, O.swa_positions(int(wl.q_pos[0]), int(wl.replay_start[0]), 128))
    ref, ref_lse = O.sparse_attention(qa_np, main, swa, 1.0 / math.sqrt(DIM))
    err = attn_close(step.out[0].cpu().numpy(), ref)
    lse_err = float(np.abs(step.lse[0].cpu().numpy() - ref_lse).max())
    assert lse_err <= 1e-3
    return {"topk_set_diff": miss, "attn_err": err, "lse_err": lse_err}


# ---------- full-size layer groups: sampled oracle parity ----------

def oracle_main_rows(wl: Workload, seq: int, positions: np.ndarray):
    """Oracle NVFP4 codes, scales and dequantised rows of one sequence's main-KV entries at
    the given positions (regenerated one by one from the seeded latents)."""
    pos = np.asarray(positions, np.int64)
    lat = np.stack([wl.main_latents(seq, int(p), 1)[0] for p in pos]) if pos.size else np.zeros((0, DIM), np.float32)
    codes, scales = O.quantize_nvfp4(lat)
    return codes, scales, O.dequant_nvfp4(codes, scales)


@functools.lru_cache(maxsize=4)
def _oracle_index_cache(name: str, seq: int, index_fmt: str) -> O.PackedCaches:
    wl = workloads.config(name)
    ik_c, ik_s = O.quantize_indexer(wl.index_k_latents(seq, 0, wl.seq_cap), index_fmt)
    return O.PackedCaches(None, None, ik_c, ik_s, index_fmt=index_fmt)


def oracle_index_cache(wl: Workload, seq: int, index_fmt: str = "mxfp4") -> O.PackedCaches:
    """Oracle caches of one sequence holding the indexer K only (the part scoring reads);
    kept for reuse across tests of the same named workload."""
    if wl.name in workloads.CONFIG_NAMES + workloads.GROUP_NAMES:
        return _oracle_index_cache(wl.name, seq, index_fmt)
    ik_c, ik_s = O.quantize_indexer(wl.index_k_latents(seq, 0, wl.seq_cap), index_fmt)
    return O.PackedCaches(None, None, ik_c, ik_s, index_fmt=index_fmt)


def run_group_snapshots(case: Case, step, caches, window_appends: bool = False, fused_window: bool = False):
    """Runs the workload's layer group on the GPU layer by layer and returns per-layer
    snapshots: idx, count (the set each layer attended over), out, lse, and the pool.
    window_appends: before its calls, each layer writes the FP8 window entry of every query
    row into its own ring (what a layer step does when the window state is not cached).
    fused_window: each row's own window entry is first zeroed in every layer's ring, and the
    layer's attention call appends it (new_win), as the single-token decode step runs; with
    one new entry per row, its main-KV and indexer-K rows are zeroed too and the Full layer's
    scoring call writes them (csa2_append), so that step makes no quantise call either."""
    wl = case.wl
    q_seq, n_vis, q_pos, rs = case.gpu_meta()
    modes = list(wl.layers)
    inputs = [case.gpu_query_inputs(L) for L in range(len(modes))]
    new_wins = None
    if fused_window:
        assert np.unique(wl.q_seq).size == wl.n_q, "the append inside attention needs distinct sequences"
        rows = torch.from_numpy(np.mod(wl.q_pos - wl.swa_base, wl.swa_cap)).long().cuda()
        seqs = torch.from_numpy(wl.q_seq.astype(np.int64)).cuda()
        new_wins = []
        for L in range(len(modes)):
            caches.swa[L][seqs, rows] = 0
            lat = np.stack([wl.swa_latents(L, int(b), int(t), 1)[0] for b, t in zip(wl.q_seq, wl.q_pos)])
            new_wins.append(torch.from_numpy(lat.astype(np.float32)).cuda())
        torch.cuda.synchronize()
    appends = None
    if fused_window and step.appends_in_call():
        # as the decode step is benchmarked: each Full layer's scoring call writes the rows'
        # new main-KV and indexer-K entries (blanked here first) and quantises the indexer Q
        first_new, n_new = int(wl.new_entries[0]), int(wl.new_entries[1])
        if n_new == 1:
            seqs = torch.from_numpy(wl.q_seq.astype(np.int64)).cuda()
            for t in (caches.kv_codes, caches.kv_scales, caches.ik_codes, caches.ik_scales):
                t[seqs, first_new] = 0
            app = (torch.full((wl.n_q,), first_new, dtype=torch.int64, device="cuda"),
                   torch.from_numpy(np.stack([wl.main_latents(int(b), first_new, 1)[0] for b in wl.q_seq])).cuda(),
                   torch.from_numpy(np.stack([wl.index_k_latents(int(b), first_new, 1)[0] for b in wl.q_seq])).cuda())
            appends = [app if m.startswith("full") else None for m in modes]
            torch.cuda.synchronize()
    calls = step.run_group(caches, modes, inputs, q_seq, n_vis, q_pos, rs, bind=True, new_wins=new_wins,
                           appends=appends)
    snaps, at = [], 0
    # the calls of each layer as the step plans them (the flat list is cut by these counts)
    plan = step.plan(modes, appends)
    assert sum(len(n) for n in plan) == len(calls)
    for L, names in enumerate(plan):
        if window_appends:
            C_ = C()
            lat = np.stack([wl.swa_latents(L, int(b), int(t), 1)[0] for b, t in zip(wl.q_seq, wl.q_pos)])
            dst = torch.from_numpy(wl.q_seq.astype(np.int64) * wl.swa_cap
                                   + np.mod(wl.q_pos - wl.swa_base, wl.swa_cap)).cuda()
            C_.csa2_quantize_kv(torch.from_numpy(lat).cuda(), C_.FMT_FP8, caches.swa[L].view(-1, DIM), None, dst)
        for fn in calls[at:at + len(names)]:
            fn()
        at += len(names)
        torch.cuda.synchronize()
        snaps.append({"idx": step.idx.cpu().numpy().copy(), "count": step.count.cpu().numpy().copy(),
                      "out": step.out.cpu().numpy().copy(), "lse": step.lse.cpu().numpy().copy(),
                      "pool": step.pool.cpu().numpy().copy(), "pool_count": step.pool_count.cpu().numpy().copy()})
    return snaps


def gather_group_row(case: Case, caches, snaps, qi: int, window: int = 128) -> dict:
    """The device bytes the oracle checks of one query row need (read on the calling thread):
    its sequence's indexer-K cache, and per layer the main-KV rows of the set it attended
    and the window rows of its key range."""
    wl = case.wl
    seq = int(wl.q_seq[qi])
    t, s = int(wl.q_pos[qi]), int(wl.replay_start[qi])
    rows = np.mod(O.swa_positions(t, s, window) - wl.swa_base, wl.swa_cap)
    rows_t = torch.from_numpy(rows).cuda()
    g = {"ik_codes": caches.ik_codes[seq].cpu().numpy(), "ik_scales": caches.ik_scales[seq].cpu().numpy(),
         "kv_codes": [], "kv_scales": [], "swa": []}
    for L in range(len(wl.layers)):
        snap = snaps[L]
        sel = torch.from_numpy(snap["idx"][qi][:int(snap["count"][qi])].astype(np.int64)).cuda()
        g["kv_codes"].append(caches.kv_codes[seq][sel].cpu().numpy())
        g["kv_scales"].append(caches.kv_scales[seq][sel].cpu().numpy())
        g["swa"].append(caches.swa[L][seq][rows_t].cpu().numpy())
    return g


# The oracle's matrix products (scores over a whole cache, attention logits) go through the
# BLAS library, whose own thread pool is not to be entered by several of our threads at once:
# concurrent 1M-entry products from a thread pool gave wrong scores on a 16-core host.  Those
# calls take this lock; the quantisation (most of the oracle's time) stays parallel.
_BLAS_LOCK = threading.Lock()


def _full_scores(*a, **kw):
    with _BLAS_LOCK:
        return O.full_scores(*a, **kw)


def _sparse_attention(*a, **kw):
    with _BLAS_LOCK:
        return O.sparse_attention(*a, **kw)


def check_group_rows(case: Case, caches, snaps, rows, workers: int = 8, shared_index: bool = False, **kw) -> list:
    """check_group_query for many rows: the device bytes are read first on this thread,
    then the oracle work runs on a thread pool (numpy releases the interpreter lock in its
    array loops; the BLAS calls are serialised).  The first failing row raises, with its row
    number."""
    from concurrent.futures import ThreadPoolExecutor
    rows = list(rows)
    data = {qi: gather_group_row(case, caches, snaps, qi, kw.get("window", 128)) for qi in rows}
    shared = {}
    if shared_index:   # few sequences, many rows each (a prefill chunk): one oracle cache each
        for seq in sorted({int(case.wl.q_seq[qi]) for qi in rows}):
            oc = oracle_index_cache(case.wl, seq, case.index_fmt)
            oc.ik_deq(case.wl.seq_cap)   # dequantised once, before the threads read it
            shared[seq] = oc

    def one(qi):
        try:
            return check_group_query(case, None, snaps, qi, gpu=data[qi],
                                     oracle_index=shared.get(int(case.wl.q_seq[qi])), **kw)
        except AssertionError as e:
            raise AssertionError(f"query row {qi}: {e}") from e

    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(one, rows))


def check_group_query(case: Case, caches, snaps, qi: int, k: int = 512, window: int = 128,
                      block: int = 8, max_blocks: int = 2048, gpu: dict | None = None,
                      oracle_index: O.PackedCaches | None = None) -> dict:
    """Oracle parity of one query row through every layer of the group.  Index sets and the
    pool pass the oracle's acceptance rules; each layer's attention is compared with the
    oracle's over the set the GPU attended (so a legitimate near-tie swap upstream does not
    fail the attention check)."""
    wl = case.wl
    seq, nv = int(wl.q_seq[qi]), int(wl.n_vis[qi])
    t, s = int(wl.q_pos[qi]), int(wl.replay_start[qi])
    if gpu is None:
        gpu = gather_group_row(case, caches, snaps, qi, window)
        oc = oracle_index_cache(wl, seq, case.index_fmt)
    elif oracle_index is not None:   # shared read-only by check_group_rows' threads
        oc = oracle_index
    else:   # a thread of check_group_rows: a cache of its own, nothing shared
        ik_c, ik_s = O.quantize_indexer(wl.index_k_latents(seq, 0, wl.seq_cap), case.index_fmt)
        oc = O.PackedCaches(None, None, ik_c, ik_s, index_fmt=case.index_fmt)
    assert np.array_equal(gpu["ik_codes"], oc.ik_codes)
    assert np.array_equal(gpu["ik_scales"], oc.ik_scales)
    stats = {"set_diff": []}
    pool = None
    for L, mode in enumerate(wl.layers):
        snap = snaps[L]
        idx, cnt = snap["idx"][qi], int(snap["count"][qi])
        if mode != "reuse":
            qc, qs, w, _ = case.oracle_query(L, qi)
            cand = pool_pos = None
            if mode == "reindex_pool":
                pool_pos = O.pool_positions(pool, nv, block)
                cand = pool_pos
            pos, sc = _full_scores(qc, qs, w, oc, nv, cand)
            stats["set_diff"].append(topk_accept(idx, cnt, pos, sc, k))
            if mode == "full_pool":
                bs = O.block_scores(sc, nv, block)
                pool = snap["pool"][qi]
                topk_accept(pool, int(snap["pool_count"][qi]), np.arange(bs.size), bs, max_blocks)
        else:
            assert np.array_equal(idx, snaps[L - 1]["idx"][qi])   # borrowed, untouched
        sel = idx[:cnt]
        codes, scales, main = oracle_main_rows(wl, seq, sel)
        assert np.array_equal(gpu["kv_codes"][L], codes)
        assert np.array_equal(gpu["kv_scales"][L], scales)
        swa = O.quantize_fp8(swa_ring_latents(wl, L, seq))
        rows = np.mod(O.swa_positions(t, s, window) - wl.swa_base, wl.swa_cap)
        assert np.array_equal(gpu["swa"][L], swa[rows])
        _, _, _, qa = case.oracle_query(L, qi)
        ref, ref_lse = _sparse_attention(qa, main, O.dequant_fp8(swa[rows]), 1.0 / math.sqrt(DIM))
        attn_close(snap["out"][qi], ref)
        assert np.abs(snap["lse"][qi] - ref_lse).max() <= 1e-3
    return stats

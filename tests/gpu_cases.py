"""Shared helpers of the GPU parity tests and the smoke check.

Both sides start from the same seeded latents (synth): the HIP path quantises them
with csa2_quantize_kv into device caches, the oracle quantises them with its own
quantiser; the caches are compared byte for byte, then each side runs the layer on
its own copy.
"""
from __future__ import annotations

import math

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

    def __init__(self, wl: Workload, swa_layers=(0,)):
        self.wl = wl
        self.swa_layers = tuple(swa_layers)

    # ---------- HIP side ----------
    def gpu_caches(self):
        from fp4_kv_cache_layer_amd.layer import Caches
        wl, C_ = self.wl, C()
        caches = Caches.empty(wl.n_seq, wl.seq_cap, self.swa_layers, wl.swa_cap)
        caches.swa_base.fill_(wl.swa_base)
        for b in range(wl.n_seq):
            for r0 in range(0, wl.seq_cap, ROWS_PER_UPLOAD):
                n = min(ROWS_PER_UPLOAD, wl.seq_cap - r0)
                lat = torch.from_numpy(wl.main_latents(b, r0, n)).cuda()
                C_.csa2_quantize_kv(lat, C_.FMT_NVFP4, caches.kv_codes[b, r0:r0 + n], caches.kv_scales[b, r0:r0 + n])
                ik = torch.from_numpy(wl.index_k_latents(b, r0, n)).cuda()
                C_.csa2_quantize_kv(ik, C_.FMT_MXFP4, caches.ik_codes[b, r0:r0 + n], caches.ik_scales[b, r0:r0 + n])
            for L in self.swa_layers:
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
        ik_c, ik_s = O.quantize_mxfp4(wl.index_k_latents(seq, 0, n))
        swa = {L: (O.quantize_fp8(swa_ring_latents(wl, L, seq)), wl.swa_base, wl.swa_cap) for L in self.swa_layers}
        return O.PackedCaches(kv_c, kv_s, ik_c, ik_s, swa)

    def oracle_query(self, layer: int, qi: int):
        wl = self.wl
        qc, qs = O.quantize_mxfp4(wl.index_q(layer, qi, 1)[0])
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

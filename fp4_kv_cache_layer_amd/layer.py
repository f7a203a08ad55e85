"""Layer-mode driver for the CSA2 layer step (host orchestration only).

[W] "CSA2：跨层复用，能借就不自己算" and Figure 4: every CSA2 layer is statically one of
  Full    -- its own global KV and indexer K, fresh Top-K indices,
  Reindex -- the previous layer's global KV, its own indexer Q re-scoring it,
  Reuse   -- the previous layer's KV and Top-K indices; attention only,
and every layer keeps its own global Q and its own sliding-window KV.
[W] "分层稀疏索引器" and Figure 5: the decoder's first Full layer builds a pool of at
most 2,048 blocks x 8 positions by max indexer score; later Reindex layers pick their
Top-K inside it.

This module only allocates buffers and sequences calls into the C ABI; it moves no
data itself.  One `Csa2Step` holds the buffers of a batch of query rows; `full`,
`reindex` and `reuse` run one layer each on the caller's stream.  With bind=True they
return the layer's calls as a list of zero-argument callables with every argument
validated and marshalled once, for tight decode loops.
"""
from __future__ import annotations

import math

import torch

from . import csa2 as C


MODES = ("full", "full_pool", "reuse", "reindex", "reindex_pool")
# indexer Q/K formats: MXFP4 (E8M0 per 32 channels, the scaled FP4 matrix-core path) or the
# main KV's NVFP4-style format (E4M3 per 16 channels, dequantised to fp16 MFMAs)
INDEX_FORMATS = {"mxfp4": (C.FMT_MXFP4, 32), "nvfp4": (C.FMT_NVFP4, 16)}


def plan_group(modes, fused: bool = True, group: int = 1, index_fmt: str = "mxfp4",
               attn_select: bool = False, pool_select=None, group_select: bool = True, q_in_call=None) -> list:
    """Checks a layer group's mode sequence and returns the calls each layer makes.

    [W] "CSA2：跨层复用，能借就不自己算" and Figure 4: a Reindex layer re-scores the KV of the
    Full layer before it, a Reuse layer borrows the index set of the last scoring layer, so
    a group opens with a Full layer.  [W] "分层稀疏索引器": only the decoder's first Full
    layer builds the pool, and Reindex-in-pool layers need it.  Raises ValueError for a
    sequence that breaks these rules.  group > 1: the query rows come in groups of `group`
    rows of one sequence, and the layers that score all visible entries read each group's
    indexer K once: fused (and group_select), scored and selected without a score array
    (csa2_index_topk_grouped); otherwise csa2_index_score_grouped, then csa2_topk.  index_fmt "nvfp4": the
    fused pool build and grouped scoring exist for MXFP4 only, so the pool-building layer
    scores, selects and builds the pool in separate calls, and group must be 1.
    attn_select (fused, group 1, and a cache whose segment survivors fit one selection,
    i.e. up to 131,072 entries at k = 512): Full and Reindex layers without a pool keep
    only the first Top-K level in the scoring call (csa2_index_segments) and finish the
    selection inside their attention call (csa2_sparse_attn_topk), which also writes the
    index set for the Reuse layers; Reindex layers inside the pool write the pool's slot
    scores and select inside their attention call (csa2_sparse_attn_pool_topk).  With the
    MXFP4 indexer those slot scores come from csa2_index_score_q, which quantises the
    layer's indexer Q itself, so such a layer (which appends nothing) makes no quantise
    call.  q_in_call (default: MXFP4 indexer, group 1): the scoring call of every Reindex
    layer (which appends nothing) reads the unquantised indexer Q and quantises it itself
    (the call names end in "_q"), so such a layer makes no quantise launch; a Full layer
    keeps its quantise launch, which also carries the step's appends of new entries (one
    launch either way, and a quantised Q keeps the scoring kernel's prologue short).
    Grouped scoring takes quantised Q only."""
    if index_fmt not in INDEX_FORMATS:
        raise ValueError(f"unknown indexer format {index_fmt!r}")
    if index_fmt != "mxfp4" and group > 1:
        raise ValueError("grouped scoring reads an MXFP4 indexer only")
    if q_in_call is None:
        q_in_call = index_fmt == "mxfp4" and group == 1
    if q_in_call and (index_fmt != "mxfp4" or group > 1):
        raise ValueError("an unquantised indexer Q is read by the ungrouped MXFP4 scoring calls only")
    plan, have_kv, have_pool = [], False, False
    for i, m in enumerate(modes):
        if m not in MODES:
            raise ValueError(f"layer {i}: unknown mode {m!r}")
        if m.startswith("full"):
            have_kv, have_pool = True, m == "full_pool"
        elif not have_kv:
            raise ValueError(f"layer {i}: {m} needs a Full layer before it in the group")
        if m == "reindex_pool" and not have_pool:
            raise ValueError(f"layer {i}: reindex_pool needs a pool built by the group's Full layer")
        if m == "reuse":
            calls = ["attend"]
        elif m == "full_pool":
            calls = (["quantize_index_q", "index_topk_pool", "attend"] if fused and index_fmt == "mxfp4" else
                     ["quantize_index_q", "score", "select", "build_pool", "attend"])
        elif group > 1 and m in ("full", "reindex"):
            calls = (["quantize_index_q", "index_topk_grouped", "attend"] if fused and group_select else
                     ["quantize_index_q", "score_grouped", "select", "attend"])
        elif attn_select and fused and m in ("full", "reindex"):
            calls = ["quantize_index_q", "index_segments", "attend_topk"]
        elif (attn_select if pool_select is None else pool_select) and fused and group == 1 and m == "reindex_pool":
            calls = (["score_pool_q", "attend_pool_topk"] if index_fmt == "mxfp4" else
                     ["quantize_index_q", "score_pool", "attend_pool_topk"])
        elif fused:
            calls = ["quantize_index_q", "index_topk_in_pool" if m == "reindex_pool" else "index_topk", "attend"]
        else:
            pool = m == "reindex_pool"
            calls = ["quantize_index_q", "score_pool" if pool else "score", "select_pool" if pool else "select",
                     "attend"]
        if q_in_call and m.startswith("reindex") and calls[0] == "quantize_index_q":
            calls = [c + "_q" if c.startswith(("score", "index_")) and not c.endswith("_q") else c for c in calls[1:]]
        plan.append(calls)
    return plan


class Caches:
    """Device caches of a layer group: main KV (NVFP4), indexer K (MXFP4, or NVFP4 with
    index_fmt "nvfp4"), and the per-layer FP8 window caches with their ring bases."""

    def __init__(self, kv_codes, kv_scales, ik_codes, ik_scales, swa: dict, swa_base):
        self.kv_codes, self.kv_scales = kv_codes, kv_scales
        self.ik_codes, self.ik_scales = ik_codes, ik_scales
        self.swa = swa              # layer -> [n_seq, swa_cap, 512] uint8
        self.swa_base = swa_base    # [n_seq] int64

    @property
    def seq_cap(self) -> int:
        return self.kv_codes.shape[1]

    @staticmethod
    def empty(n_seq: int, seq_cap: int, swa_layers, swa_cap: int, dim: int = 512, idx_dim: int = 128,
              device="cuda", index_fmt: str = "mxfp4", interleaved: bool = False):
        """interleaved: the main KV as one record per entry, its dim/2 code bytes followed by
        its dim/16 scale bytes (288 bytes at dim 512, [W] "FP4 与 SWA Bounded Replay"); codes and
        scales are then two strided views of it."""
        u8 = dict(dtype=torch.uint8, device=device)
        per = INDEX_FORMATS[index_fmt][1]
        if interleaved:
            rec = torch.zeros(n_seq, seq_cap, dim // 2 + dim // 16, **u8)
            kv_codes, kv_scales = rec[..., :dim // 2], rec[..., dim // 2:]
        else:
            kv_codes, kv_scales = torch.zeros(n_seq, seq_cap, dim // 2, **u8), torch.zeros(n_seq, seq_cap, dim // 16, **u8)
        return Caches(kv_codes, kv_scales,
                      torch.zeros(n_seq, seq_cap, idx_dim // 2, **u8), torch.zeros(n_seq, seq_cap, idx_dim // per, **u8),
                      {L: torch.zeros(n_seq, swa_cap, dim, **u8) for L in swa_layers},
                      torch.zeros(n_seq, dtype=torch.int64, device=device))


class Csa2Step:
    """Buffers and calls for one batch of query rows through the layers of a group."""

    def __init__(self, n_q: int, n_heads: int, idx_heads: int, seq_cap: int, k: int = 512, window: int = 128,
                 block: int = 8, max_blocks: int = 2048, idx_dim: int = 128, dim: int = 512,
                 out_dtype=torch.float32, fused: bool = True, group: int = 1, index_fmt: str = "mxfp4",
                 attn_select: bool = True, device="cuda"):
        """fused: score and select in one call (csa2_index_topk) wherever the layer does not
        need the score array itself (it does only when it builds the pool).  group: query
        rows come in groups of `group` consecutive rows of one sequence (several tokens of a
        sequence at once); layers scoring all visible entries then read each group's indexer
        K once.  index_fmt: the indexer Q/K format ("mxfp4" or "nvfp4", see INDEX_FORMATS).
        attn_select: finish the Top-K inside the attention call where plan_group allows it
        (the survivors of up to 131,072 entries at k = 512); False keeps the last selection
        level as a launch of its own (csa2_index_topk, then csa2_sparse_attn)."""
        plan_group(["full"], fused, group, index_fmt)   # validates the combination
        C.csa2_init()   # device check; the device status word the kernels report into
        n_cand = C.csa2_segment_keys(seq_cap, k)
        fits = fused and group == 1 and 1 <= n_cand <= 8192
        # inside a pool the attention call selects from at most 16,384 slots
        self.pool_select = bool(attn_select) and fused and group == 1 and max_blocks * block <= 16384
        self.attn_select = bool(attn_select) and fits
        # grouped rows: the fused selection keeps one wave per row and range busy, which pays
        # once the groups alone give the GPU a few hundred workgroups (a prefill chunk's
        # hundreds of groups); a few groups (several decode tokens of a few sequences) keep
        # the grouped scores and the Top-K levels
        self.group_select = fused and group > 1 and (n_q + group - 1) // group >= 128
        self.index_fmt = index_fmt
        # Reindex layers' scoring calls quantise the indexer Q themselves (no quantise launch)
        self.q_in_call = index_fmt == "mxfp4" and group == 1
        self.idx_qfmt, self.idx_group = INDEX_FORMATS[index_fmt]
        self.n_q, self.n_heads, self.idx_heads = n_q, n_heads, idx_heads
        self.fused, self.group = fused, group
        self.seq_cap, self.k, self.window = seq_cap, k, window
        self.block, self.max_blocks, self.dim = block, max_blocks, dim
        dev = dict(device=device)
        self.qi_codes = torch.empty(n_q, idx_heads, idx_dim // 2, dtype=torch.uint8, **dev)
        self.qi_scales = torch.empty(n_q, idx_heads, idx_dim // self.idx_group, dtype=torch.uint8, **dev)
        self.scores = torch.empty(n_q, max(seq_cap, max_blocks * block), dtype=torch.float32, **dev)
        self.idx = torch.empty(n_q, k, dtype=torch.int32, **dev)
        self.count = torch.empty(n_q, dtype=torch.int32, **dev)
        self.pool = torch.empty(n_q, max_blocks, dtype=torch.int32, **dev)
        self.pool_count = torch.empty(n_q, dtype=torch.int32, **dev)
        self.out = torch.empty(n_q, n_heads, dim, dtype=out_dtype, **dev)
        self.lse = torch.empty(n_q, n_heads, dtype=torch.float32, **dev)
        n_slots = max(seq_cap, max_blocks * block, 1)
        self.ws_topk = torch.empty(max(C.csa2_topk_workspace_bytes(n_q, n_slots, k), 1), dtype=torch.uint8, **dev)
        self.ws_index_topk = torch.empty(max(C.csa2_index_topk_workspace_bytes(n_q, max(seq_cap, 1), k),
                                             C.csa2_index_topk_workspace_bytes(n_q, max_blocks * block, k, True), 1),
                                         dtype=torch.uint8, **dev)
        self.ws_index_topk_pool = torch.empty(
            max(C.csa2_index_topk_pool_workspace_bytes(n_q, max(seq_cap, 1), k, block, max_blocks), 1),
            dtype=torch.uint8, **dev)
        self.ws_pool = torch.empty(max(C.csa2_pool_workspace_bytes(n_q, max(seq_cap, 1), block, max_blocks), 1),
                                   dtype=torch.uint8, **dev)
        self.ws_attn = torch.empty(max(C.csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window), 1),
                                   dtype=torch.uint8, **dev)
        self.cand_keys = torch.empty(n_q, max(n_cand, 1), dtype=torch.int64, **dev)
        self.ws_grouped = torch.empty(max(C.csa2_index_topk_grouped_workspace_bytes(n_q, seq_cap, k, group), 1)
                                      if self.group_select else 1, dtype=torch.uint8, **dev)
        self.sm_scale = 1.0 / math.sqrt(dim)

    # ---- steps ----
    def quantize_index_q(self, q_f32, bind=False):
        """indexer Q [n_q, H_I, d] f32 -> the indexer format (per query, per head, per 32
        channels for MXFP4, per 16 for NVFP4)."""
        n_q, h, d = q_f32.shape
        return C.csa2_quantize_kv(q_f32.view(n_q * h, d), self.idx_qfmt, self.qi_codes.view(n_q * h, d // 2),
                                  self.qi_scales.view(n_q * h, d // self.idx_group), _bind=bind)

    def _q(self, q):
        """The indexer-Q operands of a scoring call: the step's quantised Q, or (q given)
        the unquantised Q, which the call quantises itself."""
        return (self.qi_codes, self.qi_scales) if q is None else (q, None)

    def score(self, caches: Caches, w, q_seq, n_vis, in_pool: bool = False, bind=False):
        if in_pool:
            return C.csa2_index_score(self.qi_codes, self.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis,
                                      self.scores, self.pool, self.pool_count, self.block, fmt=self.idx_qfmt,
                                      _bind=bind)
        return C.csa2_index_score(self.qi_codes, self.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis,
                                  self.scores, fmt=self.idx_qfmt, _bind=bind)

    def score_q(self, caches: Caches, q_index_f32, w, q_seq, n_vis, in_pool: bool = False, bind=False):
        """Slot scores from the unquantised indexer Q (MXFP4, quantised inside the call)."""
        self._mx_only("scoring from an unquantised Q")
        if in_pool:
            return C.csa2_index_score_q(q_index_f32, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis, self.scores,
                                        self.pool, self.pool_count, self.block, _bind=bind)
        return C.csa2_index_score_q(q_index_f32, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis, self.scores,
                                    _bind=bind)

    def _mx_only(self, what):
        if self.index_fmt != "mxfp4":
            raise ValueError(f"{what} reads an MXFP4 indexer only")

    def score_grouped(self, caches: Caches, w, q_seq, n_vis, bind=False):
        self._mx_only("grouped scoring")
        return C.csa2_index_score_grouped(self.qi_codes, self.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq,
                                          n_vis, self.group, self.scores, _bind=bind)

    def index_topk_grouped(self, caches: Caches, w, q_seq, n_vis, bind=False):
        """grouped scoring and selection in one pass, without the score array."""
        self._mx_only("grouped scoring")
        return C.csa2_index_topk_grouped(self.qi_codes, self.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq,
                                         n_vis, self.group, self.k, self.idx, self.count, self.ws_grouped, _bind=bind)

    def select(self, n_vis, in_pool: bool = False, bind=False):
        if in_pool:
            return C.csa2_topk(self.scores, n_vis, self.seq_cap, self.k, self.idx, self.count, self.ws_topk,
                               self.pool, self.pool_count, self.block, _bind=bind)
        return C.csa2_topk(self.scores, n_vis, self.seq_cap, self.k, self.idx, self.count, self.ws_topk, _bind=bind)

    def index_topk(self, caches: Caches, w, q_seq, n_vis, in_pool: bool = False, bind=False, q=None, append=None):
        """score + select in one pass, without the score array.  q: the unquantised indexer Q
        (MXFP4: the call quantises it), else the step's quantised Q (as for the calls below).
        append: the step's new entries, written by the call itself (see Csa2Step.appends)."""
        pool = (self.pool, self.pool_count) if in_pool else (None, None)
        return C.csa2_index_topk(*self._q(q), w, caches.ik_codes, caches.ik_scales, q_seq, n_vis,
                                 self.k, self.idx, self.count, self.ws_index_topk, pool[0], pool[1], self.block,
                                 fmt=self.idx_qfmt, append=self._app(caches, append), _bind=bind)

    def index_topk_build_pool(self, caches: Caches, w, q_seq, n_vis, bind=False, q=None, append=None):
        """score + select + pool in one pass (the decoder's first Full layer)."""
        self._mx_only("the fused pool build")
        return C.csa2_index_topk_pool(*self._q(q), w, caches.ik_codes, caches.ik_scales, q_seq,
                                      n_vis, self.k, self.idx, self.count, self.pool, self.pool_count, self.block,
                                      self.ws_index_topk_pool, append=self._app(caches, append), _bind=bind)

    def index_segments(self, caches: Caches, w, q_seq, n_vis, bind=False, q=None, append=None):
        """the first Top-K level alone (its survivors feed attend_topk)."""
        return C.csa2_index_segments(*self._q(q), w, caches.ik_codes, caches.ik_scales, q_seq, n_vis,
                                     self.k, self.cand_keys, fmt=self.idx_qfmt, append=self._app(caches, append),
                                     _bind=bind)

    @staticmethod
    def _app(caches: Caches, append):
        """(row, main latents, indexer-K latents) -> the binding's csa2_append, main-KV rows into
        `caches`."""
        if append is None:
            return None
        row, main, index = append
        return {"row": row, "main": main, "index": index, "kv_codes": caches.kv_codes, "kv_scales": caches.kv_scales}

    def attend_topk(self, caches: Caches, layer: int, q_attn, q_seq, q_pos, replay_start, out=None, lse=None,
                    bind=False, new_win=None):
        """attention that first selects the Top-K from index_segments' survivors and writes it
        to the step's index set.  new_win: see attend."""
        return C.csa2_sparse_attn_topk(q_attn, caches.kv_codes, caches.kv_scales, q_seq, self.cand_keys, self.k,
                                       self.idx, self.count, caches.swa[layer], caches.swa_base, q_pos, replay_start,
                                       self.window, self.sm_scale, self.out if out is None else out,
                                       self.lse if lse is None else lse, self.ws_attn, new_win=new_win, _bind=bind)

    def attend_pool_topk(self, caches: Caches, layer: int, q_attn, q_seq, n_vis, q_pos, replay_start, out=None,
                         lse=None, bind=False, new_win=None):
        """attention that first selects the Top-K from the pool's slot scores (score with
        in_pool=True before) and writes it to the step's index set."""
        return C.csa2_sparse_attn_pool_topk(q_attn, caches.kv_codes, caches.kv_scales, q_seq, self.scores, n_vis,
                                            self.pool, self.pool_count, self.block, self.k, self.idx, self.count,
                                            caches.swa[layer], caches.swa_base, q_pos, replay_start, self.window,
                                            self.sm_scale, self.out if out is None else out,
                                            self.lse if lse is None else lse, self.ws_attn, new_win=new_win,
                                            _bind=bind)

    def _score_select(self, caches, w, q_seq, n_vis, in_pool, bind, q=None):
        if self.fused:
            return [self.index_topk(caches, w, q_seq, n_vis, in_pool, bind, q)]
        if q is not None:
            return [self.score_q(caches, q, w, q_seq, n_vis, in_pool, bind), self.select(n_vis, in_pool, bind)]
        return [self.score(caches, w, q_seq, n_vis, in_pool, bind), self.select(n_vis, in_pool, bind)]

    def build_pool(self, n_vis, bind=False):
        return C.csa2_build_pool(self.scores, n_vis, self.seq_cap, self.pool, self.pool_count, self.block,
                                 self.ws_pool, _bind=bind)

    def attend(self, caches: Caches, layer: int, q_attn, q_seq, q_pos, replay_start, out=None, lse=None,
               bind=False, new_win=None):
        """new_win: [n_q, D] window latents of each row's own token, appended to the layer's
        window cache by the attention call itself (rows of distinct sequences only)."""
        return C.csa2_sparse_attn(q_attn, caches.kv_codes, caches.kv_scales, q_seq, self.idx, caches.swa[layer],
                                  caches.swa_base, q_pos, replay_start, self.window, self.sm_scale,
                                  self.out if out is None else out, self.lse if lse is None else lse, self.ws_attn,
                                  new_win=new_win, _bind=bind)

    def run_group(self, caches: Caches, modes, inputs, q_seq, n_vis, q_pos, replay_start, outs=None, lses=None,
                  bind=False, new_wins=None, appends=None):
        """Runs the layers of a group in order.  inputs[i] = (indexer Q f32 [n_q, H_I, d] or
        None for Reuse, w [n_q, H_I] or None, attention Q bf16 [n_q, H, D]); layer i attends
        with its own window cache caches.swa[i].  outs/lses: optional per-layer outputs
        (default: the step's own buffers, overwritten by each layer).  new_wins: optional
        per-layer window latents of each row's own token, appended by the layer's attention
        call (see attend).  appends: optional per-layer new entries of Full layers, written
        by their scoring call (see full; the layer then makes no quantise call).  With
        bind=True returns the group's calls as one flat list of callables."""
        plan = self.plan(modes, appends)
        calls = []
        for i, (m, names) in enumerate(zip(modes, plan)):
            q_index, w, q_attn = inputs[i]
            out = None if outs is None else outs[i]
            lse = None if lses is None else lses[i]
            nw = None if new_wins is None else new_wins[i]
            app = None if appends is None else appends[i]
            for name in names:
                # "_q" (or a scoring call with appends): it reads the unquantised indexer Q itself
                qq = q_index if name.endswith("_q") or app is not None else None
                base = name[:-2] if name.endswith("_q") else name
                if name == "quantize_index_q":
                    c = self.quantize_index_q(q_index, bind)
                elif base == "index_topk_pool":
                    c = self.index_topk_build_pool(caches, w, q_seq, n_vis, bind, q=qq, append=app)
                elif base in ("index_topk", "index_topk_in_pool"):
                    c = self.index_topk(caches, w, q_seq, n_vis, base.endswith("in_pool"), bind, q=qq, append=app)
                elif name == "score_grouped":
                    c = self.score_grouped(caches, w, q_seq, n_vis, bind)
                elif name == "index_topk_grouped":
                    c = self.index_topk_grouped(caches, w, q_seq, n_vis, bind)
                elif name in ("score", "score_pool"):
                    c = self.score(caches, w, q_seq, n_vis, name.endswith("pool"), bind)
                elif name in ("score_q", "score_pool_q"):
                    c = self.score_q(caches, q_index, w, q_seq, n_vis, name == "score_pool_q", bind)
                elif name in ("select", "select_pool"):
                    c = self.select(n_vis, name.endswith("pool"), bind)
                elif name == "build_pool":
                    c = self.build_pool(n_vis, bind)
                elif base == "index_segments":
                    c = self.index_segments(caches, w, q_seq, n_vis, bind, q=qq, append=app)
                elif name == "attend_topk":
                    c = self.attend_topk(caches, i, q_attn, q_seq, q_pos, replay_start, out, lse, bind, new_win=nw)
                elif name == "attend_pool_topk":
                    c = self.attend_pool_topk(caches, i, q_attn, q_seq, n_vis, q_pos, replay_start, out, lse, bind,
                                              new_win=nw)
                else:
                    c = self.attend(caches, i, q_attn, q_seq, q_pos, replay_start, out, lse, bind, new_win=nw)
                calls.append(c)
        return calls if bind else None

    def plan(self, modes, appends=None) -> list:
        """The calls of each layer as run_group makes them (plan_group with this step's
        options; a Full layer with appends drops its quantise call)."""
        plan = plan_group(modes, self.fused, self.group, self.index_fmt, self.attn_select,
                          pool_select=self.pool_select, group_select=self.group_select, q_in_call=self.q_in_call)
        if appends is None:
            return plan
        for i, m in enumerate(modes):
            if appends[i] is None:
                continue
            if not m.startswith("full") or not self.appends_in_call():
                raise ValueError(f"layer {i}: appends go to a Full layer's fused MXFP4 scoring call")
            plan[i] = [n for n in plan[i] if n != "quantize_index_q"]
        return plan

    # ---- layer modes ----
    @staticmethod
    def _seq(calls, bind):
        return calls if bind else None

    def appends_in_call(self) -> bool:
        """Whether a Full layer's scoring call can write the step's new entries itself
        (csa2_append: the fused MXFP4 scoring calls, one row per query)."""
        return self.fused and self.index_fmt == "mxfp4" and self.group == 1

    def full(self, caches, layer, q_index_f32, w, q_attn, q_seq, n_vis, q_pos, replay_start, make_pool=False,
             out=None, lse=None, bind=False, append=None, new_win=None):
        """append: None, or (row [n_q] int64, main latents [n_q, 512], indexer-K latents
        [n_q, 128]) of each query's new entry (queries of distinct sequences; row < 0: none),
        written by the scoring call, which then also quantises the indexer Q itself: with
        new_win (the window entries, appended by the attention call) the layer step makes no
        quantise launch.  Without append the step quantises its indexer Q in a launch of its
        own, which a caller may extend with its appends (csa2_quantize_kv_multi)."""
        if append is not None and not self.appends_in_call():
            raise ValueError("appends inside the scoring call need the fused MXFP4 path with group 1")
        q = q_index_f32 if append is not None else None
        calls = [] if q is not None else [self.quantize_index_q(q_index_f32, bind)]
        if make_pool and self.fused and self.index_fmt == "mxfp4":
            calls.append(self.index_topk_build_pool(caches, w, q_seq, n_vis, bind, q=q, append=append))
        elif make_pool:
            calls += [self.score(caches, w, q_seq, n_vis, bind=bind), self.select(n_vis, bind=bind),
                      self.build_pool(n_vis, bind)]
        elif self.attn_select:
            calls += [self.index_segments(caches, w, q_seq, n_vis, bind, q=q, append=append),
                      self.attend_topk(caches, layer, q_attn, q_seq, q_pos, replay_start, out, lse, bind,
                                       new_win=new_win)]
            return self._seq(calls, bind)
        else:
            calls += ([self.index_topk(caches, w, q_seq, n_vis, False, bind, q, append)] if append is not None else
                      self._score_select(caches, w, q_seq, n_vis, False, bind))
        calls.append(self.attend(caches, layer, q_attn, q_seq, q_pos, replay_start, out, lse, bind, new_win=new_win))
        return self._seq(calls, bind)

    def reindex(self, caches, layer, q_index_f32, w, q_attn, q_seq, n_vis, q_pos, replay_start, in_pool=False,
                out=None, lse=None, bind=False):
        q = q_index_f32 if self.q_in_call else None
        quant = [] if q is not None else [self.quantize_index_q(q_index_f32, bind)]
        if self.attn_select and not in_pool:
            calls = quant + [self.index_segments(caches, w, q_seq, n_vis, bind, q=q),
                             self.attend_topk(caches, layer, q_attn, q_seq, q_pos, replay_start, out, lse, bind)]
            return self._seq(calls, bind)
        if self.pool_select and in_pool:
            if self.index_fmt == "mxfp4":
                calls = [self.score_q(caches, q_index_f32, w, q_seq, n_vis, True, bind)]
            else:
                calls = [self.quantize_index_q(q_index_f32, bind), self.score(caches, w, q_seq, n_vis, True, bind)]
            calls.append(self.attend_pool_topk(caches, layer, q_attn, q_seq, n_vis, q_pos, replay_start, out, lse,
                                               bind))
            return self._seq(calls, bind)
        calls = quant + [*self._score_select(caches, w, q_seq, n_vis, in_pool, bind, q),
                         self.attend(caches, layer, q_attn, q_seq, q_pos, replay_start, out, lse, bind)]
        return self._seq(calls, bind)

    def reuse(self, caches, layer, q_attn, q_seq, q_pos, replay_start, out=None, lse=None, bind=False):
        return self._seq([self.attend(caches, layer, q_attn, q_seq, q_pos, replay_start, out, lse, bind)], bind)

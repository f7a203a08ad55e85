"""Shapes of the CSA2 workloads and the seeded tensors that feed them.

Every workload is a set of sequences with a compressed main-KV cache
(``seq_cap`` entries each, compression ratio ``m``), an indexer-K cache on the
same entries, a per-layer FP8 sliding-window cache, and a set of query rows
(one per decoding sequence, or every token of a prefill chunk).

Value recipe (all seeded, see ``synth.c``):
  main-KV latent   N(0,1)^512 -> RMS norm (unit weight) -> rotary embedding on
                   the last 64 channels at position entry*m, fp32
  indexer-K latent a fixed seeded projection of the main-KV latent of the same
                   entry: channel c = (+-x[c] +- x[c+128] +- x[c+256] +- x[c+384]) / 2
                   with seeded signs (a stand-in for the learned projection: about
                   unit variance per channel, and the indexer ranks the same token
                   states the attention reads), fp32
  SWA latent       as the main latent, one row per token position, per layer
  indexer Q        N(0,1)^(H_I*128), fp32, per layer and query row
  indexer weight   U(0,1)^H_I, fp32, per layer and query row
  attention Q      N(0,1)^(H*512) rounded to bf16, per layer and query row
"""
from __future__ import annotations

from dataclasses import dataclass, field

import functools
import math

import numpy as np

from . import (ATTN_Q, INDEX_PROJ, INDEX_Q, INDEX_W, MAIN_LATENT, SWA_LATENT,
               latent_rows, normal_bf16_bits, normal_f32, tensor_id, uniform_f32)

DIM = 512          # main-KV latent channels
IDX_DIM = 128      # indexer head dimension
TOPK = 512         # entries kept per query
WINDOW = 128       # sliding-window length
BLOCK = 8          # pool block size (positions)
MAX_BLOCKS = 2048  # pool capacity in blocks



@functools.lru_cache(maxsize=4)
def index_projection(seed: int) -> np.ndarray:
    """The fixed projection from the main-KV latent to the indexer-K latent: indexer channel
    c is (s0*x[c] + s1*x[c+128] + s2*x[c+256] + s3*x[c+384]) / 2 with seeded signs s
    (every main channel feeds one indexer channel).  Returns the signs, [4, 128] f32."""
    u = uniform_f32(seed, tensor_id(INDEX_PROJ), 0, DIM)
    return np.where(u < 0.5, -1.0, 1.0).astype(np.float32).reshape(4, IDX_DIM)


@dataclass
class Workload:
    name: str
    seed: int
    n_seq: int
    seq_cap: int                 # main-KV entries allocated per sequence
    m: int                       # tokens per compressed entry
    heads: int                   # attention heads
    idx_heads: int               # indexer heads
    q_seq: np.ndarray            # [n_q] int32 sequence of each query row
    q_pos: np.ndarray            # [n_q] int64 absolute token position of each query
    replay_start: np.ndarray     # [n_q] int64 replay start s of each query
    layers: tuple                # layer modes in order: full, full_pool, reuse, reindex, reindex_pool
    new_entries: tuple           # (first, count) entries quantized inside the step
    swa_cap: int = WINDOW        # SWA ring rows per sequence (row = (pos - base) mod cap)
    swa_base: int = 0
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_q(self) -> int:
        return int(self.q_seq.shape[0])

    @property
    def n_vis(self) -> np.ndarray:
        """Visible compressed entries per query: only complete blocks of m tokens."""
        return ((self.q_pos + 1) // self.m).astype(np.int64)

    # ----- seeded tensors (host numpy) -----
    def main_latents(self, seq: int, row0: int, rows: int) -> np.ndarray:
        return latent_rows(self.seed, tensor_id(MAIN_LATENT, 0, seq), row0, rows, DIM, 64, self.m)

    def index_k_latents(self, seq: int, row0: int, rows: int, main: np.ndarray | None = None) -> np.ndarray:
        """Rows [row0, row0+rows) of the indexer-K latent: the main-KV latent of the same
        entries (`main`, when the caller already holds those rows) through the fixed seeded
        projection of index_projection, so each channel keeps unit variance and the indexer
        ranks the same token states the attention reads.  f32 sums in a fixed order (exactly
        reproducible)."""
        s = index_projection(self.seed)
        if main is None:
            main = self.main_latents(seq, row0, rows)
        x = [main[:, IDX_DIM * j:IDX_DIM * (j + 1)] * s[j] for j in range(4)]
        return ((x[0] + x[1]) + (x[2] + x[3])) * np.float32(0.5)

    def swa_latents(self, layer: int, seq: int, pos0: int, count: int) -> np.ndarray:
        return latent_rows(self.seed, tensor_id(SWA_LATENT, layer, seq), pos0, count, DIM, 64, 1)

    def index_q(self, layer: int, q0: int = 0, nq: int | None = None) -> np.ndarray:
        nq = self.n_q - q0 if nq is None else nq
        n = self.idx_heads * IDX_DIM
        return normal_f32(self.seed, tensor_id(INDEX_Q, layer), q0 * n, nq * n).reshape(
            nq, self.idx_heads, IDX_DIM)

    def index_w(self, layer: int, q0: int = 0, nq: int | None = None) -> np.ndarray:
        nq = self.n_q - q0 if nq is None else nq
        h = self.idx_heads
        return uniform_f32(self.seed, tensor_id(INDEX_W, layer), q0 * h, nq * h).reshape(nq, h)

    def attn_q_bits(self, layer: int, q0: int = 0, nq: int | None = None) -> np.ndarray:
        nq = self.n_q - q0 if nq is None else nq
        n = self.heads * DIM
        return normal_bf16_bits(self.seed, tensor_id(ATTN_Q, layer), q0 * n, nq * n).reshape(
            nq, self.heads, DIM)

    def swa_positions_needed(self, seq: int) -> tuple:
        """Token positions whose SWA rows any query of `seq` can read: [lo, hi]."""
        sel = self.q_seq == seq
        t = self.q_pos[sel]
        s = self.replay_start[sel]
        lo = int(np.maximum(s, t - WINDOW + 1).min())
        return lo, int(t.max())


def decode(name: str, seed: int, batch: int, n_entries: int, heads: int, idx_heads: int,
           layers=("full",), description: str = "") -> Workload:
    """Batched decode at m=1: query b is the newest token of sequence b, which sees all entries."""
    q_pos = np.full(batch, n_entries - 1, dtype=np.int64)
    return Workload(name=name, seed=seed, n_seq=batch, seq_cap=n_entries, m=1, heads=heads,
                    idx_heads=idx_heads, q_seq=np.arange(batch, dtype=np.int32), q_pos=q_pos,
                    replay_start=np.zeros(batch, dtype=np.int64), layers=tuple(layers),
                    new_entries=(n_entries - 1, 1), description=description)


def multi_token_decode(name: str, seed: int, batch: int, tokens: int, n_entries: int, heads: int,
                       idx_heads: int, description: str = "") -> Workload:
    """Several decode tokens of each sequence at once (draft tokens verified together): the
    last `tokens` positions of sequence b are query rows tokens*b .. tokens*b + tokens - 1,
    each seeing the entries up to its own position (m = 1)."""
    q_seq = np.repeat(np.arange(batch), tokens).astype(np.int32)
    q_pos = np.tile(np.arange(n_entries - tokens, n_entries), batch).astype(np.int64)
    wl = Workload(name=name, seed=seed, n_seq=batch, seq_cap=n_entries, m=1, heads=heads, idx_heads=idx_heads,
                  q_seq=q_seq, q_pos=q_pos, replay_start=np.zeros(batch * tokens, dtype=np.int64),
                  layers=("full",), new_entries=(n_entries - tokens, tokens), description=description)
    wl.extra["tokens_per_seq"] = tokens
    return wl


def prefill(name: str, seed: int, prefix_tokens: int, chunk_tokens: int, m: int, heads: int,
            idx_heads: int, description: str = "", layers=("full",), swa_miss: bool = False) -> Workload:
    """One sequence: a cached prefix, then a chunk of new tokens.  The query rows are the
    last WINDOW prefix tokens (bounded replay from s = prefix - WINDOW) and the new tokens.
    swa_miss: the prefix's window state is not cached (a prefix-cache miss): every layer
    writes the window entries of all its query rows, replay rows included, before attending."""
    s = prefix_tokens - WINDOW
    q_pos = np.arange(s, prefix_tokens + chunk_tokens, dtype=np.int64)
    total_entries = (prefix_tokens + chunk_tokens) // m
    first_new = prefix_tokens // m
    wl = Workload(name=name, seed=seed, n_seq=1, seq_cap=total_entries, m=m, heads=heads,
                  idx_heads=idx_heads, q_seq=np.zeros(q_pos.shape[0], dtype=np.int32), q_pos=q_pos,
                  replay_start=np.full(q_pos.shape[0], s, dtype=np.int64), layers=tuple(layers),
                  new_entries=(first_new, total_entries - first_new),
                  swa_cap=chunk_tokens + WINDOW, swa_base=s, description=description)
    wl.extra["counted_rows"] = chunk_tokens
    wl.extra["swa_miss"] = swa_miss
    return wl


def encoder_modes() -> tuple:
    """One encoder CSA2 group ([W] "CSA2：跨层复用，能借就不自己算": the encoder's 18 CSA2
    layers at m = 2 form 3 groups of 6, one Full layer and 5 Reuse layers each)."""
    return ("full",) + ("reuse",) * 5


def decoder_modes() -> tuple:
    """The decoder's 20 CSA2 layers ([W] "CSA2：跨层复用，能借就不自己算": five groups, the
    first Full + 3 Reuse, then four of Reindex + 3 Reuse; [W] "分层稀疏索引器": the first Full
    layer builds the shared candidate pool and the Reindex layers search only inside it)."""
    return ("full_pool",) + ("reuse",) * 3 + (("reindex_pool",) + ("reuse",) * 3) * 4


def config(name: str) -> Workload:
    """The five workloads: tiny decode, 128K batched decode, one layer group at 128K,
    1M decode with the candidate pool, and an m=2 encoder prefill chunk."""
    if name == "c1":
        return decode("c1", 0, 1, 4096, 16, 8, ("full",),
                      "tiny Full decode: 1 query, 16 heads, 4,096 entries, 8 indexer heads")
    if name == "c2":
        return decode("c2", 1, 64, 131072, 64, 16, ("full",),
                      "batched Full decode: 64 queries x 128K entries, 64 heads, 16 indexer heads")
    if name == "c3":
        return decode("c3", 2, 32, 131072, 64, 16, ("full", "reuse", "reuse", "reuse", "reindex"),
                      "layer group: Full + 3 Reuse + Reindex, 32 queries x 128K entries")
    if name == "c4":
        return decode("c4", 3, 8, 1048576, 64, 16,
                      ("full_pool", "reindex_pool", "reindex_pool", "reindex_pool", "reindex_pool"),
                      "1M decode: Full + pool, then 4 Reindex inside the 16,384-position pool")
    if name == "c5":
        return prefill("c5", 4, 262144, 4096, 2, 64, 16,
                       "encoder prefill chunk: 4,096 tokens after a 262,144-token prefix, m=2")
    if name == "enc_group":
        return prefill("enc_group", 7, 262144, 4096, 2, 64, 16,
                       "encoder group prefill (Full + 5 Reuse, m=2) of a 4,096-token chunk after a "
                       "262,144-token prefix, prefix-cache miss: 128 replay rows rebuild the window",
                       layers=encoder_modes(), swa_miss=True)
    if name == "mtd_128k":
        return multi_token_decode("mtd_128k", 8, 16, 4, 131072, 64, 16,
                                  "multi-token decode: 16 sequences x 4 tokens verified at once, 128K entries, "
                                  "Full layer")
    if name == "dec_128k":
        return decode("dec_128k", 5, 32, 131072, 64, 16, decoder_modes(),
                      "decoder step: the 20 CSA2 layers of one decode token, 32 queries x 128K entries")
    if name == "dec_1m":
        return decode("dec_1m", 6, 8, 1048576, 64, 16, decoder_modes(),
                      "decoder step: the 20 CSA2 layers of one decode token, 8 queries x 1M entries")
    raise KeyError(name)


CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")
DECODER_NAMES = ("dec_128k", "dec_1m")   # whole decoder steps (all 20 CSA2 layers)
GROUP_NAMES = DECODER_NAMES + ("enc_group", "mtd_128k")   # workloads beyond the five configs

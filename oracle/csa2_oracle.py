"""CPU oracle for one CSA2 (Compressed Sparse Attention 2) layer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

Plain numpy, fp64 arithmetic throughout, no blocking or fusion: each function is
the definition (or the method's steps in the pages' order) written out so it can
be checked against the sources by eye.

Sources, cited by page and section:
  [W]  shibing624.github.io walkthrough "一个 token 只花 890 字节：DeepSeek-V4.1-Flash
       把 KV 缓存压到了什么程度" -- sections "CSA2：跨层复用，能借就不自己算" (with
       Figure 4), "分层稀疏索引器" (with Figure 5), "FP4 与 SWA Bounded Replay".
  [J]  jdon.com article "557亿参数只唤醒80亿！DeepSeek把AI记忆砍掉437倍还拿了第一！" --
       sections "三条路线打架" and "缓存压缩真的是越大越好吗".
  [L]  m.lsln.cn summary of the report -- "4.3 消融实验 / Ablation Study" and
       "五、相关工作 / Related Work".
  [MX]  OCP Microscaling Formats (MX) Specification v1.0 (E2M1 element, E8M0 scale,
        shared-exponent rule).
  [FP8] OCP 8-bit Floating Point Specification (E4M3 with no infinities).

Readings where the pages are silent (each also listed in the design notes):
  * score(q, j) = sum_h w[q,h] * ReLU(q_h . k_j)  (the published DeepSeek-V3.2
    lightning-indexer form; the pages only say a lightweight indexer scores the
    main KV with indexer Q/K).            -- parity unpinned for the formula choice
  * indexer Q/K are MXFP4 (E2M1 + E8M0 per 32); the main KV is E2M1 + E4M3 per 16.
    The page leaves the indexer's scale format open, so the NVFP4-style alternative (the
    main KV's format, E4M3 per 16) is served too: `index_fmt="nvfp4"`.
  * rounding is to nearest with ties to the even code; scales saturate.
  * a compressed entry j is visible to token t iff (j+1)*m <= t+1.
  * ties in Top-K / pool ranking go to the lower position; outputs are ascending.
  * the sliding-window cache holds the same 512-channel entry as the main KV
    (K = V), unscaled E4M3.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------------------
# Codecs  [MX] E2M1 / E8M0, [FP8] E4M3.  Tables are built from the format definitions.
# --------------------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = man * 0.5                      # 0.M x 2^(1-1)
    else:
        mag = (1.0 + man * 0.5) * 2.0 ** (exp - 1)
    return sign * mag


def e4m3_value(code: int) -> float:
    """E4M3 (OCP 'FN'): bias 7, exponent 0 is subnormal, S.1111.111 is NaN, no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return sign * mag


def e8m0_value(code: int) -> float:
    """E8M0: an unsigned power of two 2^(code-127); 0xFF is NaN."""
    return math.nan if code == 0xFF else 2.0 ** (code - 127)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

# the non-negative finite grids, ascending, with their codes
_E2M1_POS_CODES = np.arange(8)
_E2M1_POS_VALUES = E2M1[:8]
_E4M3_POS_CODES = np.arange(0x7F)            # 0x00 .. 0x7E (0x7F is NaN)
_E4M3_POS_VALUES = E4M3[:0x7F]


def nearest_code(target: np.ndarray, values: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Code of the grid value nearest to each non-negative target; ties go to the even
    code (round-half-to-even on the code's last mantissa bit); targets beyond the
    grid saturate to its largest value.  `values` ascending."""
    target = np.asarray(target, dtype=np.float64)
    hi = np.clip(np.searchsorted(values, target, side="left"), 0, len(values) - 1)
    lo = np.clip(hi - 1, 0, len(values) - 1)
    d_lo = np.abs(target - values[lo])
    d_hi = np.abs(values[hi] - target)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    return np.where(pick_hi, codes[hi], codes[lo]).astype(np.int64)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """channel 2i -> low nibble of byte i, channel 2i+1 -> high nibble."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------------------
# Quantisers
# --------------------------------------------------------------------------------------


def quantize_nvfp4(x: np.ndarray):
    """Main-KV quantisation: E2M1 values with one E4M3 scale per 16 channels and no
    second-level global scale, applied to the post-RoPE latent.
    [W] "FP4 与 SWA Bounded Replay" (format and placement after RoPE);
    [L] 4.3 and 5 (global scale omitted, quantised after RoPE); [J] "缓存压缩真的是越大越好吗"
    (range 448 x 6).

    Per group: scale = E4M3 value nearest to amax/6 (saturating at 448); every element
    is the E2M1 value nearest to |x|/scale (saturating at 6) with the sign of x.
    A group whose scale rounds to 0 stores signed zeros.
    Returns (codes uint8 [rows, D/2], scales uint8 [rows, D/16])."""
    x = np.asarray(x, dtype=np.float64)
    rows, d = x.shape
    if d % 16:
        raise ValueError("dim must be a multiple of 16")
    g = x.reshape(rows, d // 16, 16)
    amax = np.abs(g).max(axis=-1)
    scale_code = nearest_code(amax / 6.0, _E4M3_POS_VALUES, _E4M3_POS_CODES)
    s = E4M3[scale_code]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.abs(g) / s[..., None]
    r = np.where(s[..., None] > 0, r, 0.0)
    mag = nearest_code(r, _E2M1_POS_VALUES, _E2M1_POS_CODES)
    codes = mag | (np.signbit(g).astype(np.int64) << 3)
    return _pack_nibbles(codes.reshape(rows, d)), scale_code.astype(np.uint8)


def quantize_mxfp4(x: np.ndarray):
    """Indexer Q/K quantisation, MXFP4 [MX]: per 32 channels a shared power-of-two scale
    2^E with E = floor(log2 amax) - 2 (2 = the E2M1 maximum exponent), clamped to the
    E8M0 range; elements are x / 2^E rounded to E2M1, saturating at 6.  An all-zero group
    gets scale code 0.  Reading of [W] "FP4 与 SWA Bounded Replay" (indexer Q/K in FP4)
    and [L] 5 (OCP MXFP4 chosen for hardware compatibility).
    Returns (codes uint8 [rows, D/2], scales uint8 [rows, D/32])."""
    x = np.asarray(x, dtype=np.float64)
    rows, d = x.shape
    if d % 32:
        raise ValueError("dim must be a multiple of 32")
    g = x.reshape(rows, d // 32, 32)
    amax = np.abs(g).max(axis=-1)
    _, e = np.frexp(amax)                    # amax = f * 2^e with f in [0.5, 1)
    exp = np.clip(e.astype(np.int64) - 1 - 2, -127, 127)
    scale_code = np.where(amax > 0, exp + 127, 0)
    r = np.abs(g) / np.ldexp(1.0, (scale_code - 127))[..., None]
    mag = nearest_code(r, _E2M1_POS_VALUES, _E2M1_POS_CODES)
    codes = mag | (np.signbit(g).astype(np.int64) << 3)
    return _pack_nibbles(codes.reshape(rows, d)), scale_code.astype(np.uint8)


def quantize_fp8(x: np.ndarray) -> np.ndarray:
    """Sliding-window KV in FP8: each value is the E4M3 value nearest to x, saturating at
    +-448, no scale.  [J] "缓存压缩真的是越大越好吗" and [L] 4.3 (SWA KV kept in FP8)."""
    x = np.asarray(x, dtype=np.float64)
    mag = nearest_code(np.abs(x), _E4M3_POS_VALUES, _E4M3_POS_CODES)
    return (mag | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = E2M1[unpack_nibbles(codes)]
    s = E4M3[np.asarray(scales, dtype=np.int64)]
    return vals * np.repeat(s, 16, axis=-1)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = E2M1[unpack_nibbles(codes)]
    s = E8M0[np.asarray(scales, dtype=np.int64)]
    return vals * np.repeat(s, 32, axis=-1)


def dequant_fp8(codes: np.ndarray) -> np.ndarray:
    return E4M3[np.asarray(codes, dtype=np.int64)]


INDEX_FORMATS = ("mxfp4", "nvfp4")


def quantize_indexer(x: np.ndarray, index_fmt: str = "mxfp4"):
    """Indexer Q / K rows in the chosen format: MXFP4 (the reading above) or the NVFP4-style
    alternative, E2M1 with one E4M3 scale per 16 channels as for the main KV.
    [W] "FP4 与 SWA Bounded Replay" (indexer Q/K in FP4; the scale format is not given)."""
    if index_fmt == "mxfp4":
        return quantize_mxfp4(x)
    if index_fmt == "nvfp4":
        return quantize_nvfp4(x)
    raise ValueError(index_fmt)


def dequant_indexer(codes: np.ndarray, scales: np.ndarray, index_fmt: str = "mxfp4") -> np.ndarray:
    if index_fmt == "mxfp4":
        return dequant_mxfp4(codes, scales)
    if index_fmt == "nvfp4":
        return dequant_nvfp4(codes, scales)
    raise ValueError(index_fmt)


# --------------------------------------------------------------------------------------
# Indexer scoring, Top-K, candidate pool
# --------------------------------------------------------------------------------------


def visible_entries(t: int, m: int) -> int:
    """Entries of an m-token compressor whose whole block ends at or before token t."""
    return (t + 1) // m


def index_scores(q_deq: np.ndarray, w: np.ndarray, k_deq: np.ndarray) -> np.ndarray:
    """Indexer scores of one query over candidate entries.
    q_deq [H_I, d] dequantised indexer Q, w [H_I] head weights, k_deq [n, d] dequantised
    indexer K.  score_j = sum_h w_h * max(0, q_h . k_j).
    [W] "CSA2：跨层复用，能借就不自己算" (lightweight indexer scores the global main KV with
    indexer Q/K); formula: reading (DeepSeek-V3.2 lightning indexer)."""
    dots = np.asarray(k_deq, np.float64) @ np.asarray(q_deq, np.float64).T    # [n, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float64)


def topk_positions(scores: np.ndarray, positions: np.ndarray, k: int) -> np.ndarray:
    """The k best candidates ranked by (score descending, position ascending), returned as
    ascending positions padded with -1 to length k.  [W] "CSA2…" (Top-K = 512)."""
    scores = np.asarray(scores, np.float64)
    positions = np.asarray(positions, np.int64)
    order = np.lexsort((positions, -scores))
    chosen = np.sort(positions[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.size] = chosen
    return out


def block_scores(scores: np.ndarray, n_vis: int, block: int) -> np.ndarray:
    """Per aligned block of `block` positions: the max score over its visible positions."""
    n_blk = -(-n_vis // block)
    return np.array([np.max(scores[b * block: min((b + 1) * block, n_vis)]) for b in range(n_blk)],
                    dtype=np.float64)


def build_pool(scores: np.ndarray, n_vis: int, block: int = 8, max_blocks: int = 2048) -> np.ndarray:
    """Hierarchical sparse indexer: the Full layer's candidate pool is the (at most)
    max_blocks aligned blocks of `block` positions with the highest max indexer score.
    Ascending block ids, -1 padded.  [W] "分层稀疏索引器" and Figure 5 (blocks chosen by max
    indexer score; at most 2,048 blocks x 8 positions)."""
    bs = block_scores(scores, n_vis, block)
    return topk_positions(bs, np.arange(bs.size), max_blocks)


def pool_positions(blocks: np.ndarray, n_vis: int, block: int = 8) -> np.ndarray:
    """Visible positions covered by the pool's blocks, ascending."""
    b = np.asarray(blocks, np.int64)
    b = b[b >= 0]
    pos = (b[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return pos[pos < n_vis]


# --------------------------------------------------------------------------------------
# Sliding window with bounded replay, sparse attention
# --------------------------------------------------------------------------------------


def swa_positions(t: int, s: int, window: int = 128) -> np.ndarray:
    """Sliding-window keys of the query at token t after a replay from token s:
    positions [max(s, t-W+1), t].  [W] "FP4 与 SWA Bounded Replay"."""
    return np.arange(max(s, t - window + 1), t + 1, dtype=np.int64)


def attention(q: np.ndarray, keys: np.ndarray, sm_scale: float):
    """Softmax attention of H heads over one key set with V = K (the shared entry).
    q [H, D], keys [n, D].  Returns (out [H, D], lse [H]) with lse the natural-log
    normaliser M + ln Z."""
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    logits = sm_scale * (q @ keys.T)                 # [H, n]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    z = e.sum(axis=1, keepdims=True)
    out = (e @ keys) / z
    return out, (mx + np.log(z))[:, 0]


def sparse_attention(q: np.ndarray, main_rows: np.ndarray, swa_rows: np.ndarray, sm_scale: float):
    """One softmax over the union of the selected main-KV entries (dequantised FP4) and the
    query's sliding-window entries (dequantised FP8); no de-duplication between the two
    caches, no sink, no bias.  [W] "CSA2…" (Top-K entries plus the layer's own sliding
    window), "FP4 与 SWA Bounded Replay" (cached FP4 values are dequantised before attention)."""
    keys = np.concatenate([np.asarray(main_rows, np.float64).reshape(-1, q.shape[1]),
                           np.asarray(swa_rows, np.float64).reshape(-1, q.shape[1])], axis=0)
    return attention(q, keys, sm_scale)


# --------------------------------------------------------------------------------------
# Layer modes (Full / Reindex / Reuse) over packed caches
# --------------------------------------------------------------------------------------


class PackedCaches:
    """Packed caches of one sequence, exactly as stored in HBM:
    kv_codes [N, D/2] u8, kv_scales [N, D/16] u8 (main KV, NVFP4);
    ik_codes [N, d/2] u8, ik_scales [N, d/32] u8 (indexer K, MXFP4; [N, d/16] with
    index_fmt "nvfp4");
    swa: dict layer -> (codes [cap, D] u8 E4M3, base, cap) with row(p) = (p - base) mod cap."""

    def __init__(self, kv_codes, kv_scales, ik_codes, ik_scales, swa=None, index_fmt: str = "mxfp4"):
        self.kv_codes, self.kv_scales = kv_codes, kv_scales
        self.ik_codes, self.ik_scales = ik_codes, ik_scales
        self.swa = swa or {}
        self.index_fmt = index_fmt
        self._ik_deq = None

    def ik_deq(self, n: int) -> np.ndarray:
        if self._ik_deq is None or self._ik_deq.shape[0] < n:
            self._ik_deq = dequant_indexer(self.ik_codes[:n], self.ik_scales[:n], self.index_fmt)
        return self._ik_deq[:n]

    def main_rows(self, positions: np.ndarray) -> np.ndarray:
        p = np.asarray(positions, np.int64)
        p = p[p >= 0]
        return dequant_nvfp4(self.kv_codes[p], self.kv_scales[p])

    def swa_rows(self, layer: int, positions: np.ndarray) -> np.ndarray:
        codes, base, cap = self.swa[layer]
        rows = np.mod(np.asarray(positions, np.int64) - base, cap)
        return dequant_fp8(codes[rows])


def full_scores(q_codes, q_scales, w, caches: PackedCaches, n_vis: int, cand=None) -> tuple:
    """Scores of one query over all visible entries (cand None) or over given candidate
    positions.  Returns (positions, scores).  The indexer Q is in the caches' indexer format."""
    qd = dequant_indexer(q_codes, q_scales, caches.index_fmt)
    kd = caches.ik_deq(n_vis)
    pos = np.arange(n_vis, dtype=np.int64) if cand is None else np.asarray(cand, np.int64)
    return pos, index_scores(qd, w, kd[pos])


def layer_step(mode: str, *, q_codes=None, q_scales=None, w=None, caches: PackedCaches,
               layer: int, q_attn, t: int, s: int, n_vis: int, k: int = 512, window: int = 128,
               sm_scale: float = 1.0 / math.sqrt(512), borrowed_idx=None, pool=None,
               build_pool_blocks: int = 0, block: int = 8):
    """One CSA2 layer for one query row.  [W] "CSA2…" and Figure 4:
      full    -- scores every visible entry with its own indexer Q, keeps the Top-K
                 (and, for the decoder's first Full layer, builds the candidate pool);
      reindex -- uses the previous layer's global KV, re-scores with its own indexer Q
                 (inside the pool when there is one, [W] "分层稀疏索引器"), keeps the Top-K;
      reuse   -- borrows the index set as well and only attends.
    Every mode attends with its own Q and its own sliding window.
    Returns dict(idx, out, lse, pool, scores)."""
    res = {}
    if mode in ("full", "reindex"):
        cand = None if pool is None else pool_positions(pool, n_vis, block)
        pos, sc = full_scores(q_codes, q_scales, w, caches, n_vis, cand)
        res["scores"] = (pos, sc)
        idx = topk_positions(sc, pos, k)
        if mode == "full" and build_pool_blocks:
            res["pool"] = build_pool(sc, n_vis, block, build_pool_blocks)
    elif mode == "reuse":
        idx = np.asarray(borrowed_idx, np.int64)
    else:
        raise ValueError(mode)
    res["idx"] = idx
    main = caches.main_rows(idx)
    swa = caches.swa_rows(layer, swa_positions(t, s, window))
    res["out"], res["lse"] = sparse_attention(q_attn, main, swa, sm_scale)
    return res


# --------------------------------------------------------------------------------------
# Sizes (global KV per token) -- [W] summary and Figure 1b (890 bytes per token)
# --------------------------------------------------------------------------------------


def nvfp4_entry_bytes(dim: int = 512) -> int:
    return dim // 2 + dim // 16


def mxfp4_entry_bytes(dim: int = 128) -> int:
    return dim // 2 + dim // 32


def layer_schedule():
    """CSA2 layer modes of the model: encoder 18 layers at m=2 in 3 groups of
    (1 Full + 5 Reuse); decoder 20 layers at m=1: (1 Full + 3 Reuse), then 4 groups of
    (1 Reindex + 3 Reuse).  [W] "CSA2…".  Returns a list of (part, m, mode)."""
    sched = []
    for _ in range(3):
        sched += [("encoder", 2, "full")] + [("encoder", 2, "reuse")] * 5
    sched += [("decoder", 1, "full")] + [("decoder", 1, "reuse")] * 3
    for _ in range(4):
        sched += [("decoder", 1, "reindex")] + [("decoder", 1, "reuse")] * 3
    return sched


def global_kv_bytes_per_token(main_dim: int = 512, idx_dim: int = 128) -> float:
    """Bytes of HBM-resident global KV per token: one main-KV entry plus one indexer-K
    entry per Full layer's cache, divided by that cache's compression ratio."""
    per_entry = nvfp4_entry_bytes(main_dim) + mxfp4_entry_bytes(idx_dim)
    return sum(per_entry / m for _, m, mode in layer_schedule() if mode == "full")

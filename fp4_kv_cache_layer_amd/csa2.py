"""Python binding of the CSA2 C ABI (include/csa2.h): argument marshalling only.

Each function has the C entry point's name, takes torch tensors (device memory and the
current stream are torch's), checks shapes and dtypes, passes raw pointers to
libcsa2.so and raises Csa2Error on a non-zero status.  Every step runs in the HIP
kernels; there is no other code path.  If the library is missing or cannot load, the
first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported before libcsa2.so so that the process holds a single HIP runtime

from .build import LIB_PATH

FMT_NVFP4, FMT_MXFP4, FMT_FP8 = 0, 1, 2
FMT_MXFP4_Q_F32, FMT_MXFP4_Q_BF16 = 3, 4   # MXFP4 indexer, Q given unquantised (scoring calls)
DT_F32, DT_BF16 = 0, 1
MAX_TOPK = 2048

_lib = None


class Csa2Error(RuntimeError):
    pass


def _hip_runtimes_mapped() -> set:
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return set()


def lib() -> ctypes.CDLL:
    """Load libcsa2.so (built by __graft_entry__.build()); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Csa2Error(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise Csa2Error(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    vp, i64, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    sig = {
        "csa2_version": ([], i32),
        "csa2_init": ([], i32),
        "csa2_device_status": ([i32], ctypes.c_uint32),
        "csa2_debug_set_wait_limit": ([i32], i32),
        "csa2_status_string": ([i32], ctypes.c_char_p),
        "csa2_last_error": ([], ctypes.c_char_p),
        "csa2_quantize_kv": ([vp, i32, i64, i32, i32, vp, i64, vp, i64, vp, i64, vp], i32),
        "csa2_quantize_kv_multi": ([vp, i32, vp], i32),
        "csa2_index_score_grouped": ([vp, vp, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp,
                                      i32, vp, i64, vp], i32),
        "csa2_index_score": ([vp, vp, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, vp, vp,
                              i32, i32, vp, i64, vp], i32),
        "csa2_index_score_q": ([vp, i32, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, vp, vp,
                                i32, i32, vp, i64, vp], i32),
        "csa2_index_topk": ([vp, vp, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, vp, vp,
                             i32, i32, i32, vp, vp, vp, sz, vp, vp], i32),
        "csa2_index_topk_workspace_bytes": ([i32, i64, i32, i32], sz),
        "csa2_index_topk_grouped": ([vp, vp, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp,
                                     i32, i32, vp, vp, vp, sz, vp], i32),
        "csa2_index_topk_grouped_workspace_bytes": ([i32, i64, i32, i32], sz),
        "csa2_index_topk_pool": ([vp, vp, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, i32,
                                  vp, vp, i32, i32, vp, vp, vp, sz, vp, vp], i32),
        "csa2_index_topk_pool_workspace_bytes": ([i32, i64, i32, i32, i32], sz),
        "csa2_topk": ([vp, i64, i32, vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp], i32),
        "csa2_topk_workspace_bytes": ([i32, i64, i32], sz),
        "csa2_build_pool": ([vp, i64, i32, vp, i64, i32, i32, vp, vp, vp, sz, vp], i32),
        "csa2_pool_workspace_bytes": ([i32, i64, i32, i32], sz),
        "csa2_sparse_attn": ([vp, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, i32, vp, i64, i64, i64,
                              vp, vp, vp, vp, i32, i32, f32, vp, i32, vp, vp, sz, vp], i32),
        "csa2_attn_workspace_bytes": ([i32, i32, i32, i32, i32], sz),
        "csa2_sparse_attn_noalloc": ([vp, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, i32, vp, i64,
                                      i64, i64, vp, vp, vp, vp, i32, i32, f32, vp, i32, vp, vp], i32),
        "csa2_sparse_attn_noalloc_max_bytes": ([], sz),
        "csa2_index_segments": ([vp, vp, vp, i32, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, i32,
                                 vp, vp, vp], i32),
        "csa2_segment_keys": ([i64, i32], i64),
        "csa2_sparse_attn_topk": ([vp, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, i32, i32, vp, vp,
                                   vp, i64, i64, i64, vp, vp, vp, vp, i32, i32, f32, vp, i32, vp, vp, sz, vp], i32),
        "csa2_sparse_attn_pool_topk": ([vp, i32, i32, i32, vp, i64, i64, vp, i64, i64, i64, i32, vp, vp, i64, vp, vp,
                                        vp, i32, i32, i32, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, i32, i32, f32,
                                        vp, i32, vp, vp, sz, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _run(name: str, args: tuple, bind: bool):
    """Call the C entry point now, or (bind=True) return a zero-argument callable that
    repeats the call with the same pointers, sizes and stream (validated once)."""
    fn = getattr(lib(), name)
    if bind:
        def call():
            _check(fn(*args), name)
        call.__name__ = name
        return call
    _check(fn(*args), name)
    return None


def _check(rc: int, name: str):
    if rc != 0:
        L = lib()
        msg = L.csa2_status_string(rc).decode()
        last = L.csa2_last_error().decode()
        raise Csa2Error(f"{name} failed ({rc}): {msg}" + (f" [{last}]" if last else ""))


def _need(t, dtype, ndim, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")


def csa2_version() -> int:
    return int(lib().csa2_version())


def csa2_init():
    _check(lib().csa2_init(), "csa2_init")


def csa2_device_status(clear: bool = False) -> int:
    """The device status word (0, or a CSA2_STATUS_* code a kernel stored); clear resets it."""
    return int(lib().csa2_device_status(int(clear)))


def csa2_debug_set_wait_limit(polls: int) -> int:
    """Testing aid: the attention kernel's partner-wait bound (negative restores the default)."""
    return int(lib().csa2_debug_set_wait_limit(int(polls)))


def _workspace(need: int, workspace, device, bind: bool, name: str):
    """The caller's workspace, or (eager calls only) a temporary one of `need` bytes.  A
    bound call keeps raw pointers, so a temporary would be freed while the callable still
    writes into it: binding requires the caller's own workspace."""
    if workspace is None and need:
        if bind:
            raise ValueError(f"{name}: a bound call needs a caller-owned workspace of {need} bytes")
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, (0 if workspace is None else workspace.numel())


def _rows2(t, name):
    """A [rows, row_bytes] uint8 device view whose rows may be strided (stride(1) == 1):
    (pointer, row stride in bytes)."""
    if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_cuda or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D uint8 device tensor with unit inner stride")
    return _p(t), t.stride(0)


def _quant_args(src, fmt: int, codes, scales, dst_row, bind: bool):
    """Checks one quantise job and returns its C arguments (src .. scales_stride).  codes and
    scales may be strided row views (e.g. the two parts of an interleaved cache record)."""
    if src.dtype not in (torch.float32, torch.bfloat16) or src.dim() != 2 or not src.is_cuda:
        raise TypeError("src must be a 2-D f32/bf16 device tensor")
    if not src.is_contiguous():
        if bind:
            raise ValueError("src must be contiguous when binding a call")
        src = src.contiguous()
    rows, dim = src.shape
    cp, cst = _rows2(codes, "codes")
    per = dim if fmt == FMT_FP8 else dim // 2
    if codes.shape[1] != per:
        raise ValueError("codes row size does not match dim")
    sp, sst = None, 0
    if fmt != FMT_FP8:
        sp, sst = _rows2(scales, "scales")
        g = 16 if fmt == FMT_NVFP4 else 32
        if tuple(scales.shape) != (codes.shape[0], dim // g):
            raise ValueError("scales shape does not match codes / dim")
    if dst_row is not None:
        _need(dst_row, torch.int64, 1, "dst_row")
        if dst_row.shape[0] != rows:
            raise ValueError("dst_row length != rows")
    dt = DT_F32 if src.dtype == torch.float32 else DT_BF16
    return (_p(src), dt, rows, dim, fmt, _p(dst_row), codes.shape[0], cp, cst, sp, sst)


def csa2_quantize_kv(src, fmt: int, codes, scales=None, dst_row=None, _bind: bool = False):
    """src [rows, dim] f32/bf16; codes [dst_rows, dim/2] (FP4) or [dst_rows, dim] (FP8) u8;
    scales [dst_rows, dim/16 | dim/32] u8 (row views, possibly strided); dst_row [rows] int64
    or None."""
    return _run("csa2_quantize_kv", _quant_args(src, fmt, codes, scales, dst_row, _bind) + (_stream(),), _bind)


class QuantJob(ctypes.Structure):
    """csa2_quant_job of include/csa2.h."""
    _fields_ = [("src", ctypes.c_void_p), ("src_dtype", ctypes.c_int), ("rows", ctypes.c_int64),
                ("dim", ctypes.c_int), ("fmt", ctypes.c_int), ("dst_row", ctypes.c_void_p),
                ("dst_rows", ctypes.c_int64), ("codes", ctypes.c_void_p), ("codes_stride", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("scales_stride", ctypes.c_int64)]


def csa2_quantize_kv_multi(jobs, _bind: bool = False):
    """Several csa2_quantize_kv jobs in one launch; jobs = [(src, fmt, codes, scales, dst_row), ...]."""
    if len(jobs) > 8:
        raise ValueError("at most 8 jobs per launch")
    arr = (QuantJob * max(len(jobs), 1))()
    for i, (src, fmt, codes, scales, dst_row) in enumerate(jobs):
        arr[i] = QuantJob(*_quant_args(src, fmt, codes, scales, dst_row, _bind))
    return _run("csa2_quantize_kv_multi", (ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream()), _bind)


def _cache3(t, name):
    """A [n_seq, seq_cap, row_bytes] uint8 device view of a cache whose entries and sequences
    may be strided (stride(2) == 1; e.g. the two parts of an interleaved record):
    (pointer, entry stride, sequence stride) in bytes."""
    if t.dtype != torch.uint8 or t.dim() != 3 or not t.is_cuda or t.stride(2) != 1:
        raise ValueError(f"{name}: expected a 3-D uint8 device tensor with unit inner stride")
    return _p(t), t.stride(1), t.stride(0)


def _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, cand_blocks, n_cand_blocks, block,
                fmt: int = FMT_MXFP4, q_lat_ok: bool = True):
    """Checks the indexer operands shared by the scoring calls and returns the C arguments
    from q_codes to max_cand_blocks, and n_slots.  fmt: the indexer format (MXFP4: one scale
    byte per 32 channels; NVFP4: one per 16).  q_scales None (MXFP4 only, calls with
    q_lat_ok): q_codes is the unquantised indexer Q, [n_q, H_I, 128] f32 or bf16, which the
    call quantises itself (fmt FMT_MXFP4_Q_F32 / _BF16 at the C boundary)."""
    if fmt not in (FMT_MXFP4, FMT_NVFP4):
        raise ValueError("indexer format must be FMT_MXFP4 or FMT_NVFP4")
    scale_group = 32 if fmt == FMT_MXFP4 else 16
    q_lat = q_scales is None
    if q_lat:
        if fmt != FMT_MXFP4 or not q_lat_ok:
            raise ValueError("an unquantised indexer Q is taken by the MXFP4 scoring calls only")
        if q_codes.dtype not in (torch.float32, torch.bfloat16) or q_codes.dim() != 3 or not q_codes.is_cuda or \
                not q_codes.is_contiguous():
            raise ValueError("unquantised indexer Q: a contiguous CUDA [n_q, H_I, 128] f32/bf16 tensor")
        fmt = FMT_MXFP4_Q_F32 if q_codes.dtype == torch.float32 else FMT_MXFP4_Q_BF16
        n_q, h, d = q_codes.shape
        half = d // 2
    else:
        _need(q_codes, torch.uint8, 3, "q_codes")
        _need(q_scales, torch.uint8, 3, "q_scales")
        n_q, h, half = q_codes.shape
    _need(w, torch.float32, 2, "w")
    kc, kce, kcs = _cache3(k_codes, "k_codes")
    ks, kse, kss = _cache3(k_scales, "k_scales")
    _need(q_seq, torch.int32, 1, "q_seq")
    _need(n_vis, torch.int64, 1, "n_vis")
    n_seq, seq_cap, kh = k_codes.shape
    n_sc = 2 * half // scale_group
    if (not q_lat and q_scales.shape != (n_q, h, n_sc)) or w.shape != (n_q, h) or kh != half or \
            tuple(k_scales.shape) != (n_seq, seq_cap, n_sc) or q_seq.shape[0] != n_q or n_vis.shape[0] != n_q:
        raise ValueError("index: inconsistent shapes")
    max_blocks = 0
    if cand_blocks is not None:
        _need(cand_blocks, torch.int32, 2, "cand_blocks")
        _need(n_cand_blocks, torch.int32, 1, "n_cand_blocks")
        max_blocks = cand_blocks.shape[1]
        if cand_blocks.shape[0] != n_q or n_cand_blocks.shape[0] != n_q:
            raise ValueError("index: inconsistent pool shapes")
    n_slots = max_blocks * block if cand_blocks is not None else seq_cap
    return (_p(q_codes), _p(q_scales), _p(w), n_q, h, 2 * half, fmt, kc, kce, kcs, ks, kse, kss, seq_cap, n_seq,
            _p(q_seq), _p(n_vis), _p(cand_blocks), _p(n_cand_blocks), block, max_blocks), n_slots


class Append(ctypes.Structure):
    """csa2_append: the new main-KV / indexer-K rows that a fused scoring call writes itself
    before it scores (each query's new entry of its own sequence)."""
    _fields_ = [("row", ctypes.c_void_p), ("main", ctypes.c_void_p), ("index", ctypes.c_void_p),
                ("dtype", ctypes.c_int), ("kv_codes", ctypes.c_void_p), ("kv_codes_stride", ctypes.c_int64),
                ("kv_codes_seq_stride", ctypes.c_int64), ("kv_scales", ctypes.c_void_p),
                ("kv_scales_stride", ctypes.c_int64), ("kv_scales_seq_stride", ctypes.c_int64)]


def _check_append_sequences(row, q_seq, seq_cap: int) -> None:
    """Raises ValueError when a query of the call shares its sequence with a query that
    appends (row in [0, seq_cap)): that query's row is written while the call runs."""
    seqs = q_seq[(row >= 0) & (row < seq_cap)]
    if seqs.numel():
        vals, counts = torch.unique(q_seq, return_counts=True)
        if bool((counts[torch.searchsorted(vals, seqs)] != 1).any()):
            raise ValueError("append: another query of the call reads the sequence of an appending query")


def _append_arg(append, n_q: int, seq_cap: int, q_seq):
    """append: None, or a dict with row ([n_q] int64: the new entry's row in the query's
    sequence, negative for none), main ([n_q, 512] latents or None) with kv_codes / kv_scales
    (the main-KV cache views, as for csa2_sparse_attn), and index ([n_q, 128] latents or
    None; written into the call's indexer-K cache).  Latents f32 or bf16 (both the same),
    contiguous.  No other query of the call may read the sequence of a query that appends
    (row in [0, seq_cap)); that is checked once per call or per bound callable, with one
    read of row and q_seq (not while the stream is being captured into a graph: calls
    recorded there are bound and checked before the capture).  Returns the C argument (a
    pointer to a csa2_append, or None)."""
    if append is None:
        return None
    row, main, index = append["row"], append.get("main"), append.get("index")
    _need(row, torch.int64, 1, "append row")
    if row.shape[0] != n_q:
        raise ValueError("append: row must have n_q entries")
    if n_q > 1 and not torch.cuda.is_current_stream_capturing():
        _check_append_sequences(row, q_seq, seq_cap)
    dts = {t.dtype for t in (main, index) if t is not None}
    if len(dts) != 1 or not dts <= {torch.float32, torch.bfloat16}:
        raise ValueError("append: main / index latents f32 or bf16, the same for both, at least one")
    a = Append(row=row.data_ptr(), dtype=DT_F32 if dts == {torch.float32} else DT_BF16)
    for t, name, d in ((main, "main", 512), (index, "index", 128)):
        if t is None:
            continue
        if t.dim() != 2 or tuple(t.shape) != (n_q, d) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"append: {name} must be a contiguous CUDA [n_q, {d}] tensor")
        setattr(a, name, t.data_ptr())
    if main is not None:
        kc, kce, kcs = _cache3(append["kv_codes"], "append kv_codes")
        ks, kse, kss = _cache3(append["kv_scales"], "append kv_scales")
        if append["kv_codes"].shape[1] < seq_cap or append["kv_scales"].shape[1] < seq_cap:
            raise ValueError("append: the main-KV cache holds fewer rows than the indexer cache")
        a.kv_codes, a.kv_codes_stride, a.kv_codes_seq_stride = kc.value, kce, kcs
        a.kv_scales, a.kv_scales_stride, a.kv_scales_seq_stride = ks.value, kse, kss
    return ctypes.byref(a)


def csa2_index_score(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, scores,
                     cand_blocks=None, n_cand_blocks=None, block: int = 8, fmt: int = FMT_MXFP4, _bind: bool = False):
    """q_codes [n_q, H_I, 64], q_scales [n_q, H_I, 4 (MXFP4) | 8 (NVFP4)], w [n_q, H_I] f32;
    k_codes [n_seq, seq_cap, 64], k_scales [n_seq, seq_cap, 4 | 8] (views, entries and
    sequences possibly strided); q_seq [n_q] int32, n_vis [n_q] int64; scores [n_q, stride]
    f32; cand_blocks [n_q, max_blocks] int32; fmt FMT_MXFP4 or FMT_NVFP4.  With MXFP4,
    q_scales None and q_codes the unquantised [n_q, H_I, 128] f32/bf16 indexer Q, the call
    quantises Q itself (the same for csa2_index_topk, _segments and _topk_pool)."""
    args, _ = _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, cand_blocks, n_cand_blocks, block,
                          fmt)
    _need(scores, torch.float32, 2, "scores")
    if scores.shape[0] != q_codes.shape[0]:
        raise ValueError("index_score: scores rows != n_q")
    return _run("csa2_index_score", args + (_p(scores), scores.stride(0), _stream()), _bind)


def csa2_index_score_q(q, w, k_codes, k_scales, q_seq, n_vis, scores, cand_blocks=None, n_cand_blocks=None,
                       block: int = 8, _bind: bool = False):
    """csa2_index_score with the indexer Q unquantised: q [n_q, H_I, 128] f32 or bf16, quantised
    to MXFP4 inside the scoring kernel; the other operands as csa2_index_score (MXFP4)."""
    if q.dtype not in (torch.float32, torch.bfloat16) or q.dim() != 3 or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous CUDA [n_q, H_I, 128] f32/bf16 tensor")
    n_q, h, d = q.shape
    _need(w, torch.float32, 2, "w")
    kc, kce, kcs = _cache3(k_codes, "k_codes")
    ks, kse, kss = _cache3(k_scales, "k_scales")
    _need(q_seq, torch.int32, 1, "q_seq")
    _need(n_vis, torch.int64, 1, "n_vis")
    n_seq, seq_cap, kh = k_codes.shape
    if w.shape != (n_q, h) or kh != d // 2 or tuple(k_scales.shape) != (n_seq, seq_cap, d // 32) or \
            q_seq.shape[0] != n_q or n_vis.shape[0] != n_q:
        raise ValueError("index_score_q: inconsistent shapes")
    max_blocks = 0
    if cand_blocks is not None:
        _need(cand_blocks, torch.int32, 2, "cand_blocks")
        _need(n_cand_blocks, torch.int32, 1, "n_cand_blocks")
        max_blocks = cand_blocks.shape[1]
        if cand_blocks.shape[0] != n_q or n_cand_blocks.shape[0] != n_q:
            raise ValueError("index_score_q: inconsistent pool shapes")
    _need(scores, torch.float32, 2, "scores")
    if scores.shape[0] != n_q:
        raise ValueError("index_score_q: scores rows != n_q")
    qdt = DT_F32 if q.dtype == torch.float32 else DT_BF16
    return _run("csa2_index_score_q", (_p(q), qdt, _p(w), n_q, h, d, FMT_MXFP4, kc, kce, kcs, ks, kse, kss, seq_cap,
                                       n_seq, _p(q_seq), _p(n_vis), _p(cand_blocks), _p(n_cand_blocks), block,
                                       max_blocks, _p(scores), scores.stride(0), _stream()), _bind)


def csa2_index_score_grouped(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, group: int, scores,
                             _bind: bool = False):
    """csa2_index_score without a pool for rows in groups of `group` consecutive rows that
    share a sequence (each group's indexer K is read once); operands as csa2_index_score (MXFP4)."""
    args, _ = _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, None, None, 8, q_lat_ok=False)
    _need(scores, torch.float32, 2, "scores")
    if scores.shape[0] != q_codes.shape[0]:
        raise ValueError("index_score_grouped: scores rows != n_q")
    return _run("csa2_index_score_grouped", args[:17] + (int(group), _p(scores), scores.stride(0), _stream()), _bind)


def csa2_index_topk_grouped_workspace_bytes(n_q: int, seq_cap: int, k: int, group: int) -> int:
    return int(lib().csa2_index_topk_grouped_workspace_bytes(n_q, seq_cap, k, group))


def csa2_index_topk_grouped(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, group: int, k: int, idx_out,
                            count_out, workspace=None, _bind: bool = False):
    """Grouped rows scored and selected without a score array: the operands of
    csa2_index_score_grouped -> idx_out [n_q, k] int32, count_out [n_q] int32, as
    csa2_index_score_grouped followed by csa2_topk returns them."""
    args, _ = _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, None, None, 8, q_lat_ok=False)
    _need(idx_out, torch.int32, 2, "idx_out")
    _need(count_out, torch.int32, 1, "count_out")
    n_q = q_codes.shape[0]
    if idx_out.shape != (n_q, k) or count_out.shape[0] != n_q:
        raise ValueError("index_topk_grouped: inconsistent output shapes")
    need = csa2_index_topk_grouped_workspace_bytes(n_q, k_codes.shape[1], k, int(group))
    workspace, ws_bytes = _workspace(need, workspace, q_codes.device, _bind, "index_topk_grouped")
    return _run("csa2_index_topk_grouped", args[:17] + (int(group), k, _p(idx_out), _p(count_out), _p(workspace),
                                                        ws_bytes, _stream()), _bind)


def csa2_index_topk_workspace_bytes(n_q: int, n_slots: int, k: int, in_pool: bool = False) -> int:
    return int(lib().csa2_index_topk_workspace_bytes(n_q, n_slots, k, int(in_pool)))


def csa2_index_topk(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, k: int, idx_out, count_out,
                    workspace=None, cand_blocks=None, n_cand_blocks=None, block: int = 8, fmt: int = FMT_MXFP4,
                    append=None, _bind: bool = False):
    """Scores and Top-K in one pass: the operands of csa2_index_score (without scores) ->
    idx_out [n_q, k] int32, count_out [n_q] int32, as csa2_topk returns them.  append: the
    new entries the call writes first (see _append_arg; not inside a pool)."""
    args, n_slots = _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, cand_blocks, n_cand_blocks,
                                block, fmt)
    _need(idx_out, torch.int32, 2, "idx_out")
    _need(count_out, torch.int32, 1, "count_out")
    n_q = q_codes.shape[0]
    if idx_out.shape != (n_q, k) or count_out.shape[0] != n_q:
        raise ValueError("index_topk: inconsistent output shapes")
    need = csa2_index_topk_workspace_bytes(n_q, max(n_slots, 1), k, cand_blocks is not None)
    workspace, ws_bytes = _workspace(need, workspace, q_codes.device, _bind, "index_topk")
    app = _append_arg(append, n_q, k_codes.shape[1], q_seq)
    return _run("csa2_index_topk", args + (k, _p(idx_out), _p(count_out), _p(workspace), ws_bytes, app, _stream()),
                _bind)


def csa2_segment_keys(n_slots: int, k: int) -> int:
    return int(lib().csa2_segment_keys(n_slots, k))


def csa2_index_segments(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, k: int, cand_keys,
                        fmt: int = FMT_MXFP4, append=None, _bind: bool = False):
    """The fused first Top-K level alone: the operands of csa2_index_score (no pool) ->
    cand_keys [n_q, csa2_segment_keys(seq_cap, k)] (opaque 64-bit keys, held in an int64
    tensor) for csa2_sparse_attn_topk.  append: the new entries the call writes first."""
    args, n_slots = _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, None, None, 8, fmt)
    _need(cand_keys, torch.int64, 2, "cand_keys")
    n_q = q_codes.shape[0]
    if tuple(cand_keys.shape) != (n_q, csa2_segment_keys(n_slots, k)):
        raise ValueError("index_segments: cand_keys must be [n_q, csa2_segment_keys(seq_cap, k)]")
    app = _append_arg(append, n_q, k_codes.shape[1], q_seq)
    return _run("csa2_index_segments", args[:17] + (k, _p(cand_keys), app, _stream()), _bind)


def csa2_index_topk_pool_workspace_bytes(n_q: int, n_slots: int, k: int, block: int, max_blocks: int) -> int:
    return int(lib().csa2_index_topk_pool_workspace_bytes(n_q, n_slots, k, block, max_blocks))


def csa2_index_topk_pool(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, k: int, idx_out, count_out,
                         blocks_out, blocks_count, block: int = 8, workspace=None, append=None, _bind: bool = False):
    """Top-K and candidate pool in one scoring pass: the operands of csa2_index_score (no
    pool, MXFP4) -> idx_out [n_q, k], count_out [n_q] (as csa2_topk) and blocks_out
    [n_q, max_blocks], blocks_count [n_q] (as csa2_build_pool).  append: the new entries the
    call writes first."""
    args, n_slots = _index_args(q_codes, q_scales, w, k_codes, k_scales, q_seq, n_vis, None, None, block)
    for t, name in ((idx_out, "idx_out"), (blocks_out, "blocks_out")):
        _need(t, torch.int32, 2, name)
    _need(count_out, torch.int32, 1, "count_out")
    _need(blocks_count, torch.int32, 1, "blocks_count")
    n_q = q_codes.shape[0]
    max_blocks = blocks_out.shape[1]
    if idx_out.shape != (n_q, k) or count_out.shape[0] != n_q or blocks_out.shape[0] != n_q or \
            blocks_count.shape[0] != n_q:
        raise ValueError("index_topk_pool: inconsistent output shapes")
    need = csa2_index_topk_pool_workspace_bytes(n_q, max(n_slots, 1), k, block, max_blocks)
    workspace, ws_bytes = _workspace(max(need, 1), workspace, q_codes.device, _bind, "index_topk_pool")
    app = _append_arg(append, n_q, k_codes.shape[1], q_seq)
    return _run("csa2_index_topk_pool", args[:17] + (k, _p(idx_out), _p(count_out), block, max_blocks, _p(blocks_out),
                                                     _p(blocks_count), _p(workspace), ws_bytes, app, _stream()),
                _bind)


def csa2_topk_workspace_bytes(n_q: int, n_slots: int, k: int) -> int:
    return int(lib().csa2_topk_workspace_bytes(n_q, n_slots, k))


def csa2_topk(scores, n_vis, max_vis: int, k: int, idx_out, count_out, workspace=None,
              cand_blocks=None, n_cand_blocks=None, block: int = 8, _bind: bool = False):
    """scores [n_q, stride] f32 -> idx_out [n_q, k] int32 ascending, -1 padded; count_out [n_q] int32."""
    _need(scores, torch.float32, 2, "scores")
    _need(n_vis, torch.int64, 1, "n_vis")
    _need(idx_out, torch.int32, 2, "idx_out")
    _need(count_out, torch.int32, 1, "count_out")
    n_q = scores.shape[0]
    if idx_out.shape != (n_q, k) or count_out.shape[0] != n_q or n_vis.shape[0] != n_q:
        raise ValueError("topk: inconsistent shapes")
    max_blocks = 0
    if cand_blocks is not None:
        _need(cand_blocks, torch.int32, 2, "cand_blocks")
        _need(n_cand_blocks, torch.int32, 1, "n_cand_blocks")
        max_blocks = cand_blocks.shape[1]
    n_slots = max_blocks * block if cand_blocks is not None else max_vis
    need = csa2_topk_workspace_bytes(n_q, max(n_slots, 1), k)
    workspace, ws_bytes = _workspace(need, workspace, scores.device, _bind, "workspace")
    return _run("csa2_topk", (_p(scores), scores.stride(0), n_q, _p(n_vis), max_vis, _p(cand_blocks),
                              _p(n_cand_blocks), block, max_blocks, k, _p(idx_out), _p(count_out), _p(workspace),
                              ws_bytes, _stream()), _bind)


def csa2_pool_workspace_bytes(n_q: int, max_vis: int, block: int, max_blocks: int) -> int:
    return int(lib().csa2_pool_workspace_bytes(n_q, max_vis, block, max_blocks))


def csa2_build_pool(scores, n_vis, max_vis: int, blocks_out, count_out, block: int = 8, workspace=None,
                    _bind: bool = False):
    """scores [n_q, stride] f32 -> blocks_out [n_q, max_blocks] int32 ascending, -1 padded."""
    _need(scores, torch.float32, 2, "scores")
    _need(n_vis, torch.int64, 1, "n_vis")
    _need(blocks_out, torch.int32, 2, "blocks_out")
    _need(count_out, torch.int32, 1, "count_out")
    n_q, max_blocks = blocks_out.shape
    need = csa2_pool_workspace_bytes(n_q, max(max_vis, 1), block, max_blocks)
    workspace, ws_bytes = _workspace(need, workspace, scores.device, _bind, "workspace")
    return _run("csa2_build_pool", (_p(scores), scores.stride(0), n_q, _p(n_vis), max_vis, block, max_blocks,
                                    _p(blocks_out), _p(count_out), _p(workspace), ws_bytes, _stream()), _bind)


def csa2_attn_workspace_bytes(n_q: int, n_heads: int, dim: int, k: int, window: int) -> int:
    return int(lib().csa2_attn_workspace_bytes(n_q, n_heads, dim, k, window))


def _attn_args(q, kv_codes, kv_scales, q_seq, swa, swa_base, q_pos, replay_start, out, lse, n_q_rows):
    """Checks the operands every attention call shares; returns the C arguments of the
    main-KV cache (codes, their strides, scales, their strides, seq_cap, n_seq) and of the
    window ring (pointer, row stride, sequence stride, swa_cap).  The caches may be strided
    views (e.g. the two parts of an interleaved 288-byte main-KV record)."""
    _need(q, torch.bfloat16, 3, "q")
    kc, kce, kcs = _cache3(kv_codes, "kv_codes")
    ks, kse, kss = _cache3(kv_scales, "kv_scales")
    sw, swr, sws = _cache3(swa, "swa")
    _need(q_seq, torch.int32, 1, "q_seq")
    _need(swa_base, torch.int64, 1, "swa_base")
    _need(q_pos, torch.int64, 1, "q_pos")
    _need(replay_start, torch.int64, 1, "replay_start")
    n_q, H, D = q.shape
    n_seq, seq_cap, _ = kv_codes.shape
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (n_q, H, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [n_q, H, D] f32/bf16 tensor")
    if kv_codes.shape[2] != D // 2 or tuple(kv_scales.shape) != (n_seq, seq_cap, D // 16) or swa.shape[0] != n_seq or \
            swa.shape[2] != D or swa_base.shape[0] != n_seq or n_q_rows != n_q:
        raise ValueError("sparse_attn: inconsistent shapes")
    if lse is not None:
        _need(lse, torch.float32, 2, "lse")
        if tuple(lse.shape) != (n_q, H):
            raise ValueError("lse shape")
    return (kc, kce, kcs, ks, kse, kss, seq_cap, n_seq), (sw, swr, sws, swa.shape[1])


def _new_win(new_win, n_q, D, q_seq=None):
    """(pointer, dtype) of the optional window append: [n_q, D] f32 / bf16 latents.  The
    append needs every row of the call in a sequence of its own (otherwise one row's
    workgroups would write a ring row that another row's workgroups read): checked here,
    once per call or per bound callable, with one read of q_seq -- except while the stream
    is being captured into a graph, where no such read may run (calls recorded there are
    bound and checked before the capture, as the layer driver and the benchmark do)."""
    if new_win is None:
        return None, DT_F32
    if new_win.dtype not in (torch.float32, torch.bfloat16) or tuple(new_win.shape) != (n_q, D) or \
            not new_win.is_contiguous() or not new_win.is_cuda:
        raise ValueError("new_win must be a contiguous [n_q, D] f32/bf16 device tensor")
    if q_seq is not None and n_q > 1 and not torch.cuda.is_current_stream_capturing() and \
            torch.unique(q_seq).numel() != n_q:
        raise ValueError("new_win: two rows of the call share a sequence (the append needs distinct sequences)")
    return _p(new_win), DT_F32 if new_win.dtype == torch.float32 else DT_BF16


def _attn_tail(q, k, window, sm_scale, out, lse, workspace, new_win, q_seq, bind, name, with_workspace=True):
    """The arguments every attention call ends with: window append .. stream."""
    n_q, H, D = q.shape
    odt = DT_F32 if out.dtype == torch.float32 else DT_BF16
    nw, nwt = _new_win(new_win, n_q, D, q_seq)
    if not with_workspace:
        return (nw, nwt, window, ctypes.c_float(sm_scale), _p(out), odt, _p(lse), _stream())
    need = csa2_attn_workspace_bytes(n_q, H, D, k, window)
    workspace, ws_bytes = _workspace(need, workspace, q.device, bind, name)
    return (nw, nwt, window, ctypes.c_float(sm_scale), _p(out), odt, _p(lse), _p(workspace), ws_bytes, _stream())


def csa2_sparse_attn_topk(q, kv_codes, kv_scales, q_seq, cand_keys, k: int, idx_out, count_out, swa, swa_base, q_pos,
                          replay_start, window: int, sm_scale: float, out, lse=None, workspace=None, new_win=None,
                          _bind: bool = False):
    """csa2_sparse_attn with the index set selected in the call from csa2_index_segments'
    cand_keys [n_q, n_cand]; writes it to idx_out [n_q, k] int32 and count_out [n_q] int32."""
    _need(cand_keys, torch.int64, 2, "cand_keys")
    _need(idx_out, torch.int32, 2, "idx_out")
    _need(count_out, torch.int32, 1, "count_out")
    kv, sw = _attn_args(q, kv_codes, kv_scales, q_seq, swa, swa_base, q_pos, replay_start, out, lse, cand_keys.shape[0])
    n_q, H, D = q.shape
    if tuple(idx_out.shape) != (n_q, k) or count_out.shape[0] != n_q:
        raise ValueError("sparse_attn_topk: inconsistent index output shapes")
    tail = _attn_tail(q, k, window, sm_scale, out, lse, workspace, new_win, q_seq, _bind, "sparse_attn_topk")
    return _run("csa2_sparse_attn_topk", (_p(q), n_q, H, D) + kv + (_p(q_seq), _p(cand_keys), cand_keys.shape[1], k,
                                                                   _p(idx_out), _p(count_out)) + sw +
                (_p(swa_base), _p(q_pos), _p(replay_start)) + tail, _bind)


def csa2_sparse_attn_pool_topk(q, kv_codes, kv_scales, q_seq, scores, n_vis, cand_blocks, n_cand_blocks, block: int,
                               k: int, idx_out, count_out, swa, swa_base, q_pos, replay_start, window: int,
                               sm_scale: float, out, lse=None, workspace=None, new_win=None, _bind: bool = False):
    """csa2_sparse_attn inside a pool, with the Top-k selected in the call from the pool's
    slot scores (scores [n_q, stride] f32 as csa2_index_score writes them with cand_blocks
    [n_q, max_blocks] / n_cand_blocks [n_q]); writes idx_out [n_q, k] and count_out [n_q]."""
    _need(scores, torch.float32, 2, "scores")
    _need(n_vis, torch.int64, 1, "n_vis")
    _need(cand_blocks, torch.int32, 2, "cand_blocks")
    _need(n_cand_blocks, torch.int32, 1, "n_cand_blocks")
    _need(idx_out, torch.int32, 2, "idx_out")
    _need(count_out, torch.int32, 1, "count_out")
    kv, sw = _attn_args(q, kv_codes, kv_scales, q_seq, swa, swa_base, q_pos, replay_start, out, lse, scores.shape[0])
    n_q, H, D = q.shape
    if tuple(idx_out.shape) != (n_q, k) or count_out.shape[0] != n_q or cand_blocks.shape[0] != n_q or \
            n_cand_blocks.shape[0] != n_q or n_vis.shape[0] != n_q:
        raise ValueError("sparse_attn_pool_topk: inconsistent shapes")
    tail = _attn_tail(q, k, window, sm_scale, out, lse, workspace, new_win, q_seq, _bind, "sparse_attn_pool_topk")
    return _run("csa2_sparse_attn_pool_topk",
                (_p(q), n_q, H, D) + kv + (_p(q_seq), _p(scores), scores.shape[1], _p(n_vis), _p(cand_blocks),
                                           _p(n_cand_blocks), block, cand_blocks.shape[1], k, _p(idx_out),
                                           _p(count_out)) + sw + (_p(swa_base), _p(q_pos), _p(replay_start)) + tail,
                _bind)


def csa2_sparse_attn(q, kv_codes, kv_scales, q_seq, idx, swa, swa_base, q_pos, replay_start, window: int,
                     sm_scale: float, out, lse=None, workspace=None, new_win=None, _bind: bool = False):
    """q [n_q, H, 512] bf16; kv_codes [n_seq, seq_cap, 256], kv_scales [n_seq, seq_cap, 32]
    (views, possibly strided: e.g. rec[..., :256] and rec[..., 256:] of one interleaved
    [n_seq, seq_cap, 288] record); idx [n_q, k] int32; swa [n_seq, swa_cap, 512] u8 (view);
    swa_base [n_seq] int64; q_pos, replay_start [n_q] int64; out [n_q, H, 512] f32/bf16; lse
    [n_q, H] f32."""
    _need(idx, torch.int32, 2, "idx")
    kv, sw = _attn_args(q, kv_codes, kv_scales, q_seq, swa, swa_base, q_pos, replay_start, out, lse, idx.shape[0])
    n_q, H, D = q.shape
    k = idx.shape[1]
    tail = _attn_tail(q, k, window, sm_scale, out, lse, workspace, new_win, q_seq, _bind, "sparse_attn")
    return _run("csa2_sparse_attn", (_p(q), n_q, H, D) + kv + (_p(q_seq), _p(idx), k) + sw +
                (_p(swa_base), _p(q_pos), _p(replay_start)) + tail, _bind)


def csa2_sparse_attn_noalloc_max_bytes() -> int:
    return int(lib().csa2_sparse_attn_noalloc_max_bytes())


def csa2_sparse_attn_noalloc(q, kv_codes, kv_scales, q_seq, idx, swa, swa_base, q_pos, replay_start, window: int,
                             sm_scale: float, out, lse=None, new_win=None, _bind: bool = False):
    """csa2_sparse_attn without a workspace: a split key list's partials go to the library's
    static per-GPU scratch (calls that overlap on one GPU race).  Arguments as csa2_sparse_attn."""
    _need(idx, torch.int32, 2, "idx")
    kv, sw = _attn_args(q, kv_codes, kv_scales, q_seq, swa, swa_base, q_pos, replay_start, out, lse, idx.shape[0])
    n_q, H, D = q.shape
    tail = _attn_tail(q, idx.shape[1], window, sm_scale, out, lse, None, new_win, q_seq, _bind,
                      "sparse_attn_noalloc", with_workspace=False)
    return _run("csa2_sparse_attn_noalloc", (_p(q), n_q, H, D) + kv + (_p(q_seq), _p(idx), idx.shape[1]) + sw +
                (_p(swa_base), _p(q_pos), _p(replay_start)) + tail, _bind)

"""The C-ABI library loads and exports every symbol include/csa2.h declares, the binding's
argument table matches every declaration, and argument validation rejects bad calls on the
host, before anything reaches the GPU (no GPU needed).  Calls below name their arguments
after the header's parameter names."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _header_src():
    return re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)


def _declared():
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", _header_src())))


def _params(name):
    """Parameter names of a declared function, in order."""
    m = re.search(r"\b%s\s*\(([^)]*)\)\s*;" % name, _header_src())
    assert m, name
    body = m.group(1).strip()
    if body in ("", "void"):
        return []
    return [re.findall(r"[A-Za-z_][A-Za-z0-9_]*", p)[-1] for p in body.split(",")]


@pytest.fixture(scope="module")
def L():
    from fp4_kv_cache_layer_amd import csa2
    from fp4_kv_cache_layer_amd.build import LIB_PATH
    if not os.path.exists(LIB_PATH):
        pytest.fail("libcsa2.so is not built; run __graft_entry__.build()")
    return csa2.lib()   # argument types set from the binding's table


def _call(L, name, **kw):
    names = _params(name)
    missing = [n for n in names if n not in kw]
    assert not missing and len(kw) == len(names), (name, missing, sorted(set(kw) - set(names)))
    return getattr(L, name)(*[kw[n] for n in names])


def test_header_declares_the_calls():
    names = _declared()
    for n in ("csa2_quantize_kv", "csa2_index_score", "csa2_index_topk", "csa2_topk", "csa2_build_pool",
              "csa2_sparse_attn"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_binding_table_matches_the_header(L):
    """Every declared function has argument types in the binding, one per parameter."""
    for name in _declared():
        fn = getattr(L, name)
        assert fn.argtypes is not None, name
        assert len(fn.argtypes) == len(_params(name)), (name, len(fn.argtypes), len(_params(name)))


def test_status_strings_and_version(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.csa2_status_string(code) != b"unknown status"
    assert L.csa2_status_string(-99) == b"unknown status"
    assert L.csa2_version() >= 100
    assert L.csa2_device_status(0) == 0          # no status word before csa2_init: nothing to report


def _quant(**over):
    kw = dict(src=FAKE, src_dtype=0, rows=4, dim=512, fmt=0, dst_row=None, dst_rows=4, codes=FAKE, codes_stride=0,
              scales=FAKE, scales_stride=0, stream=None)
    kw.update(over)
    return kw


def test_quantize_validation(L):
    assert _call(L, "csa2_quantize_kv", **_quant(src=None)) == -1
    assert _call(L, "csa2_quantize_kv", **_quant(dim=500)) == -2                    # dim % 16
    assert _call(L, "csa2_quantize_kv", **_quant(fmt=9)) == -3                      # fmt
    assert _call(L, "csa2_quantize_kv", **_quant(codes=ctypes.c_void_p(0x1001))) == -2   # misaligned
    assert _call(L, "csa2_quantize_kv", **_quant(codes_stride=200)) == -2           # below the 256-byte row
    assert _call(L, "csa2_quantize_kv", **_quant(codes_stride=260)) == -2           # not a multiple of 8
    assert _call(L, "csa2_quantize_kv", **_quant(scales_stride=16)) == -2           # below the 32-byte row
    assert _call(L, "csa2_quantize_kv", **_quant(fmt=1, codes_stride=264)) == -2    # MXFP4: multiple of 16
    assert _call(L, "csa2_quantize_kv", **_quant(rows=0)) == 0                      # empty: no launch
    assert _call(L, "csa2_quantize_kv", **_quant(rows=0, codes_stride=288, scales_stride=288)) == 0


def test_topk_validation(L):
    kw = dict(scores=FAKE, scores_stride=100, n_q=2, n_vis=FAKE, max_vis=100, cand_blocks=None, n_cand_blocks=None,
              block=8, max_cand_blocks=0, k=4096, idx_out=FAKE, count_out=FAKE, workspace=None, workspace_bytes=0,
              stream=None)
    assert _call(L, "csa2_topk", **kw) == -2                                        # k > 2048
    assert _call(L, "csa2_topk", **dict(kw, k=16, scores_stride=10)) == -2          # stride
    assert _call(L, "csa2_topk", **dict(kw, k=512, scores_stride=1 << 20, max_vis=1 << 20)) == -5
    assert L.csa2_topk_workspace_bytes(2, 8192, 512) == 0                           # one segment: no scratch
    assert L.csa2_topk_workspace_bytes(2, 1 << 20, 512) > 0


def _index(**over):
    kw = dict(q_codes=FAKE, q_scales=FAKE, w=FAKE, n_q=4, n_heads=16, dim=128, fmt=1, k_codes=FAKE, k_codes_stride=0,
              k_codes_seq_stride=0, k_scales=FAKE, k_scales_stride=0, k_scales_seq_stride=0, seq_cap=4096, n_seq=1,
              q_seq=FAKE, n_vis=FAKE)
    kw.update(over)
    return kw


def test_index_validation(L):
    seg = dict(k=512, cand_keys=FAKE, append=None, stream=None)
    assert L.csa2_segment_keys(131072, 512) == 8192
    assert L.csa2_segment_keys(131073, 512) == 8704
    assert L.csa2_segment_keys(0, 512) == 512
    assert L.csa2_segment_keys(100, 0) == 0
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, cand_keys=None)) == -1   # no key buffer
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, k=4096)) == -2            # k > 2048
    assert _call(L, "csa2_index_segments", **_index(dim=64), **seg) == -2                   # indexer dim
    assert _call(L, "csa2_index_segments", **_index(fmt=2), **seg) == -3                    # not an indexer format
    assert _call(L, "csa2_index_segments", **_index(k_codes_stride=72), **seg) == -2        # not a multiple of 16
    assert _call(L, "csa2_index_segments", **_index(k_codes_stride=48), **seg) == -2        # below the 64-byte row
    assert _call(L, "csa2_index_segments", **_index(k_scales_stride=2), **seg) == -2        # below the 4-byte row
    assert _call(L, "csa2_index_segments", **_index(fmt=0, k_scales_stride=9), **seg) == -2  # NVFP4: even stride
    assert _call(L, "csa2_index_segments", **_index(fmt=0, k_scales=ctypes.c_void_p(0x1001)), **seg) == -2
    assert _call(L, "csa2_index_segments", **_index(n_q=0), **seg) == 0                    # no rows: no launch
    # unquantised indexer Q (fmt 3 / 4): q_scales unused; 5 is no format
    assert _call(L, "csa2_index_segments", **_index(fmt=3, q_scales=None), **dict(seg, cand_keys=None)) == -1
    assert _call(L, "csa2_index_segments", **_index(fmt=5), **seg) == -3
    assert _call(L, "csa2_index_segments", **_index(fmt=1, q_scales=None), **seg) == -1   # quantised Q needs scales
    # csa2_append
    from fp4_kv_cache_layer_amd.csa2 import Append
    ok = Append(row=0x2000, main=0x3000, index=0x4000, dtype=0, kv_codes=0x5000, kv_scales=0x6000)
    app = lambda **f: ctypes.byref(Append(**{**{k: getattr(ok, k) for k, _ in Append._fields_}, **f}))
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, append=app(row=None))) == -1
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, append=app(kv_codes=None))) == -1
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, append=app(dtype=7))) == -3
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, append=app(main=0x3004))) == -2    # misaligned
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, append=app(index=0x4008))) == -2
    assert _call(L, "csa2_index_segments", **_index(), **dict(seg, append=app(kv_codes_stride=200))) == -2
    assert _call(L, "csa2_index_segments", **_index(fmt=0), **dict(seg, append=app())) == -3   # NVFP4 indexer
    topk = dict(cand_blocks=FAKE, n_cand_blocks=FAKE, block=8, max_cand_blocks=16, k=512, idx_out=FAKE,
                count_out=FAKE, workspace=None, workspace_bytes=0, append=app(), stream=None)
    assert _call(L, "csa2_index_topk", **_index(), **topk) == -3                           # no append inside a pool
    grp = dict(group=8, k=512, idx_out=FAKE, count_out=FAKE, workspace=None, workspace_bytes=0, stream=None)
    assert _call(L, "csa2_index_topk_grouped", **_index(fmt=0), **grp) == -3               # MXFP4 only
    assert _call(L, "csa2_index_topk_grouped", **_index(), **dict(grp, group=9)) == -2
    assert _call(L, "csa2_index_topk_grouped", **_index(), **dict(grp, k=705)) == -2
    assert _call(L, "csa2_index_topk_grouped", **_index(), **grp) == -5                     # workspace
    assert L.csa2_index_topk_grouped_workspace_bytes(4224, 133120, 512, 8) == 4224 * 8 * 512 * 8 + 256


def test_index_score_q_validation(L):
    """csa2_index_score_q (indexer Q unquantised) rejects bad arguments before any launch."""
    base = _index()
    del base["q_codes"], base["q_scales"]
    base.update(q=FAKE, q_dtype=0, cand_blocks=None, n_cand_blocks=None, block=8, max_cand_blocks=0, scores=FAKE,
                scores_stride=4096, stream=None)
    assert _call(L, "csa2_index_score_q", **dict(base, q_dtype=5)) == -3            # Q dtype
    assert _call(L, "csa2_index_score_q", **dict(base, fmt=0)) == -3                # MXFP4 only
    assert _call(L, "csa2_index_score_q", **dict(base, q=None)) == -1               # Q NULL
    assert _call(L, "csa2_index_score_q", **dict(base, q=ctypes.c_void_p(0x1004))) == -2   # Q not 16-byte aligned
    assert _call(L, "csa2_index_score_q", **dict(base, dim=64)) == -2               # indexer dim
    assert _call(L, "csa2_index_score_q", **dict(base, n_heads=17)) == -2           # indexer heads
    assert _call(L, "csa2_index_score_q", **dict(base, scores_stride=100)) == -2    # scores stride below seq_cap
    assert _call(L, "csa2_index_score_q", **dict(base, cand_blocks=FAKE)) == -1     # pool map without its counts
    assert _call(L, "csa2_index_score_q", **dict(base, n_q=0)) == 0                 # no rows: nothing launched


def _attn(**over):
    kw = dict(q=FAKE, n_q=4, n_heads=64, dim=512, kv_codes=FAKE, kv_codes_stride=0, kv_codes_seq_stride=0,
              kv_scales=FAKE, kv_scales_stride=0, kv_scales_seq_stride=0, seq_cap=100, n_seq=1, q_seq=FAKE,
              swa=FAKE, swa_row_stride=0, swa_seq_stride=0, swa_cap=128, swa_base=FAKE, q_pos=FAKE,
              replay_start=FAKE, new_win=None, new_win_dtype=0, window=128, sm_scale=0.05, out=FAKE, out_dtype=0,
              lse=None, stream=None)
    kw.update(over)
    return kw


def test_attention_validation(L):
    base = _attn(idx=FAKE, k=512, workspace=None, workspace_bytes=0)
    assert _call(L, "csa2_sparse_attn", **dict(base, n_heads=40)) == -2             # heads not a multiple of 16
    assert _call(L, "csa2_sparse_attn", **dict(base, window=256)) == -2             # window > swa_cap
    assert _call(L, "csa2_sparse_attn", **dict(base, out_dtype=7)) == -3            # out dtype
    assert _call(L, "csa2_sparse_attn", **dict(base, new_win=FAKE, new_win_dtype=9)) == -3
    assert _call(L, "csa2_sparse_attn", **dict(base, idx=None)) == -1               # idx NULL with k > 0
    assert _call(L, "csa2_sparse_attn", **dict(base, kv_codes_stride=264)) == -2    # code stride not % 16
    assert _call(L, "csa2_sparse_attn", **dict(base, kv_scales_stride=30)) == -2    # scale stride below 32 B
    assert _call(L, "csa2_sparse_attn", **dict(base, kv_scales_stride=34)) == -2    # scale stride not % 4
    assert _call(L, "csa2_sparse_attn", **dict(base, kv_scales=ctypes.c_void_p(0x1002))) == -2
    assert _call(L, "csa2_sparse_attn", **dict(base, swa_row_stride=500)) == -2     # window rows below 512 B
    assert _call(L, "csa2_sparse_attn", **base) == -5                               # the split needs a workspace
    # the interleaved 288-byte record: codes at +0, scales at +256, both strides 288
    rec = dict(base, kv_codes_stride=288, kv_scales=ctypes.c_void_p(0x1100), kv_scales_stride=288)
    assert _call(L, "csa2_sparse_attn", **rec) == -5                                # accepted up to the workspace
    noalloc = _attn(idx=FAKE, k=512)
    assert _call(L, "csa2_sparse_attn_noalloc", **dict(noalloc, n_heads=40)) == -2
    assert L.csa2_sparse_attn_noalloc_max_bytes() == 16 << 20


def test_attention_split_plan(L):
    """The key-list split behind csa2_attn_workspace_bytes: a window of at most 128 keys (the
    full-channel kernel) splits only while fewer than 128 (query, 16-head group) workgroups
    exist, into slices of at least 8 tiles of 16 keys; a wider window (the split-channel
    kernel) while fewer than 256, into slices of at least 4 tiles.  The workspace holds each
    split's fp32 output and (m, l) per (query, head), plus 256 bytes of alignment."""
    def ws(n_q, heads, k, window, nsplit):
        return nsplit * n_q * heads * (512 + 2) * 4 + 256
    assert L.csa2_attn_workspace_bytes(64, 64, 512, 512, 128) == 0          # 256 workgroups
    assert L.csa2_attn_workspace_bytes(32, 64, 512, 512, 128) == 0          # 128: no split
    assert L.csa2_attn_workspace_bytes(24, 64, 512, 512, 128) == ws(24, 64, 512, 128, 2)
    assert L.csa2_attn_workspace_bytes(8, 64, 512, 512, 128) == ws(8, 64, 512, 128, 4)    # 40 tiles, 10 per slice
    assert L.csa2_attn_workspace_bytes(1, 16, 512, 512, 128) == ws(1, 16, 512, 128, 5)    # at most 40 / 8 slices
    assert L.csa2_attn_workspace_bytes(32, 64, 512, 512, 256) == ws(32, 64, 512, 256, 2)  # split-channel: up to 256
    assert L.csa2_attn_workspace_bytes(6, 16, 512, 2048, 256) == ws(6, 16, 2048, 256, 36)  # 144 tiles, 4 per slice
    assert L.csa2_attn_workspace_bytes(64, 64, 512, 512, 256) == 0
    assert L.csa2_attn_workspace_bytes(8, 40, 512, 512, 128) == 0            # heads not a multiple of 16


def test_select_in_attention_validation(L):
    """csa2_sparse_attn_topk and csa2_sparse_attn_pool_topk reject bad calls on the host."""
    att = _attn(cand_keys=FAKE, cand_per_q=8192, k=512, idx_out=FAKE, count_out=FAKE, workspace=None,
                workspace_bytes=0)
    assert _call(L, "csa2_sparse_attn_topk", **dict(att, cand_keys=None)) == -1    # no candidate keys
    assert _call(L, "csa2_sparse_attn_topk", **dict(att, idx_out=None)) == -1      # no index output
    assert _call(L, "csa2_sparse_attn_topk", **dict(att, cand_per_q=8193)) == -2   # more than one selection holds
    assert _call(L, "csa2_sparse_attn_topk", **dict(att, k=0)) == -2
    assert _call(L, "csa2_sparse_attn_topk", **att) == -5                          # split: needs a workspace
    pool = _attn(scores=FAKE, scores_stride=16384, n_vis=FAKE, cand_blocks=FAKE, n_cand_blocks=FAKE, block=8,
                 max_cand_blocks=2048, k=512, idx_out=FAKE, count_out=FAKE, workspace=None, workspace_bytes=0)
    assert _call(L, "csa2_sparse_attn_pool_topk", **dict(pool, scores=None)) == -1
    assert _call(L, "csa2_sparse_attn_pool_topk", **dict(pool, max_cand_blocks=4096)) == -2
    assert _call(L, "csa2_sparse_attn_pool_topk", **dict(pool, scores_stride=1000)) == -2
    assert _call(L, "csa2_sparse_attn_pool_topk", **dict(pool, block=0)) == -2
    assert _call(L, "csa2_sparse_attn_pool_topk", **pool) == -5


def test_append_needs_its_sequence_alone():
    """A query that appends a row writes it while the call runs, so no other query of the
    call may read that sequence; the binding checks it before anything is launched."""
    import torch
    from fp4_kv_cache_layer_amd import csa2 as C
    row = torch.tensor([5, 7, -1, 9], dtype=torch.int64)      # queries 0, 1 and 3 append
    ok = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    C._check_append_sequences(row, ok, 100)
    C._check_append_sequences(row, torch.tensor([0, 1, 2, 2], dtype=torch.int32), 8)   # row 9 is past seq_cap
    for bad in ([0, 0, 2, 3], [0, 1, 1, 3], [3, 1, 2, 3]):    # two appenders, or an appender and a reader
        with pytest.raises(ValueError):
            C._check_append_sequences(row, torch.tensor(bad, dtype=torch.int32), 100)

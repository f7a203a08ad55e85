"""The C-ABI library loads and exports every symbol include/csa2.h declares; argument
validation rejects bad calls on the host, before anything reaches the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401  (the binding always loads torch's HIP runtime first)
    from fp4_kv_cache_layer_amd.build import LIB_PATH
    if not os.path.exists(LIB_PATH):
        pytest.fail("libcsa2.so is not built; run __graft_entry__.build()")
    return ctypes.CDLL(LIB_PATH)


def test_header_declares_the_calls():
    names = _declared()
    for n in ("csa2_quantize_kv", "csa2_index_score", "csa2_index_topk", "csa2_topk", "csa2_build_pool",
              "csa2_sparse_attn"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings_and_version(L):
    L.csa2_status_string.restype = ctypes.c_char_p
    for code in (0, -1, -2, -3, -4, -5):
        assert L.csa2_status_string(code)
    assert L.csa2_status_string(-99) == b"unknown status"
    assert L.csa2_version() >= 100


def test_validation_before_launch(L):
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.csa2_quantize_kv.argtypes = [vp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, vp]
    fake = vp(0x1000)   # never dereferenced: every call below fails validation first
    assert L.csa2_quantize_kv(None, 0, 4, 512, 0, None, 4, fake, fake, None) == -1
    assert L.csa2_quantize_kv(fake, 0, 4, 500, 0, None, 4, fake, fake, None) == -2     # dim % 16
    assert L.csa2_quantize_kv(fake, 0, 4, 512, 9, None, 4, fake, fake, None) == -3     # fmt
    assert L.csa2_quantize_kv(fake, 0, 4, 512, 0, None, 4, vp(0x1001), fake, None) == -2  # misaligned
    assert L.csa2_quantize_kv(fake, 0, 0, 512, 0, None, 4, fake, fake, None) == 0      # empty: no launch
    L.csa2_topk.argtypes = [vp, i64, ctypes.c_int, vp, i64, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                            vp, ctypes.c_size_t, vp]
    assert L.csa2_topk(fake, 100, 2, fake, 100, None, None, 8, 0, 4096, fake, fake, None, 0, None) == -2  # k > 2048
    assert L.csa2_topk(fake, 10, 2, fake, 100, None, None, 8, 0, 16, fake, fake, None, 0, None) == -2   # stride
    assert L.csa2_topk(fake, 1 << 20, 2, fake, 1 << 20, None, None, 8, 0, 512, fake, fake, None, 0, None) == -5
    L.csa2_topk_workspace_bytes.restype = ctypes.c_size_t
    L.csa2_topk_workspace_bytes.argtypes = [ctypes.c_int, i64, ctypes.c_int]
    assert L.csa2_topk_workspace_bytes(2, 8192, 512) == 0           # one segment: no scratch
    assert L.csa2_topk_workspace_bytes(2, 1 << 20, 512) > 0
    L.csa2_sparse_attn.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, i64, ctypes.c_int, vp, vp,
                                   ctypes.c_int, vp, i64, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                   vp, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    args = [fake, 4, 64, 512, fake, fake, 100, 1, fake, fake, 512, fake, 128, fake, fake, fake, None, 0, 128, 0.05,
            fake, 0, None, None, 0, None]
    a = list(args); a[2] = 40                       # heads not a multiple of 16
    assert L.csa2_sparse_attn(*a) == -2
    a = list(args); a[18] = 256                     # window > swa_cap
    assert L.csa2_sparse_attn(*a) == -2
    a = list(args); a[21] = 7                       # out dtype
    assert L.csa2_sparse_attn(*a) == -3
    a = list(args); a[16] = fake; a[17] = 9         # window-append dtype
    assert L.csa2_sparse_attn(*a) == -3
    a = list(args); a[9] = None                     # idx NULL with k > 0
    assert L.csa2_sparse_attn(*a) == -1
    assert L.csa2_sparse_attn(*args) == -5          # split over workgroups needs a workspace


def test_select_in_attention_validation(L):
    """csa2_index_segments / csa2_sparse_attn_topk reject bad calls on the host."""
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    fake = vp(0x1000)   # never dereferenced
    L.csa2_segment_keys.restype = i64
    L.csa2_segment_keys.argtypes = [i64, i32]
    assert L.csa2_segment_keys(131072, 512) == 8192
    assert L.csa2_segment_keys(131073, 512) == 8704
    assert L.csa2_segment_keys(0, 512) == 512
    assert L.csa2_segment_keys(100, 0) == 0
    L.csa2_index_segments.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, i64, i32, vp, vp, i32, vp, vp]
    seg = [fake, fake, fake, 4, 16, 128, fake, fake, 4096, 1, fake, fake, 512, fake, None]
    a = list(seg); a[13] = None                     # no key buffer
    assert L.csa2_index_segments(*a) == -1
    a = list(seg); a[12] = 4096                     # k > 2048
    assert L.csa2_index_segments(*a) == -2
    a = list(seg); a[5] = 64                        # indexer dim
    assert L.csa2_index_segments(*a) == -2
    L.csa2_sparse_attn_topk.argtypes = [vp, i32, i32, i32, vp, vp, i64, i32, vp, vp, i32, i32, vp, vp, vp, i64, vp,
                                        vp, vp, vp, i32, i32, ctypes.c_float, vp, i32, vp, vp, ctypes.c_size_t, vp]
    att = [fake, 4, 64, 512, fake, fake, 100, 1, fake, fake, 8192, 512, fake, fake, fake, 128, fake, fake, fake, None,
           0, 128, 0.05, fake, 0, None, None, 0, None]
    a = list(att); a[9] = None                      # no candidate keys
    assert L.csa2_sparse_attn_topk(*a) == -1
    a = list(att); a[12] = None                     # no index output
    assert L.csa2_sparse_attn_topk(*a) == -1
    a = list(att); a[10] = 8193                     # more survivors than one selection holds
    assert L.csa2_sparse_attn_topk(*a) == -2
    a = list(att); a[11] = 0                        # k = 0
    assert L.csa2_sparse_attn_topk(*a) == -2
    assert L.csa2_sparse_attn_topk(*att) == -5      # split over workgroups needs a workspace


def test_pool_select_in_attention_validation(L):
    """csa2_sparse_attn_pool_topk rejects bad pools on the host."""
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    fake = vp(0x1000)   # never dereferenced
    L.csa2_sparse_attn_pool_topk.argtypes = [vp, i32, i32, i32, vp, vp, i64, i32, vp, vp, i64, vp, vp, vp, i32, i32,
                                             i32, vp, vp, vp, i64, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp, i32,
                                             vp, vp, ctypes.c_size_t, vp]
    att = [fake, 4, 64, 512, fake, fake, 100, 1, fake, fake, 16384, fake, fake, fake, 8, 2048, 512, fake, fake, fake,
           128, fake, fake, fake, None, 0, 128, 0.05, fake, 0, None, None, 0, None]
    a = list(att); a[9] = None                      # no scores
    assert L.csa2_sparse_attn_pool_topk(*a) == -1
    a = list(att); a[15] = 4096                     # more slots than one selection holds
    assert L.csa2_sparse_attn_pool_topk(*a) == -2
    a = list(att); a[10] = 1000                     # score stride below the pool's slots
    assert L.csa2_sparse_attn_pool_topk(*a) == -2
    a = list(att); a[14] = 0                        # block
    assert L.csa2_sparse_attn_pool_topk(*a) == -2
    assert L.csa2_sparse_attn_pool_topk(*att) == -5  # split over workgroups needs a workspace


def test_index_score_q_validation(L):
    """csa2_index_score_q (indexer Q unquantised) rejects bad arguments before any launch."""
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.csa2_index_score_q.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, i64, i32, vp, vp, vp, vp, i32, i32, vp, i64,
                                     vp]
    fake = vp(0x1000)   # never dereferenced: every call below fails validation first or launches nothing
    args = [fake, 0, fake, 4, 16, 128, fake, fake, 4096, 2, fake, fake, None, None, 8, 0, fake, 4096, None]
    a = list(args); a[1] = 5                        # Q dtype
    assert L.csa2_index_score_q(*a) == -3
    a = list(args); a[0] = None                     # Q NULL
    assert L.csa2_index_score_q(*a) == -1
    a = list(args); a[0] = vp(0x1004)               # Q not 16-byte aligned
    assert L.csa2_index_score_q(*a) == -2
    a = list(args); a[5] = 64                       # indexer dim
    assert L.csa2_index_score_q(*a) == -2
    a = list(args); a[4] = 17                       # indexer heads
    assert L.csa2_index_score_q(*a) == -2
    a = list(args); a[17] = 100                     # scores stride below seq_cap
    assert L.csa2_index_score_q(*a) == -2
    a = list(args); a[12] = fake                    # pool map without its counts
    assert L.csa2_index_score_q(*a) == -1
    a = list(args); a[3] = 0                        # no rows: nothing launched
    assert L.csa2_index_score_q(*a) == 0

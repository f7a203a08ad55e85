"""GPU parity of each C-ABI call against the oracle, at sizes the oracle finishes in
seconds that still span several tiles / segments and a ragged tail."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def C():
    from fp4_kv_cache_layer_amd import csa2
    csa2.csa2_init()
    return csa2


def _adversarial_rows(rng, rows, dim, group):
    """Rows whose group maxima and elements sit on and 1 ulp beside rounding midpoints."""
    mids = [(O.E4M3[c] + O.E4M3[c + 1]) / 2 for c in range(0x7E)]
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    x = np.zeros((rows, dim), np.float32)
    for r in range(rows):
        for g in range(dim // group):
            m = mids[rng.integers(len(mids))]
            a = np.float32(6 * m)
            s = O.E4M3[O.nearest_code(np.array([a / 6.0]), O.E4M3[:0x7F], np.arange(0x7F))[0]]
            v = (s * t[rng.integers(len(t), size=group)]).astype(np.float32)
            v[0] = a
            nudge = rng.integers(3, size=group)
            v = np.where(nudge == 1, np.nextafter(v, np.float32(0)), v)
            v = np.where(nudge == 2, np.nextafter(v, np.float32(1e9)), v)
            v *= rng.choice([-1, 1], size=group).astype(np.float32)
            x[r, g * group:(g + 1) * group] = rng.permutation(v)
    return x


def _mx_adversarial_rows(rng, rows, dim):
    """MXFP4 groups (32 channels) whose maximum fixes the power-of-two scale 2^E and whose
    elements sit on and 1 ulp beside the E2M1 midpoints times 2^E, in the saturation range
    [6, 8) x 2^E, or at zero, with scales from the subnormal 2^-127 up to 2^120."""
    t = np.array([0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 7.0, 7.9])
    x = np.zeros((rows, dim), np.float32)
    for r in range(rows):
        for g in range(dim // 32):
            s = np.float32(2.0 ** int(rng.choice([-127, -126, -125, -60, -3, 0, 4, 60, 120])))
            v = (s * t[rng.integers(len(t), size=32)]).astype(np.float32)
            v[0] = np.float32(4.0) * s          # floor(log2 amax) = E + 2
            nudge = rng.integers(3, size=32)
            nudge[0] = 0
            v = np.where(nudge == 1, np.nextafter(v, np.float32(0)), v)
            v = np.where(nudge == 2, np.nextafter(v, np.float32(1e38)), v)
            v *= rng.choice([-1, 1], size=32).astype(np.float32)
            x[r, g * 32:(g + 1) * 32] = rng.permutation(v)
    return x


def _special_rows(dim):
    rows = [np.zeros(dim), -np.zeros(dim), np.full(dim, 3000.0), np.full(dim, 1e-30),
            np.linspace(-22.6, 22.6, dim), np.full(dim, 448.0), np.full(dim, 2.0 ** -130)]
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "fp8"])
@pytest.mark.parametrize("src_dt", ["f32", "bf16"])
def test_quantize_bitexact(C, fmt, src_dt):
    _say("quantize", fmt, src_dt)
    rng = np.random.default_rng(1)
    dim = 512 if fmt != "mxfp4" else 128
    group = {"nvfp4": 16, "mxfp4": 32, "fp8": 8}[fmt]
    x = np.concatenate([
        (rng.normal(size=(300, dim)) * 10.0 ** rng.uniform(-3, 2, size=(300, 1))).astype(np.float32),
        _adversarial_rows(rng, 40, dim, 16 if fmt == "nvfp4" else group),
        _special_rows(dim)] + ([_mx_adversarial_rows(rng, 60, dim)] if fmt == "mxfp4" else []))
    xt = torch.from_numpy(x).cuda()
    if src_dt == "bf16":
        xt = xt.to(torch.bfloat16)
        x = xt.float().cpu().numpy()
    rows = x.shape[0]
    # scatter into a larger table with a permutation; two rows point outside and are skipped
    dst_rows = rows + 5
    dst = rng.permutation(dst_rows)[:rows].astype(np.int64)
    dst[3], dst[7] = -1, dst_rows + 2
    f = {"nvfp4": C.FMT_NVFP4, "mxfp4": C.FMT_MXFP4, "fp8": C.FMT_FP8}[fmt]
    per = dim if fmt == "fp8" else dim // 2
    codes = torch.full((dst_rows, per), 0xAB, dtype=torch.uint8, device="cuda")
    scales = None if fmt == "fp8" else torch.full((dst_rows, dim // group), 0xCD, dtype=torch.uint8, device="cuda")
    C.csa2_quantize_kv(xt, f, codes, scales, torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    if fmt == "nvfp4":
        rc, rs = O.quantize_nvfp4(x)
    elif fmt == "mxfp4":
        rc, rs = O.quantize_mxfp4(x)
    else:
        rc, rs = O.quantize_fp8(x), None
    ok = (dst >= 0) & (dst < dst_rows)
    assert np.array_equal(gc[dst[ok]], rc[ok])
    untouched = np.setdiff1d(np.arange(dst_rows), dst[ok])
    assert np.all(gc[untouched] == 0xAB)
    if rs is not None:
        gs = scales.cpu().numpy()
        assert np.array_equal(gs[dst[ok]], rs[ok])
        assert np.all(gs[untouched] == 0xCD)


def test_quantize_multi_matches_single_calls(C):
    """One launch of several jobs (all formats, both input types, scatter rows, a job with no
    rows) writes exactly what the same jobs do as separate calls."""
    _say("quantize multi")
    rng = np.random.default_rng(11)
    mk = lambda r, d, dt: torch.from_numpy((rng.normal(size=(r, d)) * 3).astype(np.float32)).cuda().to(dt)
    specs = [(C.FMT_NVFP4, 512, 70, torch.float32), (C.FMT_MXFP4, 128, 33, torch.bfloat16),
             (C.FMT_FP8, 512, 50, torch.float32), (C.FMT_MXFP4, 2048, 9, torch.float32),
             (C.FMT_NVFP4, 512, 0, torch.bfloat16)]
    outs_a, outs_b, jobs_a = [], [], []
    for fmt, dim, rows, dt in specs:
        src = mk(rows, dim, dt)
        dst_rows = rows + 7
        dst = torch.from_numpy(rng.permutation(dst_rows)[:rows].astype(np.int64)).cuda()
        per = dim if fmt == C.FMT_FP8 else dim // 2
        g = {C.FMT_NVFP4: 16, C.FMT_MXFP4: 32, C.FMT_FP8: 1}[fmt]
        pair = []
        for _ in range(2):
            codes = torch.full((dst_rows, per), 0x5A, dtype=torch.uint8, device="cuda")
            scales = None if fmt == C.FMT_FP8 else torch.full((dst_rows, dim // g), 0xA5, dtype=torch.uint8,
                                                              device="cuda")
            pair.append((codes, scales))
        C.csa2_quantize_kv(src, fmt, pair[0][0], pair[0][1], dst)
        jobs_a.append((src, fmt, pair[1][0], pair[1][1], dst))
        outs_a.append(pair[0])
        outs_b.append(pair[1])
    C.csa2_quantize_kv_multi(jobs_a)
    torch.cuda.synchronize()
    for (ca, sa), (cb, sb) in zip(outs_a, outs_b):
        assert torch.equal(ca, cb)
        assert (sa is None) == (sb is None) and (sa is None or torch.equal(sa, sb))


def _score_case(seed, n_seq, seq_cap, n_vis, idx_heads, index_fmt="mxfp4", swa_cap=128):
    wl = G.workloads.Workload(
        name="small", seed=seed, n_seq=n_seq, seq_cap=seq_cap, m=1, heads=16, idx_heads=idx_heads,
        q_seq=np.array([i % n_seq for i in range(len(n_vis))], np.int32),
        q_pos=np.array(n_vis, np.int64) - 1, replay_start=np.zeros(len(n_vis), np.int64), layers=("full",),
        new_entries=(0, 0), swa_cap=swa_cap)
    return G.Case(wl, index_fmt=index_fmt)


@pytest.mark.parametrize("idx_heads,fmt", [(16, "mxfp4"), (8, "mxfp4"), (5, "mxfp4"), (16, "nvfp4"), (5, "nvfp4")])
def test_index_score_parity(C, idx_heads, fmt):
    """Scores of the MXFP4 indexer (scaled FP4 MFMA) and of the NVFP4-style one (dequantised
    fp16 MFMA) against the oracle's fp64 scores; the caches and the quantised indexer Q
    bit-exact against the oracle's quantiser."""
    _say("index_score", idx_heads, fmt)
    case = _score_case(10 + idx_heads, 3, 9000, [9000, 4097, 1, 8999, 64], idx_heads, fmt)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, idx_heads, wl.seq_cap, index_fmt=fmt)
    st.scores.fill_(12345.0)
    st.quantize_index_q(q_idx)
    st.score(caches, w, q_seq, n_vis)
    torch.cuda.synchronize()
    gs = st.scores.cpu().numpy()
    for qi in range(wl.n_q):
        seq = int(wl.q_seq[qi])
        oc = case.oracle_caches(seq)
        assert np.array_equal(caches.ik_codes[seq].cpu().numpy(), oc.ik_codes)
        assert np.array_equal(caches.ik_scales[seq].cpu().numpy(), oc.ik_scales)
        qc, qs, wq, _ = case.oracle_query(0, qi)
        assert np.array_equal(st.qi_codes[qi].cpu().numpy(), qc)
        assert np.array_equal(st.qi_scales[qi].cpu().numpy(), qs)
        nv = int(wl.n_vis[qi])
        _, ref = O.full_scores(qc, qs, wq, oc, nv)
        got = gs[qi, :nv]
        assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max())
        assert np.all(gs[qi, nv:] == 12345.0)   # positions past n_vis untouched


@pytest.mark.parametrize("group", [1, 3, 8])
def test_index_score_grouped_matches_per_row(C, group):
    """Rows in groups sharing a sequence: bit-identical to the per-row kernel's scores; a row
    of another sequence than its group's first row, and positions past n_vis, untouched."""
    _say("index_score grouped", group)
    q_seq = np.array([0, 0, 0, 1, 1, 1, 2, 2, 0, 1], np.int32)
    n_vis = np.array([9000, 8990, 4097, 9000, 1, 64, 8999, 5000, 7000, 3333], np.int64)
    wl = G.workloads.Workload(name="grouped", seed=31, n_seq=3, seq_cap=9000, m=1, heads=16, idx_heads=16,
                              q_seq=q_seq, q_pos=n_vis - 1, replay_start=np.zeros(10, np.int64),
                              layers=("full",), new_entries=(0, 0))
    case = G.Case(wl)
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq_d, n_vis_d, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap)
    st.quantize_index_q(q_idx)
    st.scores.fill_(12345.0)
    st.score(caches, w, q_seq_d, n_vis_d)
    ref = st.scores.clone()
    st.scores.fill_(-777.0)
    C.csa2_index_score_grouped(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq_d, n_vis_d,
                               group, st.scores)
    torch.cuda.synchronize()
    got, ref = st.scores.cpu().numpy(), ref.cpu().numpy()
    for qi in range(wl.n_q):
        nv = int(n_vis[qi])
        if q_seq[qi] == q_seq[(qi // group) * group]:
            assert np.array_equal(got[qi, :nv], ref[qi, :nv]), qi
            assert np.all(got[qi, nv:] == -777.0)
        else:
            assert np.all(got[qi] == -777.0), qi
    # and against the oracle on one row per sequence
    for qi in (1, 3, 6):
        if q_seq[qi] != q_seq[(qi // group) * group]:
            continue
        oc = case.oracle_caches(int(q_seq[qi]))
        qc, qs, wq, _ = case.oracle_query(0, qi)
        nv = int(n_vis[qi])
        _, r = O.full_scores(qc, qs, wq, oc, nv)
        assert np.all(np.abs(got[qi, :nv] - r) <= 1e-5 * np.abs(r) + 1e-6 * np.abs(r).max())


def _grouped_two_call(C, st, caches, w, q_seq_d, n_vis_d, group, k):
    """Reference for the fused grouped selection: grouped scores, then csa2_topk."""
    idx = torch.full((st.n_q, k), -5, dtype=torch.int32, device="cuda")
    cnt = torch.full((st.n_q,), -5, dtype=torch.int32, device="cuda")
    C.csa2_index_score_grouped(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq_d, n_vis_d,
                               group, st.scores)
    C.csa2_topk(st.scores, n_vis_d, st.seq_cap, k, idx, cnt)
    return idx, cnt


@pytest.mark.parametrize("group,k", [(8, 512), (3, 512), (8, 7), (8, 704), (1, 512)])
def test_index_topk_grouped_matches_score_then_topk(C, group, k):
    """Grouped rows scored and selected in one pass (no score array): exactly the index set
    of grouped scoring followed by csa2_topk, over a cache of 70,000 entries (four ranges
    whose survivors meet in the last level), ragged visible counts (a row of 1 entry, rows
    ending inside a range, a row covering all) and rows of another sequence than their
    group's first row (which get an empty set)."""
    _say("index_topk_grouped", group, k)
    q_seq = np.array([0, 0, 0, 1, 1, 1, 2, 2, 0, 1, 2, 2], np.int32)
    n_vis = np.array([70000, 69990, 40097, 70000, 1, 64, 69999, 33000, 700, 31000, 65536, 65537], np.int64)
    n_q = q_seq.size
    wl = G.workloads.Workload(name="grouped_topk", seed=47, n_seq=3, seq_cap=70000, m=1, heads=16, idx_heads=16,
                              q_seq=q_seq, q_pos=n_vis - 1, replay_start=np.zeros(n_q, np.int64),
                              layers=("full",), new_entries=(0, 0))
    case = G.Case(wl)
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq_d, n_vis_d, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(n_q, 16, 16, wl.seq_cap, k=k)
    st.quantize_index_q(q_idx)
    ref_idx, ref_cnt = _grouped_two_call(C, st, caches, w, q_seq_d, n_vis_d, group, k)
    idx = torch.full((n_q, k), -5, dtype=torch.int32, device="cuda")
    cnt = torch.full((n_q,), -5, dtype=torch.int32, device="cuda")
    ws = torch.empty(C.csa2_index_topk_grouped_workspace_bytes(n_q, wl.seq_cap, k, group), dtype=torch.uint8, device="cuda")
    for _ in range(2):   # a second call over the first one's workspace
        C.csa2_index_topk_grouped(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq_d, n_vis_d,
                                  group, k, idx, cnt, ws)
        torch.cuda.synchronize()
        gi, gc, ri, rc = idx.cpu().numpy(), cnt.cpu().numpy(), ref_idx.cpu().numpy(), ref_cnt.cpu().numpy()
        for qi in range(n_q):
            if q_seq[qi] == q_seq[(qi // group) * group]:
                assert gc[qi] == rc[qi] == min(k, n_vis[qi]), qi
                assert np.array_equal(gi[qi], ri[qi]), qi
            else:
                assert gc[qi] == 0 and np.all(gi[qi] == -1), qi
    # and the oracle's rule on one row per sequence
    for qi in (1, 3, 6):
        if q_seq[qi] != q_seq[(qi // group) * group]:
            continue
        oc = case.oracle_caches(int(q_seq[qi]))
        qc, qs, wq, _ = case.oracle_query(0, qi)
        pos, sc = O.full_scores(qc, qs, wq, oc, int(n_vis[qi]))
        G.topk_accept(gi[qi], int(gc[qi]), pos, sc, k)


def test_index_topk_grouped_rising_scores(C):
    """The worst order for a running selection: scores that rise with the position (and
    plateau where neighbouring entries quantise alike), so almost every entry enters the
    candidate lists and the lists are cut down after every step.  Same result as grouped
    scores followed by csa2_topk, ties going to the lower position."""
    _say("index_topk_grouped rising")
    n = 40000
    rng = np.random.default_rng(3)
    v = rng.standard_normal(128).astype(np.float32)
    lat = ((np.arange(n, dtype=np.float32)[:, None] + 1.0) / n) * v[None, :]
    from fp4_kv_cache_layer_amd.layer import Caches, Csa2Step
    caches = Caches.empty(1, n, (0,), 128)
    C.csa2_quantize_kv(torch.from_numpy(lat).cuda(), C.FMT_MXFP4, caches.ik_codes[0], caches.ik_scales[0])
    n_q = 8
    st = Csa2Step(n_q, 16, 16, n)
    q = torch.from_numpy(np.tile(v, (n_q, 16, 1)) * (1.0 + 0.1 * np.arange(n_q)[:, None, None])).float().cuda()
    st.quantize_index_q(q)
    w = torch.ones(n_q, 16, dtype=torch.float32, device="cuda")
    q_seq_d = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    n_vis_d = torch.tensor([n - 13 * i for i in range(n_q)], dtype=torch.int64, device="cuda")
    ref_idx, ref_cnt = _grouped_two_call(C, st, caches, w, q_seq_d, n_vis_d, 8, 512)
    idx = torch.full((n_q, 512), -5, dtype=torch.int32, device="cuda")
    cnt = torch.full((n_q,), -5, dtype=torch.int32, device="cuda")
    C.csa2_index_topk_grouped(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq_d, n_vis_d, 8,
                              512, idx, cnt)
    torch.cuda.synchronize()
    assert torch.equal(cnt, ref_cnt) and torch.equal(idx, ref_idx)
    assert int(idx[0, 0].item()) > n // 2        # the set really sits at the rising end


@pytest.mark.timeout(300)
def test_index_topk_grouped_wide_offsets(C):
    """A cache whose entry offsets within a sequence do not fit 32 bits (1,048,579 entries at
    an entry stride of 4,160 bytes: 4.36 GB of codes), so the grouped selection takes its
    64-bit address path: the same index sets as grouped scores followed by csa2_topk."""
    _say("index_topk_grouped wide offsets")
    n, pitch = (1 << 20) + 3, 4160
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    store = torch.zeros(n, pitch, dtype=torch.uint8, device="cuda")
    k_codes = store[:, :64]
    k_scales = torch.zeros(1, n, 4, dtype=torch.uint8, device="cuda")
    wl = G.workloads.Workload(name="wide", seed=53, n_seq=1, seq_cap=n, m=1, heads=16, idx_heads=16,
                              q_seq=np.zeros(8, np.int32), q_pos=np.zeros(8, np.int64),
                              replay_start=np.zeros(8, np.int64), layers=("full",), new_entries=(0, 0))
    for r0 in range(0, n, 1 << 16):
        rows = min(1 << 16, n - r0)
        lat = torch.from_numpy(wl.index_k_latents(0, r0, rows)).cuda()
        C.csa2_quantize_kv(lat, C.FMT_MXFP4, k_codes[r0:r0 + rows], k_scales[0, r0:r0 + rows])
    n_q = 8
    st = Csa2Step(n_q, 16, 16, n)
    q = torch.from_numpy(np.random.default_rng(5).standard_normal((n_q, 16, 128)).astype(np.float32)).cuda()
    st.quantize_index_q(q)
    w = torch.from_numpy(np.random.default_rng(6).random((n_q, 16)).astype(np.float32)).cuda()
    q_seq_d = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    n_vis_d = torch.tensor([n, n - 5, n - 70000, 4097, n - 1, 600000, 1, n - 64], dtype=torch.int64, device="cuda")
    codes3 = k_codes.unsqueeze(0)
    assert codes3.stride(1) == pitch
    ref_idx, ref_cnt = _grouped_two_call(C, st, Caches3(codes3, k_scales), w, q_seq_d, n_vis_d, 8, 512)
    idx = torch.full((n_q, 512), -5, dtype=torch.int32, device="cuda")
    cnt = torch.full((n_q,), -5, dtype=torch.int32, device="cuda")
    C.csa2_index_topk_grouped(st.qi_codes, st.qi_scales, w, codes3, k_scales, q_seq_d, n_vis_d, 8, 512, idx, cnt)
    torch.cuda.synchronize()
    assert torch.equal(cnt, ref_cnt) and torch.equal(idx, ref_idx)
    assert int(cnt[6].item()) == 1 and int(idx[6, 0].item()) == 0
    del store, k_codes, codes3
    torch.cuda.empty_cache()


class Caches3:
    """The indexer-K views _grouped_two_call reads (ik_codes, ik_scales)."""

    def __init__(self, ik_codes, ik_scales):
        self.ik_codes, self.ik_scales = ik_codes, ik_scales


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_index_score_pool_slots(C, fmt):
    _say("index_score pool", fmt)
    case = _score_case(21, 2, 6000, [6000, 5003, 333], 16, fmt)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, max_blocks=300, index_fmt=fmt)
    rng = np.random.default_rng(3)
    blocks = np.full((wl.n_q, 300), -1, np.int32)
    ncb = np.array([300, 250, 60], np.int32)
    for qi in range(wl.n_q):
        nb = -(-int(wl.n_vis[qi]) // 8)
        b = np.sort(rng.choice(nb + 20, size=ncb[qi], replace=False)).astype(np.int32)  # some beyond n_vis
        blocks[qi, :ncb[qi]] = b
    blocks[1, 5] = -1
    st.pool.copy_(torch.from_numpy(blocks))
    st.pool_count.copy_(torch.from_numpy(ncb))
    st.quantize_index_q(q_idx)
    st.score(caches, w, q_seq, n_vis, in_pool=True)
    torch.cuda.synchronize()
    gs = st.scores.cpu().numpy()
    for qi in range(wl.n_q):
        seq = int(wl.q_seq[qi])
        oc = case.oracle_caches(seq)
        qc, qs, wq, _ = case.oracle_query(0, qi)
        nv = int(wl.n_vis[qi])
        for slot in range(300 * 8):
            b = blocks[qi, slot // 8]
            pos = b * 8 + slot % 8
            valid = slot < ncb[qi] * 8 and b >= 0 and pos < nv
            if not valid:
                assert gs[qi, slot] == -np.inf
        slots = np.array([s for s in range(ncb[qi] * 8) if blocks[qi, s // 8] >= 0
                          and blocks[qi, s // 8] * 8 + s % 8 < nv])
        pos = blocks[qi, slots // 8].astype(np.int64) * 8 + slots % 8
        _, ref = O.full_scores(qc, qs, wq, oc, nv, cand=pos)
        got = gs[qi, slots]
        assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("pool,q_dt,heads", [(True, "f32", 16), (False, "f32", 16), (True, "bf16", 16),
                                             (False, "bf16", 5), (True, "f32", 5)])
def test_index_score_q_matches_quantize_then_score(C, pool, q_dt, heads):
    """csa2_index_score_q (the indexer Q unquantised, quantised inside the scoring call) gives
    scores bit-identical to csa2_quantize_kv (MXFP4) followed by csa2_index_score on the same
    values, inside a pool (every slot, -inf pads included) and over all visible entries;
    the quantiser and the scores are pinned to the oracle by test_quantize_bitexact and
    test_index_score_parity / test_index_score_pool_slots."""
    _say("index_score_q", pool, q_dt, heads)
    case = _score_case(31 + heads, 2, 6000, [6000, 5003, 333], heads)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, heads, wl.seq_cap, max_blocks=300)
    if pool:
        rng = np.random.default_rng(5)
        blocks = np.full((wl.n_q, 300), -1, np.int32)
        ncb = np.array([300, 250, 60], np.int32)
        for qi in range(wl.n_q):
            nb = -(-int(wl.n_vis[qi]) // 8)
            blocks[qi, :ncb[qi]] = np.sort(rng.choice(nb + 20, size=ncb[qi], replace=False))  # some beyond n_vis
        blocks[1, 5] = -1
        st.pool.copy_(torch.from_numpy(blocks))
        st.pool_count.copy_(torch.from_numpy(ncb))
    q_in = q_idx if q_dt == "f32" else q_idx.to(torch.bfloat16)
    st.quantize_index_q(q_in.float().contiguous())      # exact widening of bf16 values
    st.score(caches, w, q_seq, n_vis, in_pool=pool)
    torch.cuda.synchronize()
    ref = st.scores.clone()
    st.scores.fill_(7.0)
    st.score_q(caches, q_in.contiguous(), w, q_seq, n_vis, in_pool=pool)
    torch.cuda.synchronize()
    if pool:
        assert torch.equal(st.scores[:, :300 * 8], ref[:, :300 * 8])
    else:
        for qi in range(wl.n_q):
            nv = int(wl.n_vis[qi])
            assert torch.equal(st.scores[qi, :nv], ref[qi, :nv])


@pytest.mark.parametrize("q_dt,heads", [("f32", 16), ("bf16", 16), ("f32", 5)])
def test_scoring_calls_take_unquantised_q(C, q_dt, heads):
    """The fused scoring calls with the indexer Q given unquantised (fmt CSA2_FMT_MXFP4_Q_F32
    / _BF16 at the boundary: q_codes the f32 / bf16 Q, q_scales None) return exactly what
    csa2_quantize_kv (MXFP4) followed by the same call on its codes returns: csa2_index_score,
    csa2_index_topk (all visible entries and inside a pool), csa2_index_segments (its keys)
    and csa2_index_topk_pool (Top-K and pool).  The quantised-Q calls are pinned to the oracle
    by the tests above and below."""
    _say("unquantised Q", q_dt, heads)
    case = _score_case(41 + heads, 2, 20000, [20000, 17001, 333], heads)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    k = 512
    st = Csa2Step(wl.n_q, 16, heads, wl.seq_cap, max_blocks=300)
    rng = np.random.default_rng(9)
    blocks = np.full((wl.n_q, 300), -1, np.int32)
    ncb = np.array([300, 250, 40], np.int32)
    for qi in range(wl.n_q):
        nb = -(-int(wl.n_vis[qi]) // 8)
        blocks[qi, :ncb[qi]] = np.sort(rng.choice(nb, size=ncb[qi], replace=False))
    st.pool.copy_(torch.from_numpy(blocks))
    st.pool_count.copy_(torch.from_numpy(ncb))
    q_in = (q_idx if q_dt == "f32" else q_idx.to(torch.bfloat16)).contiguous()
    st.quantize_index_q(q_in.float().contiguous())      # exact widening of bf16 values
    ik = (caches.ik_codes, caches.ik_scales)
    n_q = wl.n_q

    def outs():
        return {"idx": torch.full((n_q, k), 77, dtype=torch.int32, device="cuda"),
                "cnt": torch.full((n_q,), 77, dtype=torch.int32, device="cuda"),
                "blk": torch.full((n_q, 64), 77, dtype=torch.int32, device="cuda"),
                "bcnt": torch.full((n_q,), 77, dtype=torch.int32, device="cuda"),
                "keys": torch.full((n_q, C.csa2_segment_keys(wl.seq_cap, k)), 77, dtype=torch.int64, device="cuda"),
                "sc": torch.full((n_q, wl.seq_cap), 7.0, dtype=torch.float32, device="cuda")}

    def run(qc, qs):
        o = {"plain": outs(), "pool": outs(), "build": outs()}
        C.csa2_index_score(qc, qs, w, *ik, q_seq, n_vis, o["plain"]["sc"])
        C.csa2_index_topk(qc, qs, w, *ik, q_seq, n_vis, k, o["plain"]["idx"], o["plain"]["cnt"])
        C.csa2_index_segments(qc, qs, w, *ik, q_seq, n_vis, k, o["plain"]["keys"])
        C.csa2_index_topk(qc, qs, w, *ik, q_seq, n_vis, k, o["pool"]["idx"], o["pool"]["cnt"], None, st.pool,
                          st.pool_count, 8)
        C.csa2_index_topk_pool(qc, qs, w, *ik, q_seq, n_vis, k, o["build"]["idx"], o["build"]["cnt"],
                               o["build"]["blk"], o["build"]["bcnt"], 8)
        torch.cuda.synchronize()
        return o

    ref = run(st.qi_codes, st.qi_scales)
    got = run(q_in, None)
    for part in ("plain", "pool", "build"):
        for name in ("idx", "cnt", "blk", "bcnt", "keys"):
            assert torch.equal(got[part][name], ref[part][name]), (part, name)
    for qi in range(n_q):
        nv = int(wl.n_vis[qi])
        assert torch.equal(got["plain"]["sc"][qi, :nv], ref["plain"]["sc"][qi, :nv])
    with pytest.raises(ValueError):   # NVFP4 and grouped calls take quantised Q only
        C.csa2_index_segments(q_in, None, w, *ik, q_seq, n_vis, k, ref["plain"]["keys"], fmt=C.FMT_NVFP4)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_scoring_calls_append_new_entries(C, dt):
    """A fused scoring call given a csa2_append writes each query's new main-KV row (NVFP4)
    and indexer-K row (MXFP4) itself and scores with the new indexer-K row: the caches and
    the results equal csa2_quantize_kv of the two rows followed by the call without an
    append (csa2_index_segments, csa2_index_topk, csa2_index_topk_pool; rows at the first and
    last entry of a segment, the last visible entry, one past the visible range, and none;
    the quantiser is pinned to the oracle by test_quantize_bitexact).  With the unquantised
    indexer Q as well, the step's quantise launch has nothing left to do."""
    _say("append", dt)
    n_vis = [20000, 17001, 8193, 333, 100]
    rows = [19999, 17000, 8192, 5000, -1]
    case = _score_case(61, 5, 20000, n_vis, 16)      # one sequence per query
    wl = case.wl
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis_t, _, _ = case.gpu_meta()
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    gen = torch.Generator().manual_seed(7)
    main = torch.randn(wl.n_q, 512, generator=gen).to(tdt).cuda()
    index = torch.randn(wl.n_q, 128, generator=gen).to(tdt).cuda()
    main[1, :16] = 0.0                                 # an all-zero NVFP4 group
    row_t = torch.tensor(rows, dtype=torch.int64, device="cuda")
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap)
    k = 512
    st.quantize_index_q(q_idx)

    def run(caches, append):
        ik = (caches.ik_codes, caches.ik_scales)
        o = {"keys": torch.full((wl.n_q, C.csa2_segment_keys(wl.seq_cap, k)), 77, dtype=torch.int64, device="cuda"),
             "idx": torch.full((wl.n_q, k), 77, dtype=torch.int32, device="cuda"),
             "cnt": torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda"),
             "pidx": torch.full((wl.n_q, k), 77, dtype=torch.int32, device="cuda"),
             "pcnt": torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda"),
             "blk": torch.full((wl.n_q, 64), 77, dtype=torch.int32, device="cuda"),
             "bcnt": torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda")}
        C.csa2_index_segments(st.qi_codes, st.qi_scales, w, *ik, q_seq, n_vis_t, k, o["keys"], append=append)
        C.csa2_index_topk(st.qi_codes, st.qi_scales, w, *ik, q_seq, n_vis_t, k, o["idx"], o["cnt"], append=append)
        C.csa2_index_topk_pool(st.qi_codes, st.qi_scales, w, *ik, q_seq, n_vis_t, k, o["pidx"], o["pcnt"], o["blk"],
                               o["bcnt"], 8, append=append)
        torch.cuda.synchronize()
        return o

    ref_c = case.gpu_caches()
    for qi, r in enumerate(rows):
        if r < 0:
            continue
        b = int(wl.q_seq[qi])
        C.csa2_quantize_kv(main[qi:qi + 1], C.FMT_NVFP4, ref_c.kv_codes[b, r:r + 1], ref_c.kv_scales[b, r:r + 1])
        C.csa2_quantize_kv(index[qi:qi + 1], C.FMT_MXFP4, ref_c.ik_codes[b, r:r + 1], ref_c.ik_scales[b, r:r + 1])
    ref = run(ref_c, None)
    got_c = case.gpu_caches()
    app = {"row": row_t, "main": main, "index": index, "kv_codes": got_c.kv_codes, "kv_scales": got_c.kv_scales}
    got = run(got_c, app)
    for name in ref:
        assert torch.equal(got[name], ref[name]), name
    for name in ("kv_codes", "kv_scales", "ik_codes", "ik_scales"):
        assert torch.equal(getattr(got_c, name), getattr(ref_c, name)), name
    # the appended rows differ from what the caches held before (the check is not vacuous)
    before = case.gpu_caches()
    for qi, r in enumerate(rows):
        b = int(wl.q_seq[qi])
        same = torch.equal(got_c.ik_codes[b, max(r, 0)], before.ik_codes[b, max(r, 0)])
        assert same == (r < 0), (qi, r)
    del before
    # indexer-K only (no main latents), and an unquantised Q on top: still the same results
    got2_c = case.gpu_caches()
    got2 = run(got2_c, {"row": row_t, "index": index})
    for name in ref:
        assert torch.equal(got2[name], ref[name]), name
    assert torch.equal(got2_c.ik_codes, ref_c.ik_codes) and torch.equal(got2_c.ik_scales, ref_c.ik_scales)
    keys_q = torch.full_like(ref["keys"], 77)
    C.csa2_index_segments(q_idx, None, w, got2_c.ik_codes, got2_c.ik_scales, q_seq, n_vis_t, k, keys_q,
                          append={"row": row_t, "index": index})
    torch.cuda.synchronize()
    assert torch.equal(keys_q, ref["keys"])


def _run_index_topk(C, st, caches, w, q_seq, n_vis, k, in_pool=False):
    """(fused idx, count), (two-call idx, count) on the same inputs."""
    idx_f = torch.full((st.n_q, k), 77, dtype=torch.int32, device="cuda")
    cnt_f = torch.full((st.n_q,), 77, dtype=torch.int32, device="cuda")
    pool = (st.pool, st.pool_count) if in_pool else (None, None)
    C.csa2_index_topk(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis, k, idx_f, cnt_f,
                      None, pool[0], pool[1], 8, fmt=st.idx_qfmt)
    idx_u = torch.empty(st.n_q, k, dtype=torch.int32, device="cuda")
    cnt_u = torch.empty(st.n_q, dtype=torch.int32, device="cuda")
    st.score(caches, w, q_seq, n_vis, in_pool)
    C.csa2_topk(st.scores, n_vis, st.seq_cap, k, idx_u, cnt_u, None, pool[0], pool[1], 8)
    torch.cuda.synchronize()
    return (idx_f.cpu().numpy(), cnt_f.cpu().numpy()), (idx_u.cpu().numpy(), cnt_u.cpu().numpy())


@pytest.mark.parametrize("k,fmt", [(512, "mxfp4"), (2048, "mxfp4"), (7, "mxfp4"), (512, "nvfp4"), (7, "nvfp4")])
def test_index_topk_fused(C, k, fmt):
    """Fused scoring + selection returns exactly what scoring then selecting returns (the same
    fp32 scores, the same exact ranking), and that set passes the oracle's Top-K rule."""
    _say("index_topk", k, fmt)
    n_vis = [40000, 8193, 1, 0, 511, 20001, 16384]
    case = _score_case(30 + k, 3, 40000, n_vis, 16, fmt)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis_t, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, k=k, index_fmt=fmt)
    st.quantize_index_q(q_idx)
    (gi, gc), (ui, uc) = _run_index_topk(C, st, caches, w, q_seq, n_vis_t, k)
    assert np.array_equal(gc, uc) and np.array_equal(gi, ui)
    for qi in (0, 1, 2, 3, 4):
        nv = int(wl.n_vis[qi])
        if nv == 0:
            assert gc[qi] == 0 and np.all(gi[qi] == -1)
            continue
        seq = int(wl.q_seq[qi])
        qc, qs, wq, _ = case.oracle_query(0, qi)
        pos, ref = O.full_scores(qc, qs, wq, case.oracle_caches(seq), nv)
        G.topk_accept(gi[qi], int(gc[qi]), pos, ref, k)


@pytest.mark.parametrize("k,fmt,window", [(512, "mxfp4", 128), (7, "mxfp4", 128), (1500, "mxfp4", 128),
                                          (512, "nvfp4", 128), (512, "mxfp4", 256)])
def test_segments_then_attention_topk(C, k, fmt, window):
    """csa2_index_segments + csa2_sparse_attn_topk (the last Top-K level inside the attention
    call) give the index set of csa2_index_topk bit for bit, and attention outputs identical
    to csa2_sparse_attn over that set; repeated calls change nothing.  7 queries of 16 heads
    split their key lists over 10 workgroups, each of which selects.  A 256-key window runs
    the split-channel attention kernel, 128 keys the full-channel one."""
    _say("segments + attention topk", k, fmt, window)
    n_vis = [40000, 8193, 1, 0, 511, 20001, 16384]
    case = _score_case(50 + k, 3, 40000, n_vis, 16, fmt, swa_cap=window)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, qa = case.gpu_query_inputs(0)
    q_seq, n_vis_t, q_pos, rs = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, k=k, index_fmt=fmt, attn_select=True)
    assert st.attn_select
    st.quantize_index_q(q_idx)
    (gi, gc), _ = _run_index_topk(C, st, caches, w, q_seq, n_vis_t, k)
    sm = 1.0 / math.sqrt(512)
    out_a = torch.empty(wl.n_q, 16, 512, dtype=torch.float32, device="cuda")
    lse_a = torch.empty(wl.n_q, 16, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(gi).cuda(), caches.swa[0],
                       caches.swa_base, q_pos, rs, window, sm, out_a, lse_a)
    for rep in range(2):
        keys = torch.full((wl.n_q, C.csa2_segment_keys(wl.seq_cap, k)), 5, dtype=torch.int64, device="cuda")
        C.csa2_index_segments(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis_t, k,
                              keys, fmt=st.idx_qfmt)
        idx_b = torch.full((wl.n_q, k), 77, dtype=torch.int32, device="cuda")
        cnt_b = torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda")
        out_b = torch.empty_like(out_a)
        lse_b = torch.empty_like(lse_a)
        C.csa2_sparse_attn_topk(qa, caches.kv_codes, caches.kv_scales, q_seq, keys, k, idx_b, cnt_b, caches.swa[0],
                                caches.swa_base, q_pos, rs, window, sm, out_b, lse_b)
        torch.cuda.synchronize()
        assert np.array_equal(idx_b.cpu().numpy(), gi) and np.array_equal(cnt_b.cpu().numpy(), gc), rep
        assert torch.equal(out_b, out_a) and torch.equal(lse_b, lse_a), rep


def test_index_topk_repeated_calls_share_workspace(C):
    """Back-to-back calls on one workspace, with pool calls (which lay the workspace out
    differently) in between, give identical results."""
    _say("index_topk repeated")
    case = _score_case(52, 2, 50000, [50000, 24577, 9000], 16)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis_t, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, max_blocks=64)
    st.quantize_index_q(q_idx)
    st.pool.copy_(torch.arange(64, dtype=torch.int32, device="cuda").repeat(wl.n_q, 1))
    st.pool_count.fill_(64)
    outs = []
    for rep in range(3):
        st.idx.fill_(99)
        st.index_topk(caches, w, q_seq, n_vis_t)
        outs.append(st.idx.clone())
        st.index_topk(caches, w, q_seq, n_vis_t, in_pool=True)   # the pool path shares the workspace
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    (gi, gc), (ui, uc) = _run_index_topk(C, st, caches, w, q_seq, n_vis_t, 512)
    assert np.array_equal(gi, ui) and np.array_equal(gc, uc) and np.array_equal(outs[0].cpu().numpy(), gi)


@pytest.mark.parametrize("block,max_blocks,k", [(8, 2048, 512), (4, 100, 64), (16, 300, 2048)])
def test_index_topk_with_pool_build(C, block, max_blocks, k):
    """Top-K and pool from one scoring pass equal csa2_index_score + csa2_topk +
    csa2_build_pool on the same inputs, exactly (ragged tails, blocks cut by n_vis, an
    empty query)."""
    _say("index_topk_pool", block, max_blocks, k)
    n_vis = [40000, 8193, 1, 0, 16385, 20001, 7]
    case = _score_case(60 + block, 3, 40000, n_vis, 16)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis_t, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, k=k, block=block, max_blocks=max_blocks)
    st.quantize_index_q(q_idx)
    idx_f = torch.full((wl.n_q, k), 77, dtype=torch.int32, device="cuda")
    cnt_f = torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda")
    blk_f = torch.full((wl.n_q, max_blocks), 77, dtype=torch.int32, device="cuda")
    bc_f = torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda")
    C.csa2_index_topk_pool(st.qi_codes, st.qi_scales, w, caches.ik_codes, caches.ik_scales, q_seq, n_vis_t, k, idx_f,
                           cnt_f, blk_f, bc_f, block)
    st.score(caches, w, q_seq, n_vis_t)
    idx_u = torch.empty(wl.n_q, k, dtype=torch.int32, device="cuda")
    cnt_u = torch.empty(wl.n_q, dtype=torch.int32, device="cuda")
    C.csa2_topk(st.scores, n_vis_t, st.seq_cap, k, idx_u, cnt_u)
    blk_u = torch.empty(wl.n_q, max_blocks, dtype=torch.int32, device="cuda")
    bc_u = torch.empty(wl.n_q, dtype=torch.int32, device="cuda")
    C.csa2_build_pool(st.scores, n_vis_t, st.seq_cap, blk_u, bc_u, block)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_u) and torch.equal(cnt_f, cnt_u)
    assert torch.equal(blk_f, blk_u) and torch.equal(bc_f, bc_u)
    for qi in (0, 4):
        nv = int(wl.n_vis[qi])
        qc, qs, wq, _ = case.oracle_query(0, qi)
        _, ref = O.full_scores(qc, qs, wq, case.oracle_caches(int(wl.q_seq[qi])), nv)
        bs = O.block_scores(ref, nv, block)
        G.topk_accept(blk_f[qi].cpu().numpy(), int(bc_f[qi]), np.arange(bs.size), bs, max_blocks)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_index_topk_fused_pool(C, fmt):
    _say("index_topk pool", fmt)
    case = _score_case(41, 2, 30000, [30000, 12000, 333], 16, fmt)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, _ = case.gpu_query_inputs(0)
    q_seq, n_vis_t, _, _ = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    mb = 2048
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, max_blocks=mb, index_fmt=fmt)
    rng = np.random.default_rng(9)
    blocks = np.full((wl.n_q, mb), -1, np.int32)
    ncb = np.array([2048, 1500, 45], np.int32)
    for qi in range(wl.n_q):
        nb = -(-int(wl.n_vis[qi]) // 8)
        blocks[qi, :ncb[qi]] = np.sort(rng.choice(nb + 10, size=ncb[qi], replace=False))
    blocks[0, 100] = -1
    st.pool.copy_(torch.from_numpy(blocks))
    st.pool_count.copy_(torch.from_numpy(ncb))
    st.quantize_index_q(q_idx)
    (gi, gc), (ui, uc) = _run_index_topk(C, st, caches, w, q_seq, n_vis_t, 512, in_pool=True)
    assert np.array_equal(gc, uc) and np.array_equal(gi, ui)
    for qi in range(wl.n_q):
        nv = int(wl.n_vis[qi])
        slots = np.arange(ncb[qi] * 8)
        b = blocks[qi, slots // 8]
        pos = b.astype(np.int64) * 8 + slots % 8
        pos = pos[(b >= 0) & (pos < nv)]
        qc, qs, wq, _ = case.oracle_query(0, qi)
        _, ref = O.full_scores(qc, qs, wq, case.oracle_caches(int(wl.q_seq[qi])), nv, cand=pos)
        G.topk_accept(gi[qi], int(gc[qi]), pos, ref, 512)


@pytest.mark.parametrize("k,mb,window", [(512, 2048, 128), (7, 2048, 128), (512, 300, 128), (512, 2048, 256)])
def test_pool_select_in_attention(C, k, mb, window):
    """csa2_sparse_attn_pool_topk (the Top-K selected inside the attention call from the
    pool's slot scores) returns csa2_topk's index set over the same scores and pool bit for
    bit, and attention outputs identical to csa2_sparse_attn over it; full pools, partial
    ones, invalid block ids, blocks past n_vis and an empty pool.  A 256-key window runs the
    split-channel attention kernel, 128 keys the full-channel one."""
    _say("pool select in attention", k, mb, window)
    case = _score_case(71 + k, 4, 30000, [30000, 12000, 333, 5000], 16, swa_cap=window)
    wl = case.wl
    caches = case.gpu_caches()
    q_idx, w, qa = case.gpu_query_inputs(0)
    q_seq, n_vis_t, q_pos, rs = case.gpu_meta()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(wl.n_q, 16, 16, wl.seq_cap, k=k, max_blocks=mb)
    assert st.pool_select
    rng = np.random.default_rng(k + mb)
    blocks = np.full((wl.n_q, mb), -1, np.int32)
    ncb = np.array([mb, min(mb * 3 // 4, 1500), 45, 0], np.int32)   # at most the blocks a query has (+10)
    for qi in range(wl.n_q):
        nb = -(-int(wl.n_vis[qi]) // 8)
        if ncb[qi]:
            blocks[qi, :ncb[qi]] = np.sort(rng.choice(nb + 10, size=ncb[qi], replace=False))
    blocks[0, 100] = -1
    st.pool.copy_(torch.from_numpy(blocks))
    st.pool_count.copy_(torch.from_numpy(ncb))
    st.quantize_index_q(q_idx)
    st.score(caches, w, q_seq, n_vis_t, in_pool=True)
    idx_a = torch.empty(wl.n_q, k, dtype=torch.int32, device="cuda")
    cnt_a = torch.empty(wl.n_q, dtype=torch.int32, device="cuda")
    C.csa2_topk(st.scores, n_vis_t, st.seq_cap, k, idx_a, cnt_a, None, st.pool, st.pool_count, 8)
    sm = 1.0 / math.sqrt(512)
    out_a = torch.empty(wl.n_q, 16, 512, dtype=torch.float32, device="cuda")
    lse_a = torch.empty(wl.n_q, 16, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, idx_a, caches.swa[0], caches.swa_base, q_pos, rs,
                       window, sm, out_a, lse_a)
    for rep in range(2):
        idx_b = torch.full((wl.n_q, k), 77, dtype=torch.int32, device="cuda")
        cnt_b = torch.full((wl.n_q,), 77, dtype=torch.int32, device="cuda")
        out_b = torch.empty_like(out_a)
        lse_b = torch.empty_like(lse_a)
        C.csa2_sparse_attn_pool_topk(qa, caches.kv_codes, caches.kv_scales, q_seq, st.scores, n_vis_t, st.pool,
                                     st.pool_count, 8, k, idx_b, cnt_b, caches.swa[0], caches.swa_base, q_pos, rs,
                                     window, sm, out_b, lse_b)
        torch.cuda.synchronize()
        assert torch.equal(idx_b, idx_a) and torch.equal(cnt_b, cnt_a), rep
        assert torch.equal(out_b, out_a) and torch.equal(lse_b, lse_a), rep
    assert cnt_a[3].item() == 0 and torch.all(idx_a[3] == -1)


@pytest.mark.parametrize("n,k", [(1, 512), (511, 512), (512, 512), (513, 512), (8192, 512), (8193, 512),
                                 (20000, 7), (70001, 512), (200000, 2048), (9000, 1), (300000, 512)])
def test_topk_exact_on_same_scores(C, n, k):
    """Selection is an integer decision: on identical fp32 scores the GPU set must equal the
    oracle's ranking (score desc, position asc) exactly, ties included."""
    _say("topk", n, k)
    rng = np.random.default_rng(n + k)
    n_q = 3
    sc = rng.normal(size=(n_q, n)).astype(np.float32)
    sc[1] = rng.integers(0, 50, size=n).astype(np.float32)     # heavy ties
    sc[2, : n // 2] = 1.0                                       # a tied plateau
    n_vis = np.array([n, max(1, n - 37), n], np.int64)
    idx = torch.empty(n_q, k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(n_q, dtype=torch.int32, device="cuda")
    C.csa2_topk(torch.from_numpy(sc).cuda(), torch.from_numpy(n_vis).cuda(), n, k, idx, cnt)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for qi in range(n_q):
        nv = int(n_vis[qi])
        ref = O.topk_positions(sc[qi, :nv].astype(np.float64), np.arange(nv), k)
        assert gc[qi] == min(k, nv)
        assert np.array_equal(gi[qi], ref.astype(np.int32))


def test_topk_pool_slots_exact(C):
    _say("topk pool slots")
    rng = np.random.default_rng(5)
    n_q, mb, k = 2, 2048, 512
    nv = np.array([100000, 7000], np.int64)
    blocks = np.full((n_q, mb), -1, np.int32)
    ncb = np.array([2048, 800], np.int32)
    for qi in range(n_q):
        nb = -(-int(nv[qi]) // 8)
        blocks[qi, :ncb[qi]] = np.sort(rng.choice(nb + 5, size=ncb[qi], replace=False))
    sc = rng.normal(size=(n_q, mb * 8)).astype(np.float32)
    idx = torch.empty(n_q, k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(n_q, dtype=torch.int32, device="cuda")
    C.csa2_topk(torch.from_numpy(sc).cuda(), torch.from_numpy(nv).cuda(), int(nv.max()), k, idx, cnt, None,
                torch.from_numpy(blocks).cuda(), torch.from_numpy(ncb).cuda(), 8)
    torch.cuda.synchronize()
    for qi in range(n_q):
        slots = np.arange(ncb[qi] * 8)
        b = blocks[qi, slots // 8]
        pos = b.astype(np.int64) * 8 + slots % 8
        ok = (b >= 0) & (pos < nv[qi])
        ref = O.topk_positions(sc[qi, slots[ok]].astype(np.float64), pos[ok], k)
        assert np.array_equal(idx[qi].cpu().numpy(), ref.astype(np.int32))


@pytest.mark.parametrize("n_vis,mb", [(1_000_003, 2048), (16384, 2048), (16385, 2048), (77, 4), (5000, 100)])
def test_build_pool_exact(C, n_vis, mb):
    _say("build_pool", n_vis, mb)
    rng = np.random.default_rng(n_vis)
    n_q = 2
    sc = rng.standard_t(3, size=(n_q, n_vis)).astype(np.float32)
    nv = np.array([n_vis, max(1, n_vis - 3)], np.int64)
    blk = torch.empty(n_q, mb, dtype=torch.int32, device="cuda")
    cnt = torch.empty(n_q, dtype=torch.int32, device="cuda")
    C.csa2_build_pool(torch.from_numpy(sc).cuda(), torch.from_numpy(nv).cuda(), n_vis, blk, cnt, 8)
    torch.cuda.synchronize()
    for qi in range(n_q):
        ref = O.build_pool(sc[qi].astype(np.float64), int(nv[qi]), 8, mb)
        assert np.array_equal(blk[qi].cpu().numpy(), ref.astype(np.int32))
        assert cnt[qi].item() == min(mb, -(-int(nv[qi]) // 8))


def _attn_case(seed, n_seq, seq_cap, heads, t_list, s_list, swa_cap=128):
    n_q = len(t_list)
    wl = G.workloads.Workload(
        name="attn", seed=seed, n_seq=n_seq, seq_cap=seq_cap, m=1, heads=heads, idx_heads=16,
        q_seq=np.array([i % n_seq for i in range(n_q)], np.int32), q_pos=np.array(t_list, np.int64),
        replay_start=np.array(s_list, np.int64), layers=("full",), new_entries=(0, 0), swa_cap=swa_cap)
    return G.Case(wl)


@pytest.mark.parametrize("heads,out_dt", [(64, "f32"), (16, "f32"), (80, "f32"), (64, "bf16")])
def test_sparse_attn_parity(C, heads, out_dt):
    _say("sparse_attn", heads, out_dt)
    t = [3000, 2999, 100, 5, 2500, 2000]
    s = [0, 2999 - 5, 0, 5, 2500 - 126, 0]
    case = _attn_case(7 + heads, len(t), 3001, heads, t, s)   # one sequence per query
    wl = case.wl
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    rng = np.random.default_rng(heads)
    k = 512
    idx = np.full((wl.n_q, k), -1, np.int32)
    counts = [512, 300, 0, 512, 17, 512]
    for qi in range(wl.n_q):
        idx[qi, :counts[qi]] = np.sort(rng.choice(3001, size=counts[qi], replace=False))
    idx[3, 10] = 3001            # out of range: skipped
    idx[5, 20] = -7              # negative: skipped
    dt = torch.float32 if out_dt == "f32" else torch.bfloat16
    out = torch.empty(wl.n_q, heads, 512, dtype=dt, device="cuda")
    lse = torch.empty(wl.n_q, heads, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(idx).cuda(), caches.swa[0],
                       caches.swa_base, q_pos, rs, 128, 1.0 / math.sqrt(512), out, lse)
    torch.cuda.synchronize()
    go, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    for qi in range(wl.n_q):
        seq = int(wl.q_seq[qi])
        oc = case.oracle_caches(seq)
        assert np.array_equal(caches.kv_codes[seq].cpu().numpy(), oc.kv_codes)
        assert np.array_equal(caches.swa[0][seq].cpu().numpy(), oc.swa[0][0])
        _, _, _, qa_np = case.oracle_query(0, qi)
        sel = idx[qi][(idx[qi] >= 0) & (idx[qi] < 3001)]
        ref, ref_lse = O.sparse_attention(qa_np, oc.main_rows(sel),
                                          oc.swa_rows(0, O.swa_positions(t[qi], s[qi], 128)), 1 / math.sqrt(512))
        if out_dt == "f32":
            G.attn_close(go[qi], ref, 2e-3)
        else:
            attn_close_bf16(go[qi], ref)
        assert np.abs(gl[qi] - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("k,window,n_q,heads", [(2048, 128, 8, 64), (2048, 128, 64, 16), (1500, 40, 64, 64),
                                                (777, 1, 3, 16), (2048, 256, 6, 16)])
def test_sparse_attn_large_k(C, k, window, n_q, heads):
    """Index lists longer than the decode's 512, up to the maximum k = 2048: long key streams
    (up to 17 tiles per stream without a split), key lists split into slices of many tiles,
    a k that is not a multiple of the 16-key tile, and the split-channel kernel (256-key
    window) at the maximum k; every row against the oracle."""
    _say("sparse_attn large k", k, window, n_q, heads)
    rng = np.random.default_rng(k + window + n_q)
    cap = 3001
    t = [int(x) for x in rng.integers(k, cap, size=n_q)]
    t[0] = cap - 1
    s = [0 if i % 2 == 0 else max(0, ti - window // 3) for i, ti in enumerate(t)]
    case = _attn_case(5 + k + n_q, n_q, cap, heads, t, s, swa_cap=256)   # one sequence per query
    wl = case.wl
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    idx = np.full((n_q, k), -1, np.int32)
    counts = [k if i % 3 == 0 else int(rng.integers(1, k + 1)) for i in range(n_q)]
    for qi in range(n_q):
        idx[qi, :counts[qi]] = np.sort(rng.choice(t[qi] + 1, size=counts[qi], replace=False))
    need = C.csa2_attn_workspace_bytes(n_q, heads, 512, k, window)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(n_q, heads, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(idx).cuda(), caches.swa[0],
                       caches.swa_base, q_pos, rs, window, 1.0 / math.sqrt(512), out, lse, workspace=ws)
    torch.cuda.synchronize()
    assert C.csa2_device_status() == 0
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    for qi in range(n_q):
        oc = case.oracle_caches(int(wl.q_seq[qi]))
        _, _, _, qa_np = case.oracle_query(0, qi)
        ref, ref_lse = O.sparse_attention(qa_np, oc.main_rows(idx[qi, :counts[qi]]),
                                          oc.swa_rows(0, O.swa_positions(t[qi], s[qi], window)), 1 / math.sqrt(512))
        G.attn_close(go[qi], ref, 2e-3)
        assert np.abs(gl[qi] - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("window,n_q,heads", [(1, 64, 64), (40, 64, 64), (200, 64, 64), (40, 6, 16), (200, 6, 16)])
def test_sparse_attn_window_sizes(C, window, n_q, heads):
    """Windows other than 128 keys: a single key, a ragged number of tiles too few for the
    early window gathers, and more than 128 keys (ring of 256 rows); 64 queries x 64 heads run
    without a key split, 6 queries x 16 heads split the key list over workgroups."""
    _say("sparse_attn window", window, n_q, heads)
    rng = np.random.default_rng(window * 100 + n_q)
    t = [int(x) for x in rng.integers(0, 1200, size=n_q)]
    t[0] = 1199
    s = []
    for i, ti in enumerate(t):   # no replay, a replay start inside the window, a start at t
        s.append(0 if i % 3 == 0 else (max(0, ti - window // 2) if i % 3 == 1 else ti))
    case = _attn_case(11 + window, n_q, 1200, heads, t, s, swa_cap=256)   # one sequence per query
    wl = case.wl
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    k = 512
    idx = np.full((n_q, k), -1, np.int32)
    counts = [int(c) for c in rng.integers(0, k + 1, size=n_q)]
    counts[0] = k
    for qi in range(n_q):
        idx[qi, :counts[qi]] = np.sort(rng.choice(1200, size=counts[qi], replace=False))
    out = torch.empty(n_q, heads, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(idx).cuda(), caches.swa[0],
                       caches.swa_base, q_pos, rs, window, 1.0 / math.sqrt(512), out, lse)
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    for qi in range(n_q):
        oc = case.oracle_caches(int(wl.q_seq[qi]))
        _, _, _, qa_np = case.oracle_query(0, qi)
        ref, ref_lse = O.sparse_attention(qa_np, oc.main_rows(idx[qi, :counts[qi]]),
                                          oc.swa_rows(0, O.swa_positions(t[qi], s[qi], window)), 1 / math.sqrt(512))
        G.attn_close(go[qi], ref, 2e-3)
        assert np.abs(gl[qi] - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("n_q", [6, 24])
def test_sparse_attn_split_workspace_reuse(C, n_q):
    """Split key lists (5 splits at 6 queries, 2 at 24): consecutive calls on one
    workspace give bit-identical outputs and match the oracle."""
    _say("sparse_attn split reuse", n_q)
    heads = 64
    t = [2000 - 37 * i for i in range(n_q)]
    s = [0] * n_q
    case = _attn_case(11 + n_q, n_q, 2001, heads, t, s)
    wl = case.wl
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    rng = np.random.default_rng(n_q)
    idx = np.stack([np.sort(rng.choice(t[i] + 1, size=512, replace=False)) for i in range(n_q)]).astype(np.int32)
    need = C.csa2_attn_workspace_bytes(n_q, heads, 512, 512, 128)
    assert need > 0                                  # the key list is split at these sizes
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        out = torch.empty(n_q, heads, 512, dtype=torch.float32, device="cuda")
        lse = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
        C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(idx).cuda(), caches.swa[0],
                           caches.swa_base, q_pos, rs, 128, 1.0 / math.sqrt(512), out, lse, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    go, gl = outs[0][0].numpy(), outs[0][1].numpy()
    for qi in (0, n_q - 1):
        seq = int(wl.q_seq[qi])
        oc = case.oracle_caches(seq)
        _, _, _, qa_np = case.oracle_query(0, qi)
        ref, ref_lse = O.sparse_attention(qa_np, oc.main_rows(idx[qi]),
                                          oc.swa_rows(0, O.swa_positions(t[qi], s[qi], 128)), 1 / math.sqrt(512))
        G.attn_close(go[qi], ref, 2e-3)
        assert np.abs(gl[qi] - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("select,dt", [(False, "f32"), (False, "bf16"), (True, "f32")])
def test_window_append_in_attention(C, select, dt):
    """Attention with new_win (the row's own window entry appended by the attention call)
    writes the ring row csa2_quantize_kv writes and gives bit-identical outputs to appending
    first and attending after; rows of distinct sequences, one with a replay start at t."""
    _say("window append in attention", select, dt)
    n_vis = [30000, 8193, 511, 20001, 16384, 3]
    n_q = len(n_vis)
    case = _score_case(61, n_q, 30000, n_vis, 16)           # one sequence per row
    wl = case.wl
    wl.replay_start[3] = wl.q_pos[3]                          # window = its own token only
    caches = case.gpu_caches()
    q_idx, w, qa = case.gpu_query_inputs(0)
    q_seq, n_vis_t, q_pos, rs = case.gpu_meta()
    rs = torch.from_numpy(wl.replay_start.astype(np.int64)).cuda()
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    st = Csa2Step(n_q, 16, 16, wl.seq_cap, attn_select=select)
    st.quantize_index_q(q_idx)
    if select:
        st.index_segments(caches, w, q_seq, n_vis_t)
    else:
        st.index_topk(caches, w, q_seq, n_vis_t)
    lat = np.stack([wl.swa_latents(0, int(wl.q_seq[i]), int(wl.q_pos[i]), 1)[0] for i in range(n_q)])
    new = torch.from_numpy(lat).cuda()
    if dt == "bf16":
        new = new.to(torch.bfloat16)
    rows = torch.from_numpy(((wl.q_pos - wl.swa_base) % wl.swa_cap).astype(np.int64)).cuda()
    flat_rows = torch.arange(n_q, device="cuda", dtype=torch.int64) * wl.swa_cap + rows
    ring = caches.swa[0].view(-1, 512)

    def attend(new_win):
        out = torch.empty(n_q, 16, 512, dtype=torch.float32, device="cuda")
        lse = torch.empty(n_q, 16, dtype=torch.float32, device="cuda")
        if select:
            st.attend_topk(caches, 0, qa, q_seq, q_pos, rs, out, lse, new_win=new_win)
        else:
            st.attend(caches, 0, qa, q_seq, q_pos, rs, out, lse, new_win=new_win)
        torch.cuda.synchronize()
        return out, lse

    C.csa2_quantize_kv(new, C.FMT_FP8, ring, None, flat_rows)     # append, then attend
    ref_rows = ring[flat_rows].clone()
    out_r, lse_r = attend(None)
    ring[flat_rows] = 0x55                                        # stale bytes in the rows
    out_f, lse_f = attend(new)
    assert torch.equal(ring[flat_rows], ref_rows)
    assert torch.equal(out_f, out_r) and torch.equal(lse_f, lse_r)


def _bf16(x: np.ndarray) -> torch.Tensor:
    """float array -> bf16 device tensor (round to nearest even, as torch converts)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda().to(torch.bfloat16)


def _peaked_q(case, idx, counts, t, s, window, heads, rng):
    """Attention Q whose logits are far from the N(0,1) of plain seeded Q: per head, Q is a
    multiple of one key's post-RoPE latent (a main entry late in the index list, or a window
    key), a scaled-up random vector, or plain N(0,1).  Then a later tile's logit exceeds the
    running reference by much more than the kernel's lazy-rescale headroom, and the key
    splits of a row end with widely separated maxima."""
    wl = case.wl
    n_q = len(t)
    q = rng.standard_normal((n_q, heads, 512)).astype(np.float32)
    for qi in range(n_q):
        seq = int(wl.q_seq[qi])
        win = O.swa_positions(t[qi], s[qi], window)
        for h in range(heads):
            kind = h % 4
            if kind == 0 and counts[qi] > 0:      # one main entry, late in the list
                j = int(idx[qi, max(0, counts[qi] - 1 - (h // 4) % 7 * 9)])
                q[qi, h] = 3.0 * wl.main_latents(seq, j, 1)[0]
            elif kind == 1 and win.size:          # one window key (its own token first)
                p = int(win[max(0, win.size - 1 - (h // 4) % 5 * 17)])
                lat = G.swa_ring_latents(wl, 0, seq)[(p - wl.swa_base) % wl.swa_cap]
                q[qi, h] = 0.5 * lat + 0.1 * q[qi, h]
            elif kind == 2:                       # broad but strongly peaked logits
                q[qi, h] *= 6.0
    return q


def _attn_ref(case, qi, q_np, sel, t, s, window, sm_scale):
    oc = case.oracle_caches(int(case.wl.q_seq[qi]))
    return O.sparse_attention(q_np.astype(np.float64), oc.main_rows(sel),
                              oc.swa_rows(0, O.swa_positions(t, s, window)), sm_scale)


attn_close_bf16 = G.attn_close_bf16


@pytest.mark.parametrize("n_q,heads,sm", [(64, 64, None), (6, 16, None), (64, 64, 0.5), (6, 16, 0.5)])
def test_sparse_attn_peaked_logits(C, n_q, heads, sm):
    """Peaked attention: Q aligned with single keys placed late in the main list or in the
    window, scaled-up random Q, or a large softmax scale (0.5 instead of 1/sqrt(512)) on
    plain Q.  Later tiles beat the running reference by far more than the lazy-rescale
    headroom (the accumulator rescale runs), and at 6 queries x 16 heads the key splits end
    with widely separated maxima (the split merge runs).  fp32 and bf16 outputs; the bf16
    output within the fp32 bar plus one bf16 ulp per element."""
    _say("sparse_attn peaked", n_q, heads, sm)
    rng = np.random.default_rng(1000 + n_q + heads)
    t = [int(x) for x in rng.integers(600, 3000, size=n_q)]
    s = [0 if i % 2 == 0 else max(0, ti - 60) for i, ti in enumerate(t)]
    case = _attn_case(31 + n_q, n_q, 3001, heads, t, s)
    wl = case.wl
    caches = case.gpu_caches()
    q_seq, _, q_pos, rs = case.gpu_meta()
    k = 512
    counts = [k if i % 3 else int(rng.integers(100, k)) for i in range(n_q)]
    idx = np.full((n_q, k), -1, np.int32)
    for qi in range(n_q):
        idx[qi, :counts[qi]] = np.sort(rng.choice(t[qi] + 1, size=counts[qi], replace=False))
    if sm is None:
        sm_scale = 1.0 / math.sqrt(512)
        q_np = _peaked_q(case, idx, counts, t, s, 128, heads, rng)
    else:
        sm_scale = sm
        q_np = rng.standard_normal((n_q, heads, 512)).astype(np.float32)
    qa = _bf16(q_np)
    q_exact = qa.float().cpu().numpy()
    idx_t = torch.from_numpy(idx).cuda()
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty(n_q, heads, 512, dtype=dt, device="cuda")
        lse = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
        C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, idx_t, caches.swa[0], caches.swa_base,
                           q_pos, rs, 128, sm_scale, out, lse)
        torch.cuda.synchronize()
        outs[dt] = (out.float().cpu().numpy(), lse.cpu().numpy())
    assert C.csa2_device_status() == 0
    peaked = 0
    for qi in range(n_q):
        oc = case.oracle_caches(int(wl.q_seq[qi]))
        keys = np.concatenate([oc.main_rows(idx[qi, :counts[qi]]),
                               oc.swa_rows(0, O.swa_positions(t[qi], s[qi], 128))])
        logit2 = sm_scale * (q_exact[qi].astype(np.float64) @ keys.T) / math.log(2.0)
        peaked += int((logit2.max(axis=1) - np.median(logit2, axis=1) > 8.0).sum())
        ref, ref_lse = _attn_ref(case, qi, q_exact[qi], idx[qi, :counts[qi]], t[qi], s[qi], 128, sm_scale)
        G.attn_close(outs[torch.float32][0][qi], ref, 2e-3)
        attn_close_bf16(outs[torch.bfloat16][0][qi], ref)
        assert np.abs(outs[torch.float32][1][qi] - ref_lse).max() <= 1e-3
        assert np.array_equal(outs[torch.bfloat16][1][qi], outs[torch.float32][1][qi])
    # the inputs are what the test is for: most heads' largest logit stands more than the
    # lazy-rescale headroom (2^8) above the typical one
    assert peaked >= n_q * heads // 2, (peaked, n_q * heads)


@pytest.mark.parametrize("mag", [1e6, 1e30, 1e-12, 1e-30])
def test_sparse_attn_bf16_q_full_range(C, mag):
    """Q far outside fp16's range (|q| up to ~1e31) or deep in its subnormals (~1e-31), with
    the softmax scale compensating so the logits are ordinary: the per-head power-of-two
    scale keeps every Q value exact, so the result matches the oracle as for unit Q.  Also
    a head of zeros (uniform weights) and, in one row, heads of very different magnitudes."""
    _say("sparse_attn bf16 Q range", mag)
    rng = np.random.default_rng(int(abs(math.log10(mag))))
    n_q, heads = 6, 32
    t = [2000 - 111 * i for i in range(n_q)]
    s = [0] * n_q
    case = _attn_case(77, n_q, 2001, heads, t, s)
    caches = case.gpu_caches()
    q_seq, _, q_pos, rs = case.gpu_meta()
    idx = np.stack([np.sort(rng.choice(t[i] + 1, size=512, replace=False)) for i in range(n_q)]).astype(np.int32)
    q_np = rng.standard_normal((n_q, heads, 512)) * mag
    q_np[0, 3] = 0.0                                    # an all-zero head
    q_np[1, 5] *= 1e-3                                  # heads of another magnitude in the row
    q_np[1, 6] *= 1e3
    sm_scale = 1.0 / (math.sqrt(512) * mag)
    qa = _bf16(q_np)
    q_exact = qa.float().cpu().numpy()
    out = torch.empty(n_q, heads, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(idx).cuda(), caches.swa[0],
                       caches.swa_base, q_pos, rs, 128, sm_scale, out, lse)
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    for qi in range(n_q):
        ref, ref_lse = _attn_ref(case, qi, q_exact[qi], idx[qi], t[qi], s[qi], 128, sm_scale)
        G.attn_close(go[qi], ref, 2e-3)
        assert np.abs(gl[qi] - ref_lse).max() <= 1e-3 * max(1.0, np.abs(ref_lse).max() * 1e-4)


def test_device_status_reports_an_expired_wait(C):
    """The status path of the attention's bounded partner wait, forced from the host: with
    a wait bound of 0 polls every exchange gives up at once (the kernel still completes, with
    a wrong output); the kernel stores its code into the device status word, the next call
    returns CSA2_ERR_DEVICE without launching and names the cause, and once the bound is
    restored the same call is correct again.  The window is 256 keys: only the split-channel
    kernel, which a window wider than 128 keys selects, has such a wait."""
    _say("device status")
    t, s = [1500, 1400], [0, 0]
    case = _attn_case(5, 2, 1501, 16, t, s, swa_cap=256)
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(1401, size=512, replace=False)) for _ in range(2)]).astype(np.int32)
    idx_t = torch.from_numpy(idx).cuda()
    out = torch.empty(2, 16, 512, dtype=torch.float32, device="cuda")
    lse = torch.empty(2, 16, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(C.csa2_attn_workspace_bytes(2, 16, 512, 512, 256), 1), dtype=torch.uint8, device="cuda")

    def attend():
        C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, idx_t, caches.swa[0], caches.swa_base, q_pos,
                           rs, 256, 1.0 / math.sqrt(512), out, lse, workspace=ws)
        torch.cuda.synchronize()

    C.csa2_device_status(clear=True)
    prev = C.csa2_debug_set_wait_limit(0)
    try:
        attend()
    finally:
        C.csa2_debug_set_wait_limit(prev)
    assert C.csa2_device_status() == 1                   # CSA2_STATUS_ATTN_WAIT
    with pytest.raises(C.Csa2Error, match=r"\(-6\).*partner"):
        attend()
    assert C.csa2_device_status() == 0                   # reported once, then cleared
    attend()
    assert C.csa2_device_status() == 0
    for qi in range(2):
        _, _, _, qa_np = case.oracle_query(0, qi)
        ref, ref_lse = _attn_ref(case, qi, qa_np, idx[qi], t[qi], s[qi], 256, 1.0 / math.sqrt(512))
        G.attn_close(out[qi].cpu().numpy(), ref, 2e-3)


def test_binding_refuses_unsafe_calls(C):
    """The binding's own checks: a bound call that would need a temporary workspace is
    refused (the callable would keep a pointer to freed memory), and a window append whose
    rows share a sequence is refused (its ring writes would race with the other rows' reads)."""
    _say("binding checks")
    t, s = [900, 800, 700], [0, 0, 0]
    case = _attn_case(9, 3, 901, 16, t, s)
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    idx = torch.full((3, 512), -1, dtype=torch.int32, device="cuda")
    out = torch.empty(3, 16, 512, dtype=torch.float32, device="cuda")
    assert C.csa2_attn_workspace_bytes(3, 16, 512, 512, 128) > 0
    with pytest.raises(ValueError, match="bound call needs a caller-owned workspace"):
        C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, idx, caches.swa[0], caches.swa_base, q_pos,
                           rs, 128, 0.05, out, _bind=True)
    new = torch.zeros(3, 512, dtype=torch.float32, device="cuda")
    dup = torch.tensor([0, 1, 0], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="share a sequence"):
        C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, dup, idx, caches.swa[0], caches.swa_base, q_pos,
                           rs, 128, 0.05, out, new_win=new)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("window,k,out_dt,peaked", [(128, 512, "f32", False), (128, 512, "bf16", True),
                                                    (40, 100, "f32", False), (1, 512, "f32", False),
                                                    (200, 512, "f32", True)])
def test_sparse_attn_many_rows(C, window, k, out_dt, peaked):
    """A batch of 1,100 rows with 64 heads and a given index list (the size of a prefill
    chunk's batch: one workgroup per row, every head): every row against the oracle.  Rows
    of 4 sequences with ragged index sets (empty ones included), invalid indices, replay
    starts inside and at the end of the window, windows of 1, 40, 128 and 200 keys (ring of
    256 rows), k not a multiple of the 32-key tile, and peaked logits (later tiles beat the
    lazy softmax reference by far more than its headroom)."""
    _say("sparse_attn many rows", window, k, out_dt, peaked)
    n_q, n_seq, cap, heads = 1100, 4, 2400, 64
    rng = np.random.default_rng(window * 7 + k)
    t = [int(x) for x in rng.integers(0, cap, size=n_q)]
    t[0] = cap - 1
    s = [0 if i % 3 == 0 else (max(0, ti - window // 2) if i % 3 == 1 else ti) for i, ti in enumerate(t)]
    case = _attn_case(50 + window, n_seq, cap, heads, t, s, swa_cap=256)
    wl = case.wl
    caches = case.gpu_caches()
    q_seq, _, q_pos, rs = case.gpu_meta()
    counts = [int(c) for c in rng.integers(0, k + 1, size=n_q)]
    counts[0], counts[1], counts[2] = k, 0, k
    idx = np.full((n_q, k), -1, np.int32)
    for qi in range(n_q):
        idx[qi, :counts[qi]] = np.sort(rng.choice(t[qi] + 1 if t[qi] + 1 >= counts[qi] else cap,
                                                  size=counts[qi], replace=False))
    idx[2, 5] = cap + 3          # out of range: skipped
    idx[2, 9] = -4               # negative: skipped
    sm_scale = 1.0 / math.sqrt(512)
    if peaked:
        q_np = _peaked_q(case, idx, counts, t, s, window, heads, rng)
    else:
        q_np = rng.standard_normal((n_q, heads, 512)).astype(np.float32)
    qa = _bf16(q_np)
    q_exact = qa.float().cpu().numpy()
    dt = torch.float32 if out_dt == "f32" else torch.bfloat16
    out = torch.empty(n_q, heads, 512, dtype=dt, device="cuda")
    lse = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
    assert C.csa2_attn_workspace_bytes(n_q, heads, 512, k, window) == 0
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, torch.from_numpy(idx).cuda(), caches.swa[0],
                       caches.swa_base, q_pos, rs, window, sm_scale, out, lse)
    torch.cuda.synchronize()
    assert C.csa2_device_status() == 0
    go, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    ocs = {b: case.oracle_caches(b) for b in range(n_seq)}
    for qi in range(n_q):
        oc = ocs[int(wl.q_seq[qi])]
        sel = idx[qi, :counts[qi]]
        sel = sel[(sel >= 0) & (sel < cap)]
        ref, ref_lse = O.sparse_attention(q_exact[qi].astype(np.float64), oc.main_rows(sel),
                                          oc.swa_rows(0, O.swa_positions(t[qi], s[qi], window)), sm_scale)
        if out_dt == "f32":
            G.attn_close(go[qi], ref, 2e-3)
        else:
            attn_close_bf16(go[qi], ref)
        finite = np.isfinite(ref_lse)
        assert np.array_equal(finite, np.isfinite(gl[qi])), qi
        assert np.abs(gl[qi][finite] - ref_lse[finite]).max(initial=0.0) <= 1e-3, qi


def test_sparse_attn_no_keys(C):
    """s > t leaves the window empty; with no main entries the output is 0 and lse -inf."""
    _say("sparse_attn no keys")
    case = _attn_case(3, 1, 100, 16, [50, 60], [51, 0])
    caches = case.gpu_caches()
    _, _, qa = case.gpu_query_inputs(0)
    q_seq, _, q_pos, rs = case.gpu_meta()
    idx = torch.full((2, 4), -1, dtype=torch.int32, device="cuda")
    out = torch.full((2, 16, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.empty(2, 16, dtype=torch.float32, device="cuda")
    C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, idx, caches.swa[0], caches.swa_base, q_pos, rs,
                       128, 0.05, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isfinite(lse[1]))


def test_smoke_tiny_decode(C):
    _say("smoke c1")
    res = G.smoke_check()
    assert res["attn_err"] < 2e-3

"""Pins of the oracle's indexer scoring, Top-K and candidate pool (no GPU)."""
import itertools
from fractions import Fraction

import numpy as np

from oracle import csa2_oracle as O


def _rand_mx(rng, rows, d, spread=4):
    x = (rng.normal(size=(rows, d)) * 2.0 ** rng.integers(-spread, spread, size=(rows, 1))).astype(np.float32)
    return O.quantize_mxfp4(x)


def _dot_exact(qc, qs, kc, ks):
    """q . k of two MXFP4 vectors with integer arithmetic: every E2M1 value is an integer
    multiple of 1/2, so each 32-block contributes 2^(Eq+Ek) * (sum of integer products)/4."""
    qn, kn = O.unpack_nibbles(qc), O.unpack_nibbles(kc)
    half = [0, 1, 2, 3, 4, 6, 8, 12]          # E2M1 magnitude in units of 1/2
    total = Fraction(0)
    for b in range(len(qs)):
        acc = 0
        for i in range(32 * b, 32 * b + 32):
            a = half[qn[i] & 7] * (-1 if qn[i] & 8 else 1)
            c = half[kn[i] & 7] * (-1 if kn[i] & 8 else 1)
            acc += a * c
        total += Fraction(acc, 4) * Fraction(2) ** (int(qs[b]) - 127) * Fraction(2) ** (int(ks[b]) - 127)
    return total


def test_single_head_unit_weight_is_relu_dot():
    rng = np.random.default_rng(1)
    qc, qs = _rand_mx(rng, 1, 128)
    kc, ks = _rand_mx(rng, 40, 128)
    sc = O.index_scores(O.dequant_mxfp4(qc, qs), np.ones(1), O.dequant_mxfp4(kc, ks))
    for j in range(40):
        d = _dot_exact(qc[0], qs[0], kc[j], ks[j])
        assert sc[j] == float(max(d, 0))       # exact: FP4 products sum exactly in fp64
    assert (sc == 0).any() and (sc > 0).any()  # both ReLU branches exercised


def test_scores_bruteforce_loops_multihead():
    rng = np.random.default_rng(2)
    H, n, d = 5, 23, 128
    qc, qs = _rand_mx(rng, H, d)
    kc, ks = _rand_mx(rng, n, d)
    w = rng.uniform(size=H)
    qd, kd = O.dequant_mxfp4(qc, qs), O.dequant_mxfp4(kc, ks)
    got = O.index_scores(qd, w, kd)
    for j in range(n):
        ref = 0.0
        for h in range(H):
            dot = float(_dot_exact(qc[h], qs[h], kc[j], ks[j]))
            ref += w[h] * (dot if dot > 0 else 0.0)
        assert abs(got[j] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_score_weight_selects_head():
    rng = np.random.default_rng(3)
    H = 4
    qc, qs = _rand_mx(rng, H, 128)
    kc, ks = _rand_mx(rng, 30, 128)
    qd, kd = O.dequant_mxfp4(qc, qs), O.dequant_mxfp4(kc, ks)
    for h in range(H):
        w = np.zeros(H)
        w[h] = 2.5
        got = O.index_scores(qd, w, kd)
        ref = [2.5 * max(float(_dot_exact(qc[h], qs[h], kc[j], ks[j])), 0.0) for j in range(30)]
        assert np.array_equal(got, np.array(ref))


def _topk_brute(scores, positions, k):
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], positions[i]))
    sel = sorted(positions[i] for i in order[:k])
    return sel + [-1] * (k - len(sel))


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(4)
    for n, k in [(1, 4), (3, 4), (50, 8), (200, 17), (1000, 64)]:
        sc = rng.integers(0, 6, size=n).astype(np.float64)      # many ties
        pos = np.arange(n) * 3 + 5
        assert list(O.topk_positions(sc, pos, k)) == _topk_brute(list(sc), list(pos), k)


def test_topk_all_when_few_candidates_and_order_invariant():
    rng = np.random.default_rng(5)
    sc = rng.normal(size=300)
    pos = np.arange(300)
    got = O.topk_positions(sc, pos, 512)
    assert list(got[:300]) == list(range(300)) and np.all(got[300:] == -1)
    got = O.topk_positions(sc, pos, 40)
    sel = got[got >= 0]
    rest = np.setdiff1d(pos, sel)
    assert sc[sel].min() >= sc[rest].max()
    perm = rng.permutation(300)
    assert np.array_equal(O.topk_positions(sc[perm], pos[perm], 40), got)


def test_block_scores_ragged_tail_ignores_invisible():
    sc = np.array([1, 2, 3, 4, 5, 6, 7, 8, 0.5, 0.25, 99, 99, 99], dtype=np.float64)
    bs = O.block_scores(sc, 10, 8)           # positions 10.. are not visible
    assert list(bs) == [8.0, 0.5]


def test_pool_bruteforce_small():
    rng = np.random.default_rng(6)
    n_vis, block, max_blocks = 77, 8, 4
    sc = rng.normal(size=n_vis)
    bmax = [max(sc[b * block:min(b * block + block, n_vis)]) for b in range((n_vis + block - 1) // block)]
    ref = sorted(sorted(range(len(bmax)), key=lambda b: (-bmax[b], b))[:max_blocks])
    assert list(O.build_pool(sc, n_vis, block, max_blocks)) == ref


def test_pool_covers_everything_when_small():
    # pool capacity 2,048 x 8 = 16,384 positions: any context that fits is kept whole
    rng = np.random.default_rng(7)
    for n_vis in (1, 8, 9, 16383, 16384):
        sc = rng.normal(size=n_vis)
        pool = O.build_pool(sc, n_vis, 8, 2048)
        nb = -(-n_vis // 8)
        assert list(pool[:nb]) == list(range(nb)) and np.all(pool[nb:] == -1)
        assert np.array_equal(O.pool_positions(pool, n_vis, 8), np.arange(n_vis))


def test_pool_contains_full_layer_topk():
    # a block whose max beats the 512th score holds a top-511 entry, so at most 512 such
    # blocks exist: the Full layer's Top-512 always lies inside a 2,048-block pool
    rng = np.random.default_rng(8)
    n_vis = 100_003
    sc = rng.standard_t(3, size=n_vis)
    idx = O.topk_positions(sc, np.arange(n_vis), 512)
    pool = O.build_pool(sc, n_vis, 8, 2048)
    assert np.isin(idx, O.pool_positions(pool, n_vis, 8)).all()
    assert (pool >= 0).sum() == 2048


def test_visible_entries():
    assert [O.visible_entries(t, 2) for t in range(6)] == [0, 1, 1, 2, 2, 3]
    assert [O.visible_entries(t, 1) for t in range(3)] == [1, 2, 3]
    for t, m in itertools.product(range(40), (1, 2, 4)):
        n = O.visible_entries(t, m)
        assert n * m <= t + 1 < (n + 1) * m

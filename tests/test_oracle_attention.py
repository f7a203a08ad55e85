"""Pins of the oracle's sliding window, sparse attention and layer modes (no GPU)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import csa2_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_attention_cases():
    with open(os.path.join(GOLD, "hand_attention.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out, lse = O.attention(np.array(c["q"]), np.array(c["keys"]), c["sm_scale"])
        assert np.allclose(out, c["out"], rtol=0, atol=1e-15), c["why"]
        assert np.allclose(lse, c["lse"], rtol=0, atol=1e-15), c["why"]


def _attention_loops(q, keys, sm_scale):
    H, D = q.shape
    out = np.zeros((H, D))
    lse = np.zeros(H)
    for h in range(H):
        logits = [sm_scale * sum(q[h, c] * k[c] for c in range(D)) for k in keys]
        m = max(logits)
        ws = [math.exp(l - m) for l in logits]
        z = math.fsum(ws)
        for c in range(D):
            out[h, c] = math.fsum(w * k[c] for w, k in zip(ws, keys)) / z
        lse[h] = m + math.log(z)
    return out, lse


def test_attention_bruteforce_loops():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(3, 6))
    keys = rng.normal(size=(9, 6)) * 3
    out, lse = O.attention(q, keys, 0.7)
    ro, rl = _attention_loops(q, keys, 0.7)
    assert np.allclose(out, ro, rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_lse_merge_identity():
    # attention over S1 u S2 equals the LSE-weighted merge of the two partial results
    rng = np.random.default_rng(2)
    q = rng.normal(size=(4, 8))
    k1, k2 = rng.normal(size=(5, 8)), rng.normal(size=(7, 8)) * 2
    o, l = O.attention(q, np.concatenate([k1, k2]), 0.5)
    o1, l1 = O.attention(q, k1, 0.5)
    o2, l2 = O.attention(q, k2, 0.5)
    L = np.logaddexp(l1, l2)
    merged = o1 * np.exp(l1 - L)[:, None] + o2 * np.exp(l2 - L)[:, None]
    assert np.allclose(L, l, atol=1e-13) and np.allclose(merged, o, atol=1e-13)


def test_zero_scale_gives_key_mean():
    rng = np.random.default_rng(3)
    keys = rng.normal(size=(11, 5))
    out, lse = O.attention(rng.normal(size=(2, 5)), keys, 0.0)
    assert np.allclose(out, keys.mean(0)[None, :], atol=1e-14)
    assert np.allclose(lse, math.log(11))


def test_swa_bounded_replay_window():
    W = 128
    for t in range(0, 400, 7):
        for s in (0, max(0, t - 5), t, max(0, t - 126), max(0, t - 300)):
            p = O.swa_positions(t, s, W)
            assert p[-1] == t and p[0] == max(s, t - W + 1)
            assert len(p) == min(W, t - s + 1)
            assert np.all(np.diff(p) == 1)
    # s = 0 with a window at least t+1 long: the whole causal prefix
    assert list(O.swa_positions(9, 0, 16)) == list(range(10))


def _tiny_caches(rng, n, layer_ids=(0, 1), cap=16, base=0, D=512, d=128):
    kv = O.quantize_nvfp4(rng.normal(size=(n, D)).astype(np.float32))
    ik = O.quantize_mxfp4(rng.normal(size=(n, d)).astype(np.float32))
    swa = {L: (O.quantize_fp8(rng.normal(size=(cap, D)).astype(np.float32)), base, cap) for L in layer_ids}
    return O.PackedCaches(kv[0], kv[1], ik[0], ik[1], swa)


def test_topk_over_few_entries_equals_dense_attention():
    # with no more visible entries than K, Top-K keeps them all and the sparse layer is
    # dense attention over all entries plus the window
    rng = np.random.default_rng(4)
    n, t, s, W = 37, 36, 30, 16
    caches = _tiny_caches(rng, n, cap=16)
    qc, qs = O.quantize_mxfp4(rng.normal(size=(4, 128)).astype(np.float32))
    q = rng.normal(size=(2, 512))
    res = O.layer_step("full", q_codes=qc, q_scales=qs, w=rng.uniform(size=4), caches=caches, layer=0,
                       q_attn=q, t=t, s=s, n_vis=n, k=64, window=W, sm_scale=0.05)
    assert list(res["idx"][:n]) == list(range(n))
    keys = np.concatenate([O.dequant_nvfp4(caches.kv_codes, caches.kv_scales),
                           O.dequant_fp8(caches.swa[0][0][np.arange(s, t + 1) % 16])])
    out, lse = O.attention(q, keys, 0.05)
    assert np.allclose(res["out"], out, atol=1e-13) and np.allclose(res["lse"], lse, atol=1e-13)


def test_reuse_equals_full_with_borrowed_indices_and_reindex_identity():
    rng = np.random.default_rng(5)
    n = 3000
    caches = _tiny_caches(rng, n)
    qc, qs = O.quantize_mxfp4(rng.normal(size=(8, 128)).astype(np.float32))
    w = rng.uniform(size=8)
    q = rng.normal(size=(2, 512))
    kw = dict(caches=caches, layer=0, q_attn=q, t=n - 1, s=0, n_vis=n, k=512, window=16, sm_scale=0.04)
    full = O.layer_step("full", q_codes=qc, q_scales=qs, w=w, build_pool_blocks=2048, **kw)
    reuse = O.layer_step("reuse", borrowed_idx=full["idx"], **kw)
    assert np.array_equal(full["out"], reuse["out"]) and np.array_equal(full["lse"], reuse["lse"])
    # re-scoring with the same indexer Q inside a pool that covers everything is the Full layer
    assert (full["pool"] >= 0).sum() == -(-n // 8)
    re = O.layer_step("reindex", q_codes=qc, q_scales=qs, w=w, pool=full["pool"], **kw)
    assert np.array_equal(re["idx"], full["idx"])
    # each layer attends with its own window cache
    other = O.layer_step("reuse", borrowed_idx=full["idx"], **{**kw, "layer": 1})
    assert not np.allclose(other["out"], full["out"])


def test_padding_indices_are_skipped():
    rng = np.random.default_rng(6)
    caches = _tiny_caches(rng, 50)
    q = rng.normal(size=(2, 512))
    idx = np.array([3, 9, 20, -1, -1])
    main = caches.main_rows(idx)
    assert main.shape[0] == 3
    out, _ = O.sparse_attention(q, main, caches.swa_rows(0, O.swa_positions(5, 5, 16)), 0.05)
    ref, _ = O.attention(q, np.concatenate([main, caches.swa_rows(0, [5])]), 0.05)
    assert np.array_equal(out, ref)

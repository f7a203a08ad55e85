"""The no-allocation attention entry point against the workspace one: csa2_sparse_attn_noalloc
must return exactly what csa2_sparse_attn returns for the same arguments (the same kernels;
only the split partials' memory differs), on two calls in a row, the second smaller, so the
second reads a static scratch that still holds the first call's partials."""
import math
import sys

import numpy as np
import pytest
import torch

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


def _case(n_q, heads, seed):
    t = [2400 - 29 * i for i in range(n_q)]
    s = [0 if i % 2 else max(0, ti - 40) for i, ti in enumerate(t)]
    wl = G.workloads.Workload(
        name="noalloc", seed=seed, n_seq=n_q, seq_cap=2401, m=1, heads=heads, idx_heads=16,
        q_seq=np.arange(n_q, dtype=np.int32), q_pos=np.array(t, np.int64), replay_start=np.array(s, np.int64),
        layers=("full",), new_entries=(0, 0))
    return G.Case(wl), t


def test_noalloc_matches_workspace_call(C):
    assert C.csa2_sparse_attn_noalloc_max_bytes() == 16 << 20
    results = []
    for n_q, heads, out_dt in ((24, 64, torch.float32), (6, 16, torch.bfloat16)):
        _say("noalloc", n_q, heads, out_dt)
        case, t = _case(n_q, heads, 40 + n_q)
        caches = case.gpu_caches()
        _, _, qa = case.gpu_query_inputs(0)
        q_seq, _, q_pos, rs = case.gpu_meta()
        rng = np.random.default_rng(n_q)
        idx = np.full((n_q, 512), -1, np.int32)
        for i in range(n_q):
            c = 512 if i % 3 else int(rng.integers(1, 512))
            idx[i, :c] = np.sort(rng.choice(t[i] + 1, size=c, replace=False))
        idx_t = torch.from_numpy(idx).cuda()
        need = C.csa2_attn_workspace_bytes(n_q, heads, 512, 512, 128)
        assert 0 < need <= C.csa2_sparse_attn_noalloc_max_bytes()      # the key list is split
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        out_a = torch.empty(n_q, heads, 512, dtype=out_dt, device="cuda")
        lse_a = torch.empty(n_q, heads, dtype=torch.float32, device="cuda")
        out_b = torch.full_like(out_a, 7.0)
        lse_b = torch.full_like(lse_a, 7.0)
        sm = 1.0 / math.sqrt(512)
        C.csa2_sparse_attn(qa, caches.kv_codes, caches.kv_scales, q_seq, idx_t, caches.swa[0], caches.swa_base, q_pos,
                           rs, 128, sm, out_a, lse_a, workspace=ws)
        C.csa2_sparse_attn_noalloc(qa, caches.kv_codes, caches.kv_scales, q_seq, idx_t, caches.swa[0],
                                   caches.swa_base, q_pos, rs, 128, sm, out_b, lse_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
        # and the oracle, on two rows
        for qi in (0, n_q - 1):
            oc = case.oracle_caches(qi)
            _, _, _, qa_np = case.oracle_query(0, qi)
            ref, ref_lse = G.O.sparse_attention(qa_np, oc.main_rows(idx[qi][idx[qi] >= 0]),
                                                oc.swa_rows(0, G.O.swa_positions(t[qi], int(case.wl.replay_start[qi]),
                                                                                 128)), sm)
            if out_dt == torch.float32:
                G.attn_close(out_b[qi].cpu().numpy(), ref, 2e-3)
            else:
                G.attn_close_bf16(out_b[qi].float().cpu().numpy(), ref)
            assert np.abs(lse_b[qi].cpu().numpy() - ref_lse).max() <= 1e-3
        results.append(n_q)
        del caches
    assert results == [24, 6]

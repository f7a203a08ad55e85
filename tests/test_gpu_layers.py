"""Full-size layer groups on the GPU: the 128K group (Full, 3 Reuse, Reindex; 32 queries),
the 1M group (Full + pool, 4 Reindex inside the pool; 8 queries), both also with the
NVFP4-style indexer, the whole 20-layer decoder step at 128K and 1M, and the m = 2 prefill
chunk, run through the layer driver exactly as
the benchmark runs them, with oracle parity on sampled query rows."""
import sys

import pytest
import torch

from synth import workloads
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


ALL = None   # every query row of the workload


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,samples,fused,attn_select,interleaved", [
    ("c2", (0, 63), True, False, False), ("c2", ALL, True, True, False), ("c3", (0, 13, 31), True, False, False),
    ("c3", (0, 13, 31), False, False, False), ("c3", ALL, True, True, False), ("c4", (0, 5), True, False, False),
    ("c4", (0, 5), False, False, False), ("c4", ALL, True, True, False),
    ("c2", ALL, True, True, True), ("c3", ALL, True, True, True), ("c4", (0, 3, 7), True, True, True)])
def test_layer_group_full_size(C, name, samples, fused, attn_select, interleaved):
    """Every layer of a group at full size against the oracle: fused scoring + selection,
    two calls, and the last Top-K level inside the attention call.  The cases with the
    selection inside attention run as the single-token decode step is benchmarked (each
    row's own window entry appended by the attention call, its ring row zeroed beforehand)
    and are checked on every query row: index set and pool by the acceptance rule, cache
    bytes, and attention.  The other variants attend over a prefilled ring and are checked
    on sampled rows.  interleaved: the main KV as one 288-byte record per entry (codes, then
    scales; both strides 288), written by the quantiser and read by every attention call
    through the strides of the boundary."""
    _say("layer group", name, "fused" if fused else "two-call", "select in attention" if attn_select else "",
         "interleaved main KV" if interleaved else "")
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config(name)
    case = G.Case(wl, swa_layers=range(len(wl.layers)), interleaved=interleaved)
    caches = case.gpu_caches()
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap, fused=fused, attn_select=attn_select)
    # at 1M the segment survivors exceed one selection, so only the pool's Top-K (Reindex
    # inside the pool) moves into the attention call
    assert (step.attn_select or step.pool_select) == attn_select
    if interleaved:
        assert caches.kv_codes.stride(1) == 288 and caches.kv_scales.stride(1) == 288
        assert caches.kv_scales.data_ptr() == caches.kv_codes.data_ptr() + 256
    snaps = G.run_group_snapshots(case, step, caches, fused_window=attn_select)
    rows = range(wl.n_q) if samples is ALL else samples
    _say("  oracle rows", len(rows))
    G.check_group_rows(case, caches, snaps, rows, workers=8 if wl.seq_cap > (1 << 18) else 16)
    del caches, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,samples", [("c2", (0, 63)), ("c4", (0, 5))])
def test_nvfp4_indexer_full_size(C, name, samples):
    """The NVFP4-style indexer variant (E4M3 per 16 channels, fp16 matrix-core scoring) at
    full size: the 64 x 128K Full step and the 1M group (Full + pool through the unfused
    score / select / pool calls, then Reindex inside the pool), with oracle parity of
    every layer on sampled query rows."""
    _say("nvfp4 indexer", name)
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config(name)
    case = G.Case(wl, swa_layers=range(len(wl.layers)), index_fmt="nvfp4")
    caches = case.gpu_caches()
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap, index_fmt="nvfp4")
    snaps = G.run_group_snapshots(case, step, caches)
    for qi in samples:
        _say("  oracle query", qi)
        G.check_group_query(case, caches, snaps, qi)
    del caches, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,samples", [("dec_128k", (0, 31)), ("dec_1m", (0, 7))])
def test_decoder_step_full_size(C, name, samples):
    """The whole decoder step: 20 CSA2 layers (Full + pool, 3 Reuse, 4 x (Reindex in the pool,
    3 Reuse)) at 128K and 1M, through the layer driver as the benchmark runs it (each layer's
    attention call appending the row's own window entry), with oracle parity of every layer
    on sampled query rows."""
    _say("decoder step", name)
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config(name)
    case = G.Case(wl, swa_layers=range(len(wl.layers)))
    caches = case.gpu_caches()
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap)
    snaps = G.run_group_snapshots(case, step, caches, fused_window=True)
    for qi in samples:
        _say("  oracle query", qi)
        G.check_group_query(case, caches, snaps, qi)
    del caches, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("group,fused", [(4, True), (1, True), (1, False)])
def test_multi_token_decode_full_size(C, group, fused):
    """Multi-token decode: 16 sequences x 4 tokens at 128K through a Full layer, the 4 rows
    of a sequence scored in one pass over its indexer K (group 4: grouped scores, then the
    Top-K levels) or apart (group 1: fused per row, or scores then Top-K), with oracle parity
    on rows of several sequences and token offsets."""
    _say("multi-token decode, group", group, "fused" if fused else "two-call")
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config("mtd_128k")
    case = G.Case(wl, swa_layers=range(len(wl.layers)))
    caches = case.gpu_caches()
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap, group=group, fused=fused)
    snaps = G.run_group_snapshots(case, step, caches)
    for qi in (0, 3, 29, 62):
        _say("  oracle query", qi)
        G.check_group_query(case, caches, snaps, qi)
    del caches, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_encoder_group_prefill_window_miss(C):
    """An encoder CSA2 group (Full + 5 Reuse, m = 2) over a 4,096-token chunk after a
    262,144-token prefix whose window state is not cached: every layer writes the FP8 window
    entries of its 128 replay rows and 4,096 new rows, then attends with the window bounded
    at the replay start.  Oracle parity of every layer (index set, window rows written,
    attention) on replay and new rows."""
    _say("encoder group prefill, window miss")
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config("enc_group")
    assert wl.extra["swa_miss"]
    case = G.Case(wl, swa_layers=range(len(wl.layers)))
    caches = case.gpu_caches(window_empty=True)
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap, group=8)   # the chunk's rows: one sequence
    snaps = G.run_group_snapshots(case, step, caches, window_appends=True)
    for qi in (0, 127, 128, 3000, wl.n_q - 1):
        _say("  oracle query", qi, "t", int(wl.q_pos[qi]))
        G.check_group_query(case, caches, snaps, qi)
    del caches, step
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("group", [8, 1])
def test_prefill_chunk_full_size(C, group):
    """The m = 2 encoder prefill chunk: 4,096 new tokens after a 262,144-token prefix plus the
    128 bounded-replay rows, one sequence of 133,120 entries, run as one Full layer; oracle
    parity on replay rows (first, middle, last), the first new row, a middle and the last row;
    the rows scored in groups of 8 over one pass of the indexer K, and one by one."""
    _say("prefill chunk, group", group)
    from fp4_kv_cache_layer_amd.layer import Csa2Step
    wl = workloads.config("c5")
    case = G.Case(wl, swa_layers=(0,))
    caches = case.gpu_caches()
    step = Csa2Step(wl.n_q, wl.heads, wl.idx_heads, wl.seq_cap, group=group)
    assert step.group_select == (group > 1)          # grouped rows: scored and selected in one pass
    snaps = G.run_group_snapshots(case, step, caches)
    rows = sorted({0, 1, 63, 126, 127, 128, 129, wl.n_q - 1} | set(range(128, wl.n_q, 61)))
    _say("  oracle rows", len(rows))
    G.check_group_rows(case, caches, snaps, rows, workers=16, shared_index=True)
    del caches, step
    torch.cuda.empty_cache()

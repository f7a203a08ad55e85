"""Host-side orchestration of a layer group (no GPU): the mode rules of the pages and the
calls each layer makes, checked against the oracle's model schedule."""
import pytest

from fp4_kv_cache_layer_amd.layer import plan_group
from oracle import csa2_oracle as O


def _groups(schedule):
    """Splits the model schedule into groups, each opened by a Full layer."""
    groups = []
    for part, _, mode in schedule:
        if mode == "full":
            groups.append([])
        groups[-1].append(mode)
    return groups


def test_model_schedule_groups_plan():
    groups = _groups(O.layer_schedule())
    assert len(groups) == 4            # 3 encoder groups, 1 decoder group with 4 Reindex layers
    for g in groups:
        plan = plan_group(g)
        assert len(plan) == len(g)
        for mode, calls in zip(g, plan):
            assert calls[-1] == "attend"
            if mode == "reuse":
                assert calls == ["attend"]          # borrows the index set: no scoring
            elif mode == "full":
                assert calls[0] == "quantize_index_q"   # its own indexer Q (and the step's appends)
            else:
                assert calls[0].endswith("_q")      # its own indexer Q, quantised by the scoring call
                assert "quantize_index_q" not in calls
        assert all(p[0] == "quantize_index_q" for m, p in zip(g, plan_group(g, q_in_call=False)) if m != "reuse")
    dec = _groups(O.layer_schedule())[-1]
    dec = ["full_pool"] + ["reindex_pool" if m == "reindex" else m for m in dec[1:]]
    plan = plan_group(dec)
    assert plan[0] == ["quantize_index_q", "index_topk_pool", "attend"]     # Top-K and pool in one pass
    assert all(p == ["index_topk_in_pool_q", "attend"] for m, p in zip(dec, plan) if m == "reindex_pool")
    plan = plan_group(dec, q_in_call=False)
    assert all(p == ["quantize_index_q", "index_topk_in_pool", "attend"] for m, p in zip(dec, plan)
               if m == "reindex_pool")
    plan = plan_group(dec, fused=False)
    assert "build_pool" in plan[0] and plan[0].index("build_pool") < plan[0].index("attend")


def test_decoder_step_is_the_model_decoder():
    """The benchmarked decoder step runs the model's 20 decoder layers, pool-based."""
    from synth.workloads import decoder_modes, config
    dec = _groups(O.layer_schedule())[-1]
    assert len(dec) == 20
    want = ["full_pool"] + ["reindex_pool" if m == "reindex" else m for m in dec[1:]]
    assert list(decoder_modes()) == want
    plan = plan_group(decoder_modes())
    assert sum(1 for p in plan if p != ["attend"]) == 5      # 1 Full + 4 Reindex score
    for name in ("dec_128k", "dec_1m"):
        assert config(name).layers == decoder_modes()


def test_grouped_plan_scores_then_selects():
    plan = plan_group(["full", "reuse", "reindex", "full_pool", "reindex_pool"], group=4)
    assert plan[0] == ["quantize_index_q", "index_topk_grouped", "attend"]   # no score array
    assert plan[2] == ["quantize_index_q", "index_topk_grouped", "attend"]
    assert plan[3] == ["quantize_index_q", "index_topk_pool", "attend"]      # pool layers keep their path
    assert plan[4] == ["quantize_index_q", "index_topk_in_pool", "attend"]
    assert plan_group(["full"], group=1)[0] == ["quantize_index_q", "index_topk", "attend"]
    assert plan_group(["full", "reindex"], group=1)[1] == ["index_topk_q", "attend"]
    assert plan_group(["full"], fused=False, group=4)[0] == ["quantize_index_q", "score_grouped", "select", "attend"]
    with pytest.raises(ValueError):   # grouped scoring reads quantised Q only
        plan_group(["full"], group=4, q_in_call=True)


def test_unfused_plan_keeps_two_calls():
    plan = plan_group(["full", "reuse", "reindex", "reindex"], fused=False)
    assert plan[0] == ["quantize_index_q", "score", "select", "attend"]
    assert plan[2] == ["score_q", "select", "attend"]
    plan = plan_group(["full", "reuse", "reindex", "reindex"], fused=False, q_in_call=False)
    assert plan[0] == ["quantize_index_q", "score", "select", "attend"]
    plan = plan_group(["full", "reindex"], fused=False, index_fmt="nvfp4")   # NVFP4: quantised Q
    assert plan[1] == ["quantize_index_q", "score", "select", "attend"]


@pytest.mark.parametrize("modes", [["reuse"], ["reindex", "reuse"], ["full", "reindex_pool"], ["full_pool", "bogus"],
                                   ["reindex_pool"]])
def test_invalid_groups_rejected(modes):
    with pytest.raises(ValueError):
        plan_group(modes)


def test_plan_select_in_attention():
    """With attn_select, Full and Reindex layers without a pool score with csa2_index_segments
    and finish the Top-K in their attention call, Reindex layers in the pool write the slot
    scores and select in their attention call (pool_select, default attn_select); the pool
    build and grouped scoring keep their calls."""
    plan = plan_group(["full", "reuse", "reindex"], attn_select=True)
    assert plan[0] == ["quantize_index_q", "index_segments", "attend_topk"]
    assert plan[1] == ["attend"]
    assert plan[2] == ["index_segments_q", "attend_topk"]    # the scoring call quantises Q itself
    plan = plan_group(["full", "reuse", "reindex"], attn_select=True, q_in_call=False)
    assert plan[2] == ["quantize_index_q", "index_segments", "attend_topk"]
    plan = plan_group(["full_pool", "reuse", "reindex_pool"], attn_select=True)
    assert plan[0] == ["quantize_index_q", "index_topk_pool", "attend"]
    assert plan[2] == ["score_pool_q", "attend_pool_topk"]
    plan = plan_group(["full_pool", "reuse", "reindex_pool"], attn_select=False, pool_select=True)
    assert plan[2] == ["score_pool_q", "attend_pool_topk"]
    plan = plan_group(["full_pool", "reuse", "reindex_pool"], index_fmt="nvfp4", pool_select=True)
    assert plan[2] == ["quantize_index_q", "score_pool", "attend_pool_topk"]
    plan = plan_group(["full_pool", "reuse", "reindex_pool"], attn_select=True, pool_select=False)
    assert plan[2] == ["index_topk_in_pool_q", "attend"]
    assert plan_group(["full"], group=4, attn_select=True)[0] == ["quantize_index_q", "index_topk_grouped", "attend"]
    assert plan_group(["full"], fused=False, attn_select=True)[0] == ["quantize_index_q", "score", "select", "attend"]

"""Pins of the cache sizes and layer schedule against the pages' numbers, and of the
synthetic inputs against the pages' magnitude argument (no GPU)."""
import json
import math
import os

import numpy as np

from oracle import csa2_oracle as O
from synth import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "pages_constants.json")) as f:
    PAGES = json.load(f)


def test_entry_sizes():
    assert O.nvfp4_entry_bytes(512) == 256 + 32 == 288
    assert O.mxfp4_entry_bytes(128) == 64 + 4 == 68


def test_schedule_counts():
    sched = O.layer_schedule()
    modes = [m for _, _, m in sched]
    assert len(sched) == PAGES["csa2_layers"]["value"] == 38
    assert modes.count("full") == PAGES["csa2_layers"]["full_layers"] == 4
    assert modes.count("reindex") == 4 and modes.count("reuse") == 30
    assert sum(1 for p, m, _ in sched if p == "encoder" and m == 2) == 18
    assert sum(1 for p, m, _ in sched if p == "decoder" and m == 1) == 20


def test_890_bytes_per_token():
    # 356 B per entry (288 main + 68 indexer K) over the decoder's m=1 cache and the three
    # encoder m=2 caches: 356 + 3 * 178 = 890
    assert O.global_kv_bytes_per_token() == PAGES["global_kv_bytes_per_token"]["value"]
    # an E4M3-per-16 indexer-K format would give 72 B per entry and 900 B per token
    assert (288 + 64 + 8) * (1 + 3 / 2) == 900


def test_one_million_token_session_under_1gb():
    assert O.global_kv_bytes_per_token() * 2 ** 20 < PAGES["session_1m_tokens_under_bytes"]["value"]


def test_pool_capacity():
    assert PAGES["pool_max_blocks"]["value"] * PAGES["pool_block_positions"]["value"] == \
        PAGES["pool_max_positions"]["value"]


def test_synthetic_latents_respect_magnitude_bound():
    # unit-weight RMS norm makes the 512-channel L2 norm sqrt(512) (up to eps), RoPE keeps
    # it, so no channel exceeds 22.63 and no E4M3 group scale exceeds 22.63/6 -> 3.75
    wl = workloads.config("c1")
    x = wl.main_latents(0, 0, 2048).astype(np.float64)
    norms = np.linalg.norm(x, axis=1)
    bound = PAGES["latent_l2_bound"]["value"]
    assert np.allclose(norms, math.sqrt(512), rtol=1e-5)
    assert abs(math.sqrt(512) - bound) < 0.05
    assert np.abs(x).max() <= math.sqrt(512)
    _, scales = O.quantize_nvfp4(x.astype(np.float32))
    assert O.E4M3[scales].max() <= 3.75
    # observed magnitudes are far below the representable 2688
    assert np.abs(x).max() < PAGES["fp4_range"]["value"]


def test_synth_is_counter_based():
    wl = workloads.config("c2")
    a = wl.main_latents(3, 1000, 40)
    b = wl.main_latents(3, 1010, 10)
    assert np.array_equal(a[10:20], b)
    assert not np.array_equal(wl.main_latents(4, 1010, 10), b)
    q = wl.index_q(0, 5, 3)
    assert np.array_equal(q, wl.index_q(0)[5:8])

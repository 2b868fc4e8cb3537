"""Synthetic workload shapes against the numbers the pages print
(fixtures in tests/golden/page_numbers.json, each with its citation)."""
import json
import math
import os

import numpy as np

from replay_inputs import PAGE, config_c3, group_weights, suffix_pool_case

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "page_numbers.json")))


def test_replay_budget_ceil():
    for case in GOLD["replay_budget_ratio"]["cases"]:
        assert math.ceil(case["r"] * case["m"]) == case["k"]
    # the hit generator draws k = ceil(r m) for its own (m, r)
    pc = suffix_pool_case(40, 8192, 32768, 0.05, 0.10, 8, seed=3)
    for m, r, k in zip(pc.matched_len, pc.meta["r"], pc.suffix_len):
        assert k == math.ceil(r * int(m))
        assert 0.05 * m <= k <= 0.10 * m + 1
        assert 8192 <= m <= 32768


def test_capped_budget_formula():
    for case in GOLD["replay_budget_capped"]["cases"]:
        assert min(0.05 * case["n"], case["k_max"]) == case["k"]


def test_page_size():
    assert PAGE == GOLD["page_tokens"]["value"]


def test_head_shapes_match_printed_state_size():
    # 32 value heads x 128 x 128 fp32 per GDN layer (the shapes the GDN
    # workloads use), 24 GDN layers of a 32-layer 3:1 hybrid, plus the
    # short-conv windows (3 rows of the 8192 q|k|v channels, bf16): about
    # 49 MiB.  KV: 8 full-attention layers x K,V x 4 heads x 256 x bf16.
    c = config_c3(n_seqs=1, seqlen=4)
    w = group_weights(np.random.default_rng(0), 64, 16, 32, 128)
    conv_dim = w.conv_w.shape[0]
    state = 24 * c.h_v * c.d_k * c.d_v * 4 + 24 * conv_dim * 3 * 2
    mib = state / 2 ** 20
    kv = 8 * 2 * 4 * 256 * 2 / 2 ** 10
    g = GOLD["state_vs_kv_size"]
    assert abs(mib - g["checkpoint_mib_approx"]) < 1.0
    assert kv == g["kv_kib_per_token_approx"]
    assert abs(state / (kv * 2 ** 10) / g["ratio_approx"] - 1) < 0.05

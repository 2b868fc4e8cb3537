"""Pins of the oracle's token-wise sparse anchors and capped replay budget
("SuffixReplay", Algorithm Design 2-3), and of the library's host-side
budget function against it.  No GPU."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))
NEAR = (60, 61, 62, 63)     # density 1/16 next to the page boundary
UNIFORM = (15, 31, 47, 63)  # density 1/16 spread over the page


def test_density_one_sixteenth():
    for offs in (NEAR, UNIFORM):
        assert len(offs) / 64 == GOLD["anchor_density"]["value"]
        # a whole page keeps exactly its 4 anchors; the last one is the page's last token
        assert oracle.anchor_positions(64, offs) == list(offs)
        assert oracle.anchor_positions(128, offs)[-1] == 127


@pytest.mark.parametrize("offs", [NEAR, UNIFORM, (0,), tuple(range(64)), (3, 9, 40)])
def test_anchor_count_closed_form(offs):
    # n(m) = A floor(m/64) + #{o < m mod 64}: every page before the partial
    # one contributes all A anchors
    for m in list(range(0, 300)) + [8192, 8193, 32767, 32768]:
        n = len(offs) * (m // 64) + sum(o < m % 64 for o in offs)
        pos = oracle.anchor_positions(m, offs)
        assert len(pos) == n
        assert pos == sorted(pos) and all(0 <= p < m for p in pos)
        assert all(p % 64 in offs for p in pos)


def test_dense_anchors_are_the_plain_suffix_gather():
    rng = np.random.default_rng(0)
    P, D = 40, 8
    pool = rng.integers(0, 2 ** 16, size=(P, 64, D), dtype=np.uint16)
    pt = rng.permutation(P).astype(np.int32).reshape(4, 10)
    m = np.array([640, 1, 333, 64], np.int32)
    k = np.array([100, 1, 333, 0], np.int32)
    a, cu_a, pos = oracle.gather_anchors(pool, tuple(range(64)), pt, m, k)
    b, cu_b = oracle.gather_suffix(pool, pt, m, k)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(cu_a, cu_b)
    for i in range(4):
        np.testing.assert_array_equal(pos[cu_a[i]:cu_a[i + 1]], np.arange(m[i] - k[i], m[i]))


@pytest.mark.parametrize("offs", [NEAR, UNIFORM, (5, 6, 50)])
def test_sparse_gather_reads_the_anchor_positions_of_a_token_pool(offs):
    """Brute force: a token-level pool holds every position; keeping only the
    rows at the anchor offsets gives the sparse pool; each packed row must be
    the token row at its returned position, and the positions the last k of
    the prefix's anchor positions."""
    rng = np.random.default_rng(1)
    n_req, P, D = 5, 60, 6
    full = rng.integers(0, 2 ** 16, size=(P, 64, D), dtype=np.uint16)
    sparse = np.ascontiguousarray(full[:, list(offs), :])
    pt = rng.permutation(P).astype(np.int32).reshape(n_req, 12)
    m = np.array([768, 700, 64, 63, 1], np.int32)
    n_anchor = [len(oracle.anchor_positions(x, offs)) for x in m]
    k = np.array([min(n, x) for n, x in zip(n_anchor, [40, 7, 2, 9, 5])], np.int32)
    packed, cu, pos = oracle.gather_anchors(sparse, offs, pt, m, k)
    assert cu[-1] == k.sum() == packed.shape[0] == pos.shape[0]
    for i in range(n_req):
        want = oracle.anchor_positions(m[i], offs)[n_anchor[i] - k[i]:]
        got = pos[cu[i]:cu[i + 1]]
        np.testing.assert_array_equal(got, want)
        for r, p in zip(range(cu[i], cu[i + 1]), got):
            np.testing.assert_array_equal(packed[r], full[pt[i][p // 64], p % 64])


def test_gather_rejects_more_anchors_than_held():
    pool = np.zeros((2, 4, 2), np.uint16)
    with pytest.raises(ValueError):
        oracle.gather_anchors(pool, NEAR, np.array([[0, 1]], np.int32), [64], [5])


def test_budget_against_page_numbers():
    for case in GOLD["replay_budget_capped"]["cases"]:
        assert oracle.replay_budget([case["n"]], 0.05, case["k_max"]) == [math.ceil(case["k"])]
    for case in GOLD["replay_budget_ratio"]["cases"]:
        assert oracle.replay_budget([case["m"]], case["r"], 0) == [case["k"]]
    # 7 % of 100 is exactly 7 (not 8: the ratio is the decimal it is written as)
    assert oracle.replay_budget([100], 0.07, 0) == [7]
    assert oracle.replay_budget([0, 1, 19, 20, 21], 0.05, 0) == [0, 1, 1, 1, 2]


def test_library_budget_equals_oracle_budget():
    """The library's host-side budget (sr_replay_budget) against the oracle's
    exact-decimal definition on every count up to 40000."""
    from linear_attention_state_anchor_amd import _lib, build, replay_budget
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    n = list(range(0, 40001))
    for ratio in (0.05, 0.10, 0.07, 0.0625, 0.3, 1.0):
        for k_max in (0, 256, 512):
            assert replay_budget(n, ratio, k_max) == oracle.replay_budget(n, ratio, k_max), \
                (ratio, k_max)

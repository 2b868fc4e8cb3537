"""Pins of the fp64 recurrence oracle to closed forms, invariants and brute
force ("SuffixReplay", Eq. 4; "Tail-Replay", section 2).

Each test fixes the oracle against something other than itself, chosen so
that a plausible slip (a dropped decay, a sign of the erase term, a transposed
state, a wrong GQA index, the output taken before the update) fails at least
one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from replay_inputs import gdn_case, widen

RNG = np.random.default_rng(1234)


def _run(c, **kw):
    return oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, c.h_k, c.h_v,
                      alpha_is_log=c.alpha_is_log, erase=c.erase,
                      initial_state=c.initial_state, **kw)


def _log_alpha(c):
    a = widen(c.alpha)
    return a if c.alpha_is_log else np.log(a)


# ---------------------------------------------------------------------------
# single token from zero state: S_1 = b v k^T, o_1 = b (k.q) v
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("erase", [True, False])
def test_single_token_closed_form(erase):
    c = gdn_case([1], 2, 4, 8, "f32", seed=5, erase=erase, d_v=6)
    S, o = _run(c)
    q, k, v, b = widen(c.q), widen(c.k), widen(c.v), widen(c.beta)
    for h in range(4):
        g = h // 2
        expect_S = b[0, h] * np.outer(k[0, g], v[0, h])       # [d_k][d_v]
        np.testing.assert_allclose(S[0, h], expect_S, rtol=1e-15, atol=1e-15)
        expect_o = b[0, h] * np.dot(k[0, g], q[0, g]) * v[0, h]
        np.testing.assert_allclose(o[0, h], expect_o, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# delta-rule invariant: with b = 1 and |k_t| = 1, S_t k_t = v_t for any decay
# and any history, because (I - k k^T) k = 0.  With q_t = k_t, o_t = v_t.
# ---------------------------------------------------------------------------
def test_beta_one_unit_key_stores_value():
    T, d = 40, 16
    k = np.zeros((T, 1, d))
    for t in range(T):  # four entries of +-0.5: unit norm, exact in bf16
        idx = RNG.choice(d, 4, replace=False)
        k[t, 0, idx] = RNG.choice([-0.5, 0.5], 4)
    v = RNG.standard_normal((T, 1, d))
    alpha = RNG.uniform(0.2, 1.0, size=(T, 1))
    cu = np.array([0, T], np.int32)
    s0 = RNG.standard_normal((1, 1, d, d))
    S, o = oracle.gdn(k, k, v, alpha, np.ones((T, 1)), cu, 1, 1,
                      alpha_is_log=False, initial_state=s0)
    np.testing.assert_allclose(o[:, 0], v[:, 0], rtol=0, atol=1e-12)
    # and the last key reads back the last value from the final state
    np.testing.assert_allclose(k[-1, 0] @ S[0, 0], v[-1, 0], atol=1e-12)


# ---------------------------------------------------------------------------
# alpha = 1, b = 1, distinct basis-vector keys: S_T = sum_t v_t k_t^T exactly
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("erase", [True, False])
def test_orthonormal_keys_store_values_exactly(erase):
    d, T = 32, 20
    perm = RNG.permutation(d)[:T]
    k = np.zeros((T, 1, d))
    k[np.arange(T), 0, perm] = 1.0
    v = np.round(RNG.standard_normal((T, 1, d)) * 64) / 64
    cu = np.array([0, T], np.int32)
    S, _ = oracle.gdn(k, k, v, np.ones((T, 1)), np.ones((T, 1)), cu, 1, 1,
                      alpha_is_log=False, erase=erase, want_o=False)
    expect = k[:, 0].T @ v[:, 0]                       # K^T V = [d_k][d_v]
    assert np.array_equal(S[0, 0], expect)


# ---------------------------------------------------------------------------
# b = 0 with a nonzero initial state: pure decay of S_0
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("erase", [True, False])
def test_beta_zero_pure_decay(erase):
    c = gdn_case([17, 5], 2, 2, 8, "f32", seed=9, beta="zero", erase=erase,
                 initial_state=True)
    S, o = _run(c)
    ga = _log_alpha(c)
    q = widen(c.q)
    s0 = widen(c.initial_state)
    for n in range(2):
        a, b = c.cu_seqlens[n], c.cu_seqlens[n + 1]
        for h in range(2):
            decay = np.exp(np.cumsum(ga[a:b, h]))
            np.testing.assert_allclose(S[n, h], decay[-1] * s0[n, h], rtol=1e-13)
            for t in range(a, b):
                expect = decay[t - a] * (s0[n, h].T @ q[t, h])
                np.testing.assert_allclose(o[t, h], expect, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# erase-free closed form: S_T^T = K^T diag(w) V, w_t = b_t prod_{s>t} a_s;
# O = (M * Q K^T) diag(b) V with M_tj = prod_{s=j+1..t} a_s (j <= t).
# One library matmul each.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("beta", ["sigmoid", "none"])
def test_erase_free_closed_form(beta):
    c = gdn_case([50, 31], 2, 4, 16, "bf16", seed=11, normalize_k=False,
                 alpha=("uniform", 0.90, 0.999), beta=beta, erase=False)
    S, o = _run(c)
    q, k, v = widen(c.q), widen(c.k), widen(c.v)
    ga = _log_alpha(c)
    bb = np.ones(ga.shape) if c.beta is None else widen(c.beta)
    for n in range(2):
        a, e = c.cu_seqlens[n], c.cu_seqlens[n + 1]
        for h in range(4):
            g = h // 2
            G = np.cumsum(ga[a:e, h])
            w = bb[a:e, h] * np.exp(G[-1] - G)
            expect = k[a:e, g].T @ (w[:, None] * v[a:e, h])
            np.testing.assert_allclose(S[n, h], expect, rtol=1e-11, atol=1e-11)
            L = e - a
            M = np.tril(np.exp(G[:, None] - G[None, :]))
            O = (M * (q[a:e, g] @ k[a:e, g].T)) @ (bb[a:e, h][:, None] * v[a:e, h])
            np.testing.assert_allclose(o[a:e, h], O, rtol=1e-10, atol=1e-10)
            assert L > 0


# ---------------------------------------------------------------------------
# brute force: S_T = S_0 M_1...M_T + sum_t B_t M_{t+1}...M_T with explicit
# d_k x d_k matrices M_t = a_t (I - b_t k_t k_t^T) (erase) or a_t I, and
# B_t = b_t v_t k_t^T.  Tiny sizes, an independent formulation.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("T,d_k,d_v", [(1, 1, 1), (4, 3, 2), (6, 2, 3), (6, 3, 3)])
def test_brute_force_tiny(erase, T, d_k, d_v):
    rng = np.random.default_rng(T * 100 + d_k * 10 + d_v)
    k = rng.standard_normal((T, 1, d_k))
    q = rng.standard_normal((T, 1, d_k))
    v = rng.standard_normal((T, 1, d_v))
    a = rng.uniform(0.3, 1.0, (T, 1))
    b = rng.uniform(0.0, 1.5, (T, 1))
    s0 = rng.standard_normal((1, 1, d_k, d_v))
    cu = np.array([0, T], np.int32)
    S, o = oracle.gdn(q, k, v, a, b, cu, 1, 1, alpha_is_log=False, erase=erase,
                      initial_state=s0)
    I = np.eye(d_k)
    Ms = [a[t, 0] * (I - b[t, 0] * np.outer(k[t, 0], k[t, 0])) if erase
          else a[t, 0] * I for t in range(T)]
    for t_end in range(1, T + 1):
        acc = s0[0, 0].T.copy()                       # d_v x d_k
        for t in range(t_end):
            acc = acc @ Ms[t]
        for t in range(t_end):
            B = b[t, 0] * np.outer(v[t, 0], k[t, 0])
            for s in range(t + 1, t_end):
                B = B @ Ms[s]
            acc = acc + B
        np.testing.assert_allclose(o[t_end - 1, 0], acc @ q[t_end - 1, 0],
                                   rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], acc.T, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# exact rational arithmetic on dyadic inputs: the fp64 oracle is exact here
# ---------------------------------------------------------------------------
def test_exact_rationals():
    F = Fraction
    k = [[F(1, 2), F(1, 2)], [F(1), F(0)], [F(0), F(-1, 2)]]
    v = [[F(1), F(-2)], [F(3, 4), F(1, 4)], [F(-1, 8), F(1)]]
    q = [[F(1), F(1)], [F(0), F(2)], [F(1, 4), F(-1)]]
    a = [F(1, 2), F(3, 4), F(1)]
    b = [F(1, 2), F(1), F(1, 4)]
    S = [[F(0)] * 2 for _ in range(2)]              # d_v x d_k
    outs = []
    for t in range(3):
        x = [sum(S[i][j] * k[t][j] for j in range(2)) for i in range(2)]
        S = [[a[t] * S[i][j] - a[t] * b[t] * x[i] * k[t][j] + b[t] * v[t][i] * k[t][j]
              for j in range(2)] for i in range(2)]
        outs.append([sum(S[i][j] * q[t][j] for j in range(2)) for i in range(2)])
    f = lambda m: np.array([[float(e) for e in r] for r in m])
    So, oo = oracle.gdn(f(q)[:, None], f(k)[:, None], f(v)[:, None],
                        np.array([[float(x)] for x in a]),
                        np.array([[float(x)] for x in b]),
                        np.array([0, 3], np.int32), 1, 1, alpha_is_log=False)
    assert np.array_equal(So[0, 0], f(S).T)
    assert np.array_equal(oo[:, 0], f(outs))


# ---------------------------------------------------------------------------
# the replay bound: S_n - S'_n = S_{n-k} M_{n-k+1} ... M_n, so
# |S_n - S'_n|_F <= (prod of the replayed alphas) |S_{n-k}|_F when
# 0 <= b |k|^2 <= 2, with equality in erase-free mode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("erase", [True, False])
def test_replay_error_bound(erase):
    n, kk = 300, 60
    c = gdn_case([n], 2, 2, 16, "f32", seed=21, erase=erase, normalize_k=True,
                 alpha=("uniform", 0.9, 1.0))
    full, _ = _run(c, want_o=False)
    run = lambda a, b: oracle.gdn(None, c.k[a:b], c.v[a:b], c.alpha[a:b],
                                  c.beta[a:b], np.array([0, b - a], np.int32), 2, 2,
                                  alpha_is_log=False, erase=erase, want_o=False)[0]
    prefix = run(0, n - kk)
    replay = run(n - kk, n)
    ga = _log_alpha(c)
    for h in range(2):
        bound = np.exp(np.sum(ga[n - kk:, h])) * np.linalg.norm(prefix[0, h])
        err = np.linalg.norm(full[0, h] - replay[0, h])
        assert bound > 1e-3 * np.linalg.norm(full[0, h])
        if erase:
            assert 0 < err <= bound * (1 + 1e-9)
        else:
            assert err == pytest.approx(bound, rel=1e-9)


# ---------------------------------------------------------------------------
# splitting a sequence and resuming from the carried state changes nothing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("j", [1, 63, 64, 65, 199])
def test_chunk_split_invariance(j):
    n = 200
    c = gdn_case([n], 2, 4, 16, "bf16", seed=31)
    full, o_full = _run(c)
    sl = lambda x, a, b: None if x is None else x[a:b]
    first, o1 = oracle.gdn(sl(c.q, 0, j), sl(c.k, 0, j), sl(c.v, 0, j),
                           sl(c.alpha, 0, j), sl(c.beta, 0, j),
                           np.array([0, j], np.int32), 2, 4, alpha_is_log=True)
    second, o2 = oracle.gdn(sl(c.q, j, n), sl(c.k, j, n), sl(c.v, j, n),
                            sl(c.alpha, j, n), sl(c.beta, j, n),
                            np.array([0, n - j], np.int32), 2, 4, alpha_is_log=True,
                            initial_state=first)
    np.testing.assert_allclose(second, full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_full, rtol=1e-11,
                               atol=1e-12)


# ---------------------------------------------------------------------------
# grouped keys: value head h reads key head h // (h_v / h_k) -- the same as
# repeating each key head over its contiguous value heads
# ---------------------------------------------------------------------------
def test_gqa_contiguous_grouping():
    c = gdn_case([33, 40], 2, 6, 8, "f32", seed=41)
    S, o = _run(c)
    rep = lambda x: np.repeat(x, 3, axis=1)
    S2, o2 = oracle.gdn(rep(c.q), rep(c.k), c.v, c.alpha, c.beta, c.cu_seqlens,
                        6, 6, alpha_is_log=True)
    assert np.array_equal(S, S2) and np.array_equal(o, o2)
    # and not the interleaved mapping h % h_k
    til = lambda x: np.tile(x, (1, 3, 1))
    S3, _ = oracle.gdn(til(c.q), til(c.k), c.v, c.alpha, c.beta, c.cu_seqlens,
                       6, 6, alpha_is_log=True)
    assert not np.allclose(S, S3)


# ---------------------------------------------------------------------------
# packed varlen equals solo runs; empty sequences return S_0 and no rows
# ---------------------------------------------------------------------------
def test_varlen_packed_equals_solo_and_empty():
    lens = [5, 0, 64, 1, 70]
    c = gdn_case(lens, 1, 2, 8, "bf16", seed=51, initial_state=True)
    S, o = _run(c)
    cu = c.cu_seqlens
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        Sn, on = oracle.gdn(c.q[a:b], c.k[a:b], c.v[a:b], c.alpha[a:b],
                            c.beta[a:b], np.array([0, L], np.int32), 1, 2,
                            alpha_is_log=True, initial_state=c.initial_state[n:n + 1])
        assert np.array_equal(Sn[0], S[n])
        assert np.array_equal(on, o[a:b])
    np.testing.assert_array_equal(S[1], widen(c.initial_state[1]))


def test_output_scale_and_alpha_log_equivalence():
    c = gdn_case([30], 1, 1, 8, "f32", seed=61)
    S, o = _run(c)
    _, o2 = _run(c, scale=0.25)
    np.testing.assert_allclose(o2, 0.25 * o, rtol=1e-15)
    S3, o3 = oracle.gdn(c.q, c.k, c.v, np.exp(widen(c.alpha)), c.beta,
                        c.cu_seqlens, 1, 1, alpha_is_log=False)
    np.testing.assert_allclose(S3, S, rtol=1e-14, atol=1e-15)

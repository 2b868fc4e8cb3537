"""The chunkwise form that the HIP kernel evaluates, checked in fp64 against
the token-by-token oracle.

The pages give only the per-token recurrence ("SuffixReplay", Eq. 4;
"Tail-Replay", section 2).  The chunked form below is derived from it; this
test is what ties the derivation to the recurrence, before any GPU code.

Per chunk of C tokens entering with state S0 (d_v x d_k), g_t = log a_t,
G_t = sum_{s<=t} g_s, e^{G} <= 1:
  A[t,j]  = b_t e^{G_t - G_j} (k_t . k_j)  for j < t, else 0
  Tm      = (I + A)^{-1}                    (unit lower triangular)
  U       = Tm diag(b) V - Tm diag(b e^{G}) K S0^T
  O       = diag(e^{G}) Q S0^T + (P o Q K^T) U,  P[t,j] = e^{G_t - G_j}, j <= t
  S_C^T   = e^{G_C} S0^T + K^T diag(e^{G_C - G}) U
Erase-free mode: A = 0, so U = diag(b) V.
"""
import numpy as np
import pytest

import oracle
from replay_inputs import gdn_case, widen


def chunked(q, k, v, g, b, erase, C, s0T=None):
    L, d_k = k.shape
    d_v = v.shape[1]
    ST = np.zeros((d_k, d_v)) if s0T is None else s0T.copy()
    O = np.zeros((L, d_v))
    for s in range(0, L, C):
        e = min(s + C, L)
        n = e - s
        K, Q, V, gg, bb = k[s:e], q[s:e], v[s:e], g[s:e], b[s:e]
        G = np.cumsum(gg)
        D = G[:, None] - G[None, :]
        low = np.tril(np.ones((n, n)), -1) > 0
        P = np.where(np.tril(np.ones((n, n))) > 0, np.exp(np.where(low | np.eye(n, dtype=bool), D, 0)), 0)
        if erase:
            A = np.where(low, bb[:, None] * np.exp(np.where(low, D, 0)) * (K @ K.T), 0)
            Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
            U = Tm @ (bb[:, None] * V) - Tm @ ((bb * np.exp(G))[:, None] * K) @ ST
        else:
            U = bb[:, None] * V
        O[s:e] = np.exp(G)[:, None] * (Q @ ST) + (P * (Q @ K.T)) @ U
        ST = np.exp(G[-1]) * ST + K.T @ (np.exp(G[-1] - G)[:, None] * U)
    return ST, O


@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("C", [1, 4, 64])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_chunk_form_matches_token_loop(erase, C, L):
    c = gdn_case([L], 1, 2, 16, "bf16", seed=L + C, erase=erase,
                 initial_state=True, normalize_q=True)
    S_ref, o_ref = oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, 1, 2,
                              alpha_is_log=True, erase=erase,
                              initial_state=c.initial_state)
    q, k, v = widen(c.q), widen(c.k), widen(c.v)
    g, b = widen(c.alpha), widen(c.beta)
    for h in range(2):
        ST, O = chunked(q[:, 0], k[:, 0], v[:, h], g[:, h], b[:, h], erase, C,
                        widen(c.initial_state[0, h]))
        np.testing.assert_allclose(ST, S_ref[0, h], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(O, o_ref[:, h], rtol=1e-10, atol=1e-11)

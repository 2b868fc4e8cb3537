"""Pins of the group oracle (front end, short conv, gates, output path, group
driver) and of the anchor gather.

The pages do not write the layer internals out; the oracle takes the plainest
readings (unit-weight RMSNorm, conv over q|k|v channels, L2-normalised q/k,
log alpha = -softplus, beta = sigmoid, gated RMSNorm, no FFN).  What can be
pinned is that each step equals its textbook definition computed another way
(a library routine or a property), and that the group behaves as the pages
say: full-attention layers are skipped, each layer starts from zero state,
and a layer's state depends only on the layers before it ("SuffixReplay",
Algorithm Design 1; "Tail-Replay", section 3).
"""
import numpy as np
import pytest
from scipy import special

import oracle
from replay_inputs import (GDN, FA, _group, bf16_bits_to_f32, suffix_pool_case,
                           to_bf16_bits, widen)

RNG = np.random.default_rng(77)


# ---------------------------------------------------------------------------
# pointwise pieces against library routines and identities
# ---------------------------------------------------------------------------
def test_softplus_sigmoid_silu_against_library():
    x = np.concatenate([RNG.standard_normal(1000) * 8, [-800.0, -40, 0, 40, 800]])
    np.testing.assert_allclose(oracle.sigmoid(x), special.expit(x), rtol=1e-14,
                               atol=0)
    np.testing.assert_allclose(oracle.silu(x), x * special.expit(x), rtol=1e-14,
                               atol=1e-300)
    sp = oracle.softplus(x)
    # softplus(x) - softplus(-x) = x, softplus(0) = ln 2, d/dx softplus = sigmoid
    np.testing.assert_allclose(sp - oracle.softplus(-x), x, rtol=1e-13, atol=1e-13)
    assert oracle.softplus(np.array(0.0)) == pytest.approx(np.log(2.0), rel=1e-15)
    h = 1e-6
    xs = RNG.standard_normal(50)
    num = (oracle.softplus(xs + h) - oracle.softplus(xs - h)) / (2 * h)
    np.testing.assert_allclose(num, special.expit(xs), rtol=1e-8)
    assert np.all(np.isfinite(sp)) and np.all(sp >= 0)


def test_rmsnorm_and_l2norm_properties():
    x = RNG.standard_normal((20, 37)) * 3
    r = oracle.rmsnorm_rows(x, 0.0)
    np.testing.assert_allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm_rows(5.0 * x, 0.0), r, rtol=1e-14)
    # eps enters inside the root: mean square of the output = ms / (ms + eps)
    ms = np.mean(x * x, axis=1)
    re = oracle.rmsnorm_rows(x, 0.5)
    np.testing.assert_allclose(np.mean(re * re, axis=1), ms / (ms + 0.5), rtol=1e-13)
    l2 = oracle.l2norm_rows(x.reshape(20, 1, 37), 0.0)
    np.testing.assert_allclose(np.linalg.norm(l2, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(l2[:, 0] * np.linalg.norm(x, axis=1)[:, None], x,
                               rtol=1e-13)


@pytest.mark.parametrize("lens", [[7, 1, 2, 12], [3], [0, 5]])
def test_causal_conv_against_numpy_convolve(lens):
    C, W = 6, 4
    T = sum(lens)
    u = RNG.standard_normal((T, C))
    w = RNG.standard_normal((C, W))
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    y, state = oracle.causal_conv_silu(u, w, cu)
    for n, L in enumerate(lens):
        a = cu[n]
        if L == 0:
            np.testing.assert_array_equal(state[n], np.zeros((C, W - 1)))
            continue
        for c in range(C):
            # np.convolve(u, w[::-1]) puts tap W-1 on the current sample and
            # treats samples before the sequence start as zero
            ref = np.convolve(u[a:a + L, c], w[c, ::-1])[:L]
            np.testing.assert_allclose(y[a:a + L, c], special.expit(ref) * ref,
                                       rtol=1e-12, atol=1e-14)
            tail = np.concatenate([np.zeros(W - 1), u[a:a + L, c]])[-(W - 1):]
            np.testing.assert_array_equal(state[n, c], tail)


def test_output_path_properties():
    T, H, d, D = 5, 3, 8, 7
    o = RNG.standard_normal((T, H, d))
    z = RNG.standard_normal((T, H, d))
    w = to_bf16_bits(RNG.standard_normal((H * d, D)))
    y1 = oracle.output_path(o, z, w, 0.0)
    # the gated RMSNorm is per value head: scaling one head's o changes nothing
    o2 = o.copy()
    o2[:, 1] *= 7.0
    np.testing.assert_allclose(oracle.output_path(o2, z, w, 0.0), y1, rtol=1e-12)
    # SiLU(0) = 0 closes the gate
    np.testing.assert_array_equal(oracle.output_path(o, np.zeros_like(z), w, 0.0),
                                  np.zeros((T, D)))
    # the projection is the library matmul of the gated, normalised heads
    y = (o / np.sqrt(np.mean(o * o, -1, keepdims=True))) * special.expit(z) * z
    np.testing.assert_allclose(y1, y.reshape(T, -1) @ widen(w), rtol=1e-11,
                               atol=1e-12)


def _tiny_group(lens, kinds, seed=3, hidden=24, h_k=2, h_v=4, d=4):
    return _group(lens, seed, hidden, h_k, h_v, d, kinds)


def test_frontend_column_layout_and_gates():
    g = _tiny_group([6, 3], [GDN])
    w = g.weights[0]
    x = widen(g.anchors)
    fe = oracle.frontend(x, w.w_in, w.conv_w, g.cu_seqlens, 2, 4, 4)
    p = oracle.rmsnorm_rows(x, 1e-6) @ widen(w.w_in)
    np.testing.assert_allclose(fe["u"], p[:, :32], rtol=1e-14)
    np.testing.assert_allclose(fe["z"].reshape(9, -1), p[:, 32:48], rtol=1e-14)
    np.testing.assert_allclose(np.exp(fe["log_alpha"]),
                               special.expit(-p[:, 48:52]), rtol=1e-12)
    np.testing.assert_allclose(fe["beta"], special.expit(p[:, 52:56]), rtol=1e-14)
    assert np.all(fe["log_alpha"] < 0)
    # q and k are the conv outputs of their columns, L2-normalised per head
    # with eps inside the root: |q_hat|^2 = s / (s + eps), s = |q|^2
    for name, lo in (("q", 0), ("k", 8)):
        raw = fe["c"][:, lo:lo + 8].reshape(9, 2, 4)
        s_ = np.sum(raw * raw, -1)
        np.testing.assert_allclose(np.sum(fe[name] ** 2, -1), s_ / (s_ + 1e-6),
                                   rtol=1e-12)
        np.testing.assert_allclose(fe[name] * np.sqrt(s_ + 1e-6)[..., None], raw,
                                   rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(fe["v"].reshape(9, -1), fe["c"][:, 16:32])


def test_group_single_layer_is_frontend_then_recurrence():
    g = _tiny_group([9, 4], [GDN])
    S, conv = oracle.replay_group(g.anchors, g.weights, g.cu_seqlens, g.layer_kind,
                                  2, 4, 4)
    w = g.weights[0]
    fe = oracle.frontend(widen(g.anchors), w.w_in, w.conv_w, g.cu_seqlens, 2, 4, 4)
    S1, _ = oracle.gdn(fe["q"], fe["k"], fe["v"], fe["log_alpha"], fe["beta"],
                       g.cu_seqlens, 2, 4, alpha_is_log=True, want_o=False)
    np.testing.assert_array_equal(S[0], S1)
    np.testing.assert_array_equal(conv[0], fe["conv_state"])


def test_group_skips_full_attention_layers():
    base = _tiny_group([8, 5], [GDN, GDN, FA])
    S, _ = oracle.replay_group(base.anchors, base.weights, base.cu_seqlens,
                               base.layer_kind, 2, 4, 4)
    for kinds in ([GDN, GDN], [FA, GDN, GDN], [FA, GDN, GDN, FA]):
        S2, _ = oracle.replay_group(base.anchors, base.weights, base.cu_seqlens,
                                    kinds, 2, 4, 4)
        np.testing.assert_array_equal(S2, S)


def test_group_state_depends_only_on_earlier_layers():
    g = _tiny_group([10, 6], [GDN, GDN, GDN, FA])
    S, _ = oracle.replay_group(g.anchors, g.weights, g.cu_seqlens, g.layer_kind,
                               2, 4, 4)
    # the last layer's output projection is never used
    w = list(g.weights)
    w[2] = type(w[2])(w_in=w[2].w_in, conv_w=w[2].conv_w,
                      w_out=to_bf16_bits(RNG.standard_normal(w[2].w_out.shape)))
    S2, _ = oracle.replay_group(g.anchors, w, g.cu_seqlens, g.layer_kind, 2, 4, 4)
    np.testing.assert_array_equal(S2, S)
    # changing layer 2's output projection leaves layers 1-2 alone, moves layer 3
    w = list(g.weights)
    w[1] = type(w[1])(w_in=w[1].w_in, conv_w=w[1].conv_w,
                      w_out=to_bf16_bits(RNG.standard_normal(w[1].w_out.shape)))
    S3, _ = oracle.replay_group(g.anchors, w, g.cu_seqlens, g.layer_kind, 2, 4, 4)
    np.testing.assert_array_equal(S3[:2], S[:2])
    assert not np.allclose(S3[2], S[2])
    # the residual stream: layer 2 sees x + y W_out of layer 1
    _, _, tr = oracle.replay_group(g.anchors, g.weights, g.cu_seqlens,
                                   g.layer_kind, 2, 4, 4, return_trace=True)
    upd = oracle.output_path(tr[0]["o"], tr[0]["z"], g.weights[0].w_out)
    np.testing.assert_allclose(tr[1]["x"], tr[0]["x"] + upd, rtol=1e-14)
    assert tr[2]["o"] is None


def test_group_requests_are_independent():
    g = _tiny_group([7, 11, 3], [GDN, GDN])
    S, conv = oracle.replay_group(g.anchors, g.weights, g.cu_seqlens, g.layer_kind,
                                  2, 4, 4)
    cu = g.cu_seqlens
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        Sn, cn = oracle.replay_group(g.anchors[a:b], g.weights,
                                     np.array([0, b - a], np.int32), g.layer_kind,
                                     2, 4, 4)
        np.testing.assert_allclose(Sn[:, 0], S[:, n], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(cn[:, 0], conv[:, n], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# gather: brute force per token over the page table
# ---------------------------------------------------------------------------
def test_gather_against_token_loop():
    pc = suffix_pool_case(5, 70, 300, 0.05, 0.5, 16, seed=8, spare_pages=3)
    pool = pc.pool()
    packed, cu = oracle.gather_suffix(pool, pc.page_table, pc.matched_len,
                                      pc.suffix_len)
    row = 0
    for i in range(5):
        m, k = int(pc.matched_len[i]), int(pc.suffix_len[i])
        assert cu[i] == row
        for j in range(k):
            pos = m - k + j
            page = pc.page_table[i][pos // 64]
            assert np.array_equal(packed[row], pool[page, pos % 64])
            row += 1
    assert cu[-1] == row == packed.shape[0]


def test_pool_pages_are_independent_of_the_rest():
    pc = suffix_pool_case(3, 100, 200, 0.1, 0.2, 8, seed=4)
    full = pc.pool()
    np.testing.assert_array_equal(pc.pool_pages([2, 0]), full[[2, 0]])


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40])
    b = bf16_bits_to_f32(to_bf16_bits(x))
    assert b[0] == 1.0
    assert b[1] == 1.0                     # tie to even (down)
    assert b[2] == 1.0 + 2 ** -6           # tie to even (up)
    assert b[3] == -2.5
    assert np.isfinite(b[4])


# ---------------------------------------------------------------------------
# continuation from a carried-in state ("Tail-Replay", section 3: the
# unmatched tokens continue from the reconstructed states)
# ---------------------------------------------------------------------------
def test_causal_conv_with_history_against_numpy_convolve():
    """With a carried-in window the conv is np.convolve over history +
    sequence, and the returned window is the last W-1 rows of that."""
    rng = np.random.default_rng(5)
    W, C = 4, 3
    lens = [5, 1, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    u = rng.standard_normal((cu[-1], C))
    w = rng.standard_normal((C, W))
    hist = rng.standard_normal((len(lens), C, W - 1))
    y, st = oracle.causal_conv_silu(u, w, cu, hist)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        for c in range(C):
            seq = np.concatenate([hist[s, c], u[a:b, c]])
            # tap W-1 on the current sample; the history supplies the W-1
            # samples before the sequence start
            ref = np.convolve(seq, w[c, ::-1])[W - 1:W - 1 + (b - a)]
            np.testing.assert_allclose(y[a:b, c], special.expit(ref) * ref, rtol=1e-12,
                                       atol=1e-14)
            np.testing.assert_allclose(st[s, c], seq[-(W - 1):], rtol=0, atol=0)


def test_extend_group_equals_the_whole_run():
    """Replaying a prefix and extending it by the rest from the carried
    states and conv windows gives the states, windows and output hidden
    states of one run over the whole sequence (the state and the window
    summarise the prefix exactly)."""
    g = _group([23, 9, 40], 21, 16, 2, 4, 4, [GDN, GDN, GDN])
    cut = [10, 9, 1]
    cu = g.cu_seqlens
    pre_rows = np.concatenate([np.arange(cu[i], cu[i] + cut[i]) for i in range(3)])
    tail_rows = np.concatenate([np.arange(cu[i] + cut[i], cu[i + 1]) for i in range(3)])
    cu_pre = np.concatenate([[0], np.cumsum(cut)]).astype(np.int32)
    tail_lens = [int(cu[i + 1] - cu[i]) - cut[i] for i in range(3)]
    cu_tail = np.concatenate([[0], np.cumsum(tail_lens)]).astype(np.int32)
    S_full, C_full, H_full, _ = oracle.extend_group(g.anchors, g.weights, cu, g.layer_kind,
                                                    2, 4, 4)
    S_pre, C_pre = oracle.replay_group(g.anchors[pre_rows], g.weights, cu_pre, g.layer_kind,
                                       2, 4, 4)
    S_ext, C_ext, H_ext, _ = oracle.extend_group(g.anchors[tail_rows], g.weights, cu_tail,
                                                 g.layer_kind, 2, 4, 4, initial_states=S_pre,
                                                 initial_conv_states=C_pre)
    np.testing.assert_allclose(S_ext, S_full, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(C_ext, C_full, rtol=0, atol=0)
    np.testing.assert_allclose(H_ext, H_full[tail_rows], rtol=1e-10, atol=1e-12)
    # replay without the carried window (zero history) is a different result
    S_bad, _, _, _ = oracle.extend_group(g.anchors[tail_rows], g.weights, cu_tail, g.layer_kind,
                                         2, 4, 4, initial_states=S_pre)
    assert oracle.rel_fro(S_bad, S_full) > 1e-6


# ---------------------------------------------------------------------------
# FFN blocks between the group's GDN layers ("Tail-Replay", section 3: the
# group's final FFN is omitted from replay).  The pages give no FFN form; the
# SwiGLU block is a reading, pinned here only to its structure.
# ---------------------------------------------------------------------------
def test_ffn_block_structure():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 16))
    wg, wu = rng.standard_normal((16, 32)), rng.standard_normal((16, 32))
    wd = rng.standard_normal((32, 16))
    f = lambda a, b, c: oracle.ffn_block(x, a, b, c)
    np.testing.assert_array_equal(f(wg, wu, np.zeros_like(wd)), x)      # no down: identity
    np.testing.assert_array_equal(f(np.zeros_like(wg), wu, wd), x)      # SiLU(0) = 0
    # linear in the down projection, and the gate enters through SiLU
    np.testing.assert_allclose(f(wg, wu, 2 * wd) - x, 2 * (f(wg, wu, wd) - x), rtol=1e-12)
    xh = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)
    g, u = xh @ wg, xh @ wu
    np.testing.assert_allclose(f(wg, wu, wd), x + (special.expit(g) * g * u) @ wd, rtol=1e-12)


def test_group_ffn_only_reaches_later_layers():
    """An FFN after layer l changes the states of layers after l only, and
    the last layer's FFN changes no state at all (skipped in replay)."""
    g = _group([20, 7], 23, 16, 2, 4, 4, [GDN, GDN, GDN], ffn_dim=32)
    plain = _group([20, 7], 23, 16, 2, 4, 4, [GDN, GDN, GDN])
    S_f, _ = oracle.replay_group(g.anchors, g.weights, g.cu_seqlens, g.layer_kind, 2, 4, 4)
    S_p, _ = oracle.replay_group(plain.anchors, plain.weights, g.cu_seqlens, g.layer_kind, 2, 4, 4)
    np.testing.assert_array_equal(S_f[0], S_p[0])
    assert oracle.rel_fro(S_f[1], S_p[1]) > 1e-6 and oracle.rel_fro(S_f[2], S_p[2]) > 1e-6
    w_last = list(g.weights)
    w_last[2] = type(w_last[2])(**{**w_last[2].__dict__, "w_down": w_last[2].w_down * 0})
    S_l, _ = oracle.replay_group(g.anchors, w_last, g.cu_seqlens, g.layer_kind, 2, 4, 4)
    np.testing.assert_array_equal(S_l, S_f)

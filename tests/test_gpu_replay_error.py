"""Replay error of suffix replay against the full-prefix state (Eq. 1 vs
Eq. 2 of "SuffixReplay", Theoretical Foundation), computed on the GPU.

* kernel level: with the dropped prefix's state S_{n-k}, the error of the
  replayed state is bounded by (product of the replayed alphas) x
  |S_{n-k}|_F when 0 <= b |k|^2 <= 2, and equals it without the erase term;
* group level: the error shrinks as k grows, vanishes at k = m, and agrees
  with the fp64 oracle where it is large enough to be resolved.
"""
import math

import numpy as np
import pytest

import oracle
from replay_inputs import GDN, FA, _group, gdn_case, widen
from tests.util import rel_fro, to_dev, to_np

pytestmark = pytest.mark.gpu


def _gdn(c, a, b, s0=None):
    import torch
    import linear_attention_state_anchor_amd as sr
    S, _ = sr.gdn_replay_state(None, to_dev(c.k[a:b]), to_dev(c.v[a:b]),
                               to_dev(c.alpha[a:b]), None if c.beta is None else to_dev(c.beta[a:b]),
                               to_dev(np.array([0, b - a], np.int32)), s0,
                               erase=c.erase, alpha_is_log=c.alpha_is_log, want_o=False)
    torch.cuda.synchronize()
    return to_np(S)[0]


@pytest.mark.parametrize("erase", [True, False])
def test_replay_error_bound_on_gpu(erase):
    n, kk = 2000, 100
    c = gdn_case([n], 2, 4, 128, "bf16", seed=77, erase=erase,
                 alpha=("uniform", 0.98, 1.0))
    print(f"[replay-error] erase={erase}", flush=True)
    full = _gdn(c, 0, n)
    prefix = _gdn(c, 0, n - kk)
    replay = _gdn(c, n - kk, n)
    la = np.log(widen(c.alpha))
    for h in range(4):
        bound = np.exp(np.sum(la[n - kk:, h])) * np.linalg.norm(prefix[h])
        err = np.linalg.norm(full[h] - replay[h])
        noise = 1e-3 * np.linalg.norm(full[h])
        print(f"    head {h}: err {err:.4e} bound {bound:.4e}", flush=True)
        assert bound > 10 * noise
        if erase:
            assert err <= bound + noise
        else:
            assert abs(err - bound) <= noise


def test_group_error_shrinks_with_k_and_matches_oracle():
    import torch
    import linear_attention_state_anchor_amd as sr
    g = _group([700, 500], 91, 256, 2, 4, 128, [GDN, GDN, FA])
    print("[replay-error] group", flush=True)
    packed = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 2, 4, 128)
              for w in g.weights]
    cu = g.cu_seqlens

    def suffix_states(k):
        rows = np.concatenate([np.arange(cu[i + 1] - min(k, cu[i + 1] - cu[i]), cu[i + 1])
                               for i in range(2)])
        lens = [min(k, int(cu[i + 1] - cu[i])) for i in range(2)]
        cuk = np.zeros(3, np.int32)
        cuk[1:] = np.cumsum(lens)
        S = sr.replay_group(to_dev(g.anchors[rows]), packed, to_dev(cuk), g.layer_kind, 2, 4, 128)
        torch.cuda.synchronize()
        return to_np(S), g.anchors[rows], cuk

    full, _, _ = suffix_states(10 ** 6)
    errs = []
    for k in (8, 16, 64, 256, 1000):
        S, anc, cuk = suffix_states(k)
        e = [rel_fro(S[l], full[l]) for l in range(2)]
        errs.append(e)
        print(f"    k={k}: rel err per layer {e}", flush=True)
        if k == 8:
            # the oracle sees the same effect at the same size
            Sr_full, _ = oracle.replay_group(g.anchors, g.weights, cu, g.layer_kind, 2, 4, 128)
            Sr_k, _ = oracle.replay_group(anc, g.weights, cuk, g.layer_kind, 2, 4, 128)
            for l in range(2):
                er = rel_fro(Sr_k[l], Sr_full[l])
                print(f"      oracle layer {l}: {er:.4e}", flush=True)
                assert abs(e[l] - er) <= 0.1 * er + 3e-3
    errs = np.array(errs)
    assert np.all(errs[-1] == 0.0)           # k >= m: the same replay
    for l in range(2):
        assert errs[0, l] > errs[2, l]       # longer suffix, smaller error


@pytest.mark.parametrize("erase", [True, False])
def test_slow_decay_error_vs_k_matches_oracle(erase):
    """alpha ~ U[0.90, 0.999] (slow forgetting): the replay error falls from
    tens of percent at k = 16 to the rounding floor at k = 256.  The GPU's
    error at each k matches the oracle's (fp64) error."""
    import torch
    import linear_attention_state_anchor_amd as sr
    m, ks = 2048, (16, 64, 256)
    c = gdn_case([m, m], 2, 4, 128, "bf16", seed=78, alpha=("uniform", 0.90, 0.999),
                 normalize_k=erase, beta="sigmoid" if erase else "none", erase=erase)
    print(f"[replay-error] slow decay erase={erase}", flush=True)

    def rows(lo):
        return np.concatenate([np.arange(i * m + lo, (i + 1) * m) for i in range(2)])

    def cu(L):
        return np.array([0, L, 2 * L], np.int32)

    def gpu(lo):
        r = rows(lo)
        S, _ = sr.gdn_replay_state(None, to_dev(c.k[r]), to_dev(c.v[r]), to_dev(c.alpha[r]),
                                   None if c.beta is None else to_dev(c.beta[r]),
                                   to_dev(cu(m - lo)), erase=erase, want_o=False)
        torch.cuda.synchronize()
        return to_np(S)

    def orc(lo):
        r = rows(lo)
        S, _ = oracle.gdn(None, c.k[r], c.v[r], c.alpha[r], None if c.beta is None else c.beta[r],
                          cu(m - lo), 2, 4, alpha_is_log=False, erase=erase, want_o=False)
        return S

    full_g, full_o = gpu(0), orc(0)
    prev = None
    for k in ks:
        eg = rel_fro(gpu(m - k), full_g)
        eo = rel_fro(orc(m - k), full_o)
        print(f"    k={k}: gpu {eg:.4e} oracle {eo:.4e}", flush=True)
        assert abs(eg - eo) <= 0.05 * eo + 3e-3
        if prev is not None:
            assert eo < prev
        prev = eo
    assert rel_fro(orc(m - 16), full_o) > 0.05     # slow forgetting: k = 16 is far off


def test_varlen_group_error_vs_k_two_requests_matches_oracle():
    """Two hits of the 64-hit varlen workload (the two shortest prefixes, to
    keep the fp64 full-prefix replay short): GPU and oracle replay errors at
    k = 16, 64 and ceil(0.05 m) against the full-prefix states of the group."""
    import torch
    import linear_attention_state_anchor_amd as sr
    from replay_inputs import PAGE, config_c5
    pc, wts = config_c5()
    sel = list(np.argsort(pc.matched_len)[:2])
    print(f"[replay-error] varlen requests {sel} m={[int(pc.matched_len[i]) for i in sel]}",
          flush=True)
    packed = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32, 128)
              for w in wts]
    kinds = [GDN, GDN, GDN, FA]
    rng = np.random.default_rng(9)
    m = [int(pc.matched_len[i]) for i in sel]
    # the two prefixes' anchors (bf16 ~ N(0,1)), page structure irrelevant here
    prefixes = [pc.pool_pages(pc.page_table[i][:(mi + PAGE - 1) // PAGE]).reshape(-1, 2560)[:mi]
                for i, mi in zip(sel, m)]

    def run(klist):
        parts = [p[len(p) - k:] for p, k in zip(prefixes, klist)]
        a = np.concatenate(parts)
        cu = np.concatenate([[0], np.cumsum(klist)]).astype(np.int32)
        S = sr.replay_group(to_dev(a), packed, to_dev(cu), kinds, 16, 32, 128)
        torch.cuda.synchronize()
        Sr, _ = oracle.replay_group(a, wts, cu, kinds, 16, 32, 128)
        return to_np(S), Sr

    full_g, full_o = run(m)
    for label, klist in (("16", [16, 16]), ("64", [64, 64]),
                         ("ceil(0.05m)", [int(np.ceil(0.05 * x)) for x in m])):
        Sg, So = run(klist)
        for l in range(3):
            eg, eo = rel_fro(Sg[l], full_g[l]), rel_fro(So[l], full_o[l])
            print(f"    k={label} layer {l}: gpu {eg:.4e} oracle {eo:.4e}", flush=True)
            assert abs(eg - eo) <= 0.1 * eo + 3e-3

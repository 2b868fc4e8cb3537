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

"""Continuation from a reconstructed state ("Tail-Replay", section 3: the
unmatched tokens continue from the reconstructed linear-attention states),
on the GPU against the fp64 oracle run over the whole sequence:

* single-token decode steps (sr_gdn_decode_step) after a chunked replay of
  the prefix: states and outputs;
* a group extended over new tokens (sr_extend_group) from the states and
  conv windows a prefix replay (sr_replay_group) returned: states, conv
  windows and the group's output hidden states.
"""
import numpy as np
import pytest

import oracle
from replay_inputs import FA, GDN, GroupCase, _group, gdn_case
from tests.util import rel_fro, to_dev, to_np

pytestmark = pytest.mark.gpu

N_DECODE = 6


@pytest.mark.parametrize("dtype,d,erase", [("bf16", 128, True), ("bf16", 128, False),
                                           ("bf16", 64, True), ("f32", 64, True)])
def test_decode_steps_continue_the_replay(dtype, d, erase):
    import torch
    import linear_attention_state_anchor_amd as sr
    print(f"[continue] decode dtype={dtype} d={d} erase={erase}", flush=True)
    prefix = [300, 64, 1, 0, 129]
    lens = [p + N_DECODE for p in prefix]
    c = gdn_case(lens, 2, 4, d, dtype, seed=81 + d + int(erase), normalize_q=True, erase=erase,
                 initial_state=True)
    cu = c.cu_seqlens
    n = len(lens)
    pre = np.concatenate([np.arange(cu[i], cu[i] + prefix[i]) for i in range(n)])
    cu_pre = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int32)
    beta = lambda rows: None if c.beta is None else to_dev(c.beta[rows])
    S, _ = sr.gdn_replay_state(None, to_dev(c.k[pre]), to_dev(c.v[pre]), to_dev(c.alpha[pre]),
                               beta(pre), to_dev(cu_pre), to_dev(c.initial_state), erase=erase,
                               alpha_is_log=c.alpha_is_log, want_o=False)
    S_copy = S.clone()
    outs = []
    for j in range(N_DECODE):
        rows = np.array([cu[i] + prefix[i] + j for i in range(n)])
        S, o = sr.gdn_decode_step(to_dev(c.q[rows]), to_dev(c.k[rows]), to_dev(c.v[rows]),
                                  to_dev(c.alpha[rows]), beta(rows), S, erase=erase,
                                  alpha_is_log=c.alpha_is_log, o_dtype=torch.float32)
        outs.append(o)
    torch.cuda.synchronize()
    Sr, orf = oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, cu, c.h_k, c.h_v,
                         alpha_is_log=c.alpha_is_log, erase=erase,
                         initial_state=c.initial_state)
    o_gpu = np.stack([to_np(o) for o in outs], axis=1)          # [n][N_DECODE][h_v][d]
    o_ref = np.stack([orf[cu[i] + prefix[i]:cu[i + 1]] for i in range(n)])
    tol = 1e-5 if dtype == "f32" else 2e-3
    es, eo = rel_fro(to_np(S), Sr), rel_fro(o_gpu, o_ref)
    print(f"    rel S {es:.3e} rel o {eo:.3e}", flush=True)
    assert es <= tol and eo <= tol
    # an out-of-place step equals the in-place one
    rows = np.array([cu[i] + prefix[i] for i in range(n)])
    S2 = torch.empty_like(S_copy)
    sr.gdn_decode_step(to_dev(c.q[rows]), to_dev(c.k[rows]), to_dev(c.v[rows]),
                       to_dev(c.alpha[rows]), beta(rows), S_copy, erase=erase,
                       alpha_is_log=c.alpha_is_log, out_state=S2, want_o=False)
    S3 = S_copy.clone()
    sr.gdn_decode_step(to_dev(c.q[rows]), to_dev(c.k[rows]), to_dev(c.v[rows]),
                       to_dev(c.alpha[rows]), beta(rows), S3, erase=erase,
                       alpha_is_log=c.alpha_is_log, want_o=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(S2), to_np(S3))


def test_decode_from_zero_state_is_one_token_replay():
    """From S = 0 one decode step is the single-token closed form S = b v k^T,
    o = b (k.q) v, which the oracle gives too."""
    import torch
    import linear_attention_state_anchor_amd as sr
    c = gdn_case([1] * 7, 2, 4, 128, "bf16", seed=85, normalize_q=True)
    S, o = sr.gdn_decode_step(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.alpha),
                              to_dev(c.beta), None, alpha_is_log=True, o_dtype=torch.float32)
    torch.cuda.synchronize()
    Sr, orf = oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, 2, 4, alpha_is_log=True)
    assert rel_fro(to_np(S), Sr) < 1e-6 and rel_fro(to_np(o), orf) < 1e-6


def _split(g, cut):
    cu = g.cu_seqlens
    n = len(cut)
    pre = np.concatenate([np.arange(cu[i], cu[i] + cut[i]) for i in range(n)])
    tail = np.concatenate([np.arange(cu[i] + cut[i], cu[i + 1]) for i in range(n)])
    cu_pre = np.concatenate([[0], np.cumsum(cut)]).astype(np.int32)
    tl = [int(cu[i + 1] - cu[i]) - cut[i] for i in range(n)]
    cu_tail = np.concatenate([[0], np.cumsum(tl)]).astype(np.int32)
    return pre, tail, cu_pre, cu_tail


@pytest.mark.parametrize("hidden,hk,hv,d,F", [(256, 2, 4, 128, 0), (256, 2, 4, 64, 0),
                                               (2560, 16, 32, 128, 0), (256, 2, 4, 128, 320)])
def test_extend_group_continues_the_replay(hidden, hk, hv, d, F):
    """Also with FFN blocks (F > 0): the last layer's FFN, skipped by the
    prefix replay, runs in the extension, whose output includes it."""
    import torch
    import linear_attention_state_anchor_amd as sr
    print(f"[continue] group hidden={hidden} hk={hk} hv={hv} d={d} ffn={F}", flush=True)
    lens = [300, 70, 65, 2]
    cut = [200, 1, 64, 2]              # the last request has no new tokens
    g = _group(lens, 91 + d, hidden, hk, hv, d, [GDN, GDN, GDN, FA], ffn_dim=F)
    packed = []
    for w in g.weights:
        mix = sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), hk, hv, d)
        packed.append((mix, sr.pack_ffn(to_dev(w.w_gate), to_dev(w.w_up), to_dev(w.w_down)))
                      if F else mix)
    pre, tail, cu_pre, cu_tail = _split(g, cut)
    S_pre, C_pre = sr.replay_group(to_dev(g.anchors[pre]), packed, to_dev(cu_pre), g.layer_kind,
                                   hk, hv, d, want_conv_state=True, ffn_dim=F)
    S, C, H = sr.extend_group(to_dev(g.anchors[tail]), packed, to_dev(cu_tail), g.layer_kind,
                              hk, hv, d, initial_states=S_pre, initial_conv_states=C_pre,
                              ffn_dim=F)
    torch.cuda.synchronize()
    Sr, Cr, Hr, _ = oracle.extend_group(g.anchors, g.weights, g.cu_seqlens, g.layer_kind,
                                        hk, hv, d)
    for li in range(3):
        e, ec = rel_fro(to_np(S[li]), Sr[li]), rel_fro(to_np(C[li]), Cr[li])
        print(f"    layer {li}: rel state {e:.3e} conv {ec:.3e}", flush=True)
        assert e <= 2e-3 and ec <= 2e-3
    eh = rel_fro(to_np(H), Hr[tail])
    print(f"    rel hidden out {eh:.3e}", flush=True)
    assert eh <= 2e-3
    assert np.all(np.isfinite(to_np(S)))

"""GPU parity of the gated-delta-rule replay (sr_gdn_replay_state) against
the fp64 oracle, element by element on the same seeded inputs.

Tolerances (relative Frobenius error over each whole output tensor):
  * 2e-3 for bf16 / fp16 inputs (states and outputs);
  * 1e-5 for fp32 inputs (token-serial fp32 kernel).
Emitting o in bf16 alone costs about 1.7e-3 of the 2e-3 (one round to
nearest of a 7-bit mantissa); fp32 outputs are checked to 5e-4.
"""
import numpy as np
import pytest

import oracle
from replay_inputs import config_c1, config_c2, config_c3, gdn_case
from tests.util import rel_fro, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
TOL_F32_IN = 1e-5


def gpu_run(c, want_o=True, o_dtype=None):
    import torch
    import linear_attention_state_anchor_amd as sr
    print(f"[gdn] {c.meta.get('name', '')} lens={c.meta.get('lens', '')[:8]} "
          f"hk={c.h_k} hv={c.h_v} d={c.d_k} erase={c.erase}", flush=True)
    s0 = None if c.initial_state is None else to_dev(c.initial_state)
    S, o = sr.gdn_replay_state(
        to_dev(c.q) if want_o else None, to_dev(c.k), to_dev(c.v), to_dev(c.alpha),
        None if c.beta is None else to_dev(c.beta), to_dev(c.cu_seqlens), s0,
        erase=c.erase, alpha_is_log=c.alpha_is_log, want_o=want_o, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return to_np(S), (None if o is None else to_np(o))


def oracle_run(c, want_o=True):
    return oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, c.h_k, c.h_v,
                      alpha_is_log=c.alpha_is_log, erase=c.erase,
                      initial_state=c.initial_state, want_o=want_o)


def check(c, tol, want_o=True, o_dtype=None, o_tol=None):
    S, o = gpu_run(c, want_o, o_dtype)
    Sr, orf = oracle_run(c, want_o)
    es = rel_fro(S, Sr)
    print(f"    rel S {es:.3e}", flush=True)
    assert es <= tol, es
    if want_o:
        eo = rel_fro(o, orf)
        print(f"    rel o {eo:.3e}", flush=True)
        assert eo <= (tol if o_tol is None else o_tol), eo
    return S, o, Sr, orf


def test_fp32_single_sequence_config():
    """1 sequence x 256 tokens, 4 heads, d = 64, fp32 (token-serial kernel)."""
    check(config_c1(), TOL_F32_IN)


@pytest.mark.parametrize("erase", [True, False])
def test_fp32_varlen_heads(erase):
    c = gdn_case([5, 0, 130, 64], 2, 4, 32, "f32", seed=7, erase=erase, d_v=64,
                 initial_state=True)
    check(c, TOL_F32_IN)


def test_erase_free_bf16_small():
    """Scalar-decay replay, bf16, alpha ~ U[0.90, 0.999], beta = 1."""
    check(config_c2(n_seqs=2, seqlen=2048, heads=4), TOL_BF16)


def test_gdn_bf16_small():
    """Gated delta rule, bf16, 16 key / 32 value head layout at reduced count."""
    c = gdn_case([3276, 700], 2, 4, 128, "bf16", seed=103, normalize_q=True,
                 normalize_k=True)
    check(c, TOL_BF16)


# 16 ragged sequences (empty, single-token, chunk-boundary and multi-chunk)
PAIR_LENS = [0, 1, 63, 64, 65, 127, 128, 129, 200, 17, 3, 90, 150, 64, 31, 70]


@pytest.mark.parametrize("d,hk", [(64, 16), (128, 16), (128, 8)])
@pytest.mark.parametrize("erase", [True, False])
def test_value_head_pairs(d, hk, erase):
    """16 ragged sequences x 32 value heads sharing 16 (or 8) key heads: 512
    (sequence, head) chains, enough for the launch to put two value heads of
    a key head in one workgroup.  Full parity of states and outputs (with an
    initial state), and the state-only run equals the full run bit for bit."""
    c = gdn_case(PAIR_LENS, hk, 32, d, "bf16", seed=31 + d + hk + int(erase), normalize_q=True,
                 erase=erase, initial_state=True)
    S, _, _, _ = check(c, TOL_BF16)
    S2, o2 = gpu_run(c, want_o=False)
    assert o2 is None
    np.testing.assert_array_equal(S, S2)


@pytest.mark.parametrize("n_seqs,hk,hv", [(16, 32, 32), (12, 16, 32), (4, 16, 32)])
@pytest.mark.parametrize("erase", [True, False])
def test_launch_shapes(n_seqs, hk, hv, erase):
    """The launch picks its workgroup shape from the number of (sequence,
    value head) chains: 512 chains with one value head per key head and 384
    chains take one head of 4 waves per workgroup, 128 chains one head of 8
    waves (pairs of heads are covered above).  Full parity with ragged
    lengths and an initial state, and state-only equals the full run."""
    lens = (PAIR_LENS * 2)[:n_seqs]
    c = gdn_case(lens, hk, hv, 128, "bf16", seed=7 * n_seqs + hk + int(erase), normalize_q=True,
                 erase=erase, initial_state=True)
    S, _, _, _ = check(c, TOL_BF16)
    S2, o2 = gpu_run(c, want_o=False)
    assert o2 is None
    np.testing.assert_array_equal(S, S2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("hk,hv", [(1, 1), (1, 2), (2, 4)])
def test_edge_lengths(d, erase, hk, hv):
    lens = [0, 1, 2, 63, 64, 65, 127, 128, 129, 200]
    c = gdn_case(lens, hk, hv, d, "bf16", seed=d + hk * 10 + hv, erase=erase,
                 normalize_q=True, normalize_k=True)
    check(c, TOL_BF16)


def test_initial_state_and_empty_sequence():
    c = gdn_case([70, 0, 3], 1, 2, 128, "bf16", seed=17, normalize_q=True,
                 initial_state=True)
    S, _, Sr, _ = check(c, TOL_BF16)
    np.testing.assert_array_equal(S[1], c.initial_state[1])


def test_beta_zero_is_pure_decay_on_gpu():
    c = gdn_case([100], 1, 1, 128, "bf16", seed=19, beta="zero", initial_state=True)
    S, _ = gpu_run(c, want_o=False)
    decay = np.exp(np.sum(c.alpha[:, 0].astype(np.float64)))
    assert rel_fro(S[0, 0], decay * c.initial_state[0, 0].astype(np.float64)) < 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_state_only_matches_full_run(d, dtype):
    """State-only replay (the last layer of a group) equals the state of the
    full run bit for bit and matches the oracle, for sequences whose last
    chunk is full (64, 128) as well as ragged ones."""
    c = gdn_case([300, 77, 64, 128], 2, 4, d, "bf16", seed=23, normalize_q=True)
    if dtype == "f16":   # the same values stored as fp16 (bf16 -> fp16 is exact here)
        f16 = lambda x: ((x.astype(np.uint32) << 16).view(np.float32)).astype(np.float16)
        c.q, c.k, c.v = f16(c.q), f16(c.k), f16(c.v)
    S1, _ = gpu_run(c, want_o=True)
    S2, o2 = gpu_run(c, want_o=False)
    assert o2 is None
    np.testing.assert_array_equal(S1, S2)
    Sr, _ = oracle_run(c, want_o=False)
    assert rel_fro(S2, Sr) <= TOL_BF16


@pytest.mark.parametrize("o_dtype", ["f32", "f16"])
def test_output_dtypes(o_dtype):
    import torch
    dt = {"f32": torch.float32, "f16": torch.float16}[o_dtype]
    c = gdn_case([500, 129], 2, 4, 128, "bf16", seed=29, normalize_q=True)
    # with an fp32 or fp16 output the final rounding no longer dominates
    check(c, TOL_BF16, o_dtype=dt, o_tol=5e-4)


@pytest.mark.parametrize("d", [64, 128])
def test_output_scale(d):
    """o_t = scale * S_t q_t with a non-unit scale (1/sqrt(d), as attention
    scales queries); fp32 outputs so the scale's effect is not hidden by the
    final rounding; the state does not depend on it."""
    import torch
    import linear_attention_state_anchor_amd as sr
    c = gdn_case([200, 64, 77], 2, 4, d, "bf16", seed=41, normalize_q=True)
    scale = d ** -0.5
    S, o = sr.gdn_replay_state(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.alpha),
                               to_dev(c.beta), to_dev(c.cu_seqlens), None, erase=True,
                               alpha_is_log=c.alpha_is_log, scale=scale, o_dtype=torch.float32)
    torch.cuda.synchronize()
    Sr, orf = oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, c.h_k, c.h_v,
                         alpha_is_log=c.alpha_is_log, erase=True, scale=scale)
    es, eo = rel_fro(to_np(S), Sr), rel_fro(to_np(o), orf)
    print(f"    scale {scale:.4f}: rel S {es:.3e} rel o {eo:.3e}", flush=True)
    assert es <= TOL_BF16 and eo <= 5e-4, (es, eo)


def test_fp16_inputs():
    c = gdn_case([400, 33], 1, 2, 128, "bf16", seed=31, normalize_q=True)
    # the same values as fp16 storage (bf16 -> fp16 is exact here)
    f16 = lambda x: ((x.astype(np.uint32) << 16).view(np.float32)).astype(np.float16)
    c16 = gdn_case([400, 33], 1, 2, 128, "bf16", seed=31, normalize_q=True)
    c16.q, c16.k, c16.v = f16(c.q), f16(c.k), f16(c.v)
    S_b, o_b = gpu_run(c)
    S_h, o_h = gpu_run(c16)
    np.testing.assert_array_equal(S_b, S_h)
    check(c16, TOL_BF16)


def test_deterministic_and_packed_equals_solo():
    lens = [190, 64, 1, 257]
    c = gdn_case(lens, 2, 4, 128, "bf16", seed=37, normalize_q=True)
    S1, o1 = gpu_run(c)
    S2, o2 = gpu_run(c)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(o1, o2)
    cu = c.cu_seqlens
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        solo = gdn_case([lens[n]], 2, 4, 128, "bf16", seed=0)
        solo.q, solo.k, solo.v = c.q[a:b], c.k[a:b], c.v[a:b]
        solo.alpha, solo.beta = c.alpha[a:b], c.beta[a:b]
        Sn, on = gpu_run(solo)
        np.testing.assert_array_equal(Sn[0], S1[n])
        np.testing.assert_array_equal(on, o1[a:b])


def test_unnormalised_keys_bf16():
    # keys not normalised: |k|^2 ~ 128, beta small enough that the erase stays
    # a contraction (0 <= beta |k|^2 <= 2)
    c = gdn_case([300], 1, 2, 128, "bf16", seed=41, normalize_k=False,
                 normalize_q=False)
    c.beta = (c.beta * np.float32(1.0 / 128)).astype(np.float32)
    check(c, TOL_BF16)


# ---------------------------------------------------------------------------
# full-size workloads in the launch configuration the benchmark times; the
# oracle checks a sample of whole sequences
# ---------------------------------------------------------------------------
def _sampled(c, seqs, want_o=True):
    cu = c.cu_seqlens
    sub = gdn_case([int(cu[s + 1] - cu[s]) for s in seqs], c.h_k, c.h_v, c.d_k, c.dtype,
                   seed=0, erase=c.erase)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    sub.q, sub.k, sub.v = c.q[idx], c.k[idx], c.v[idx]
    sub.alpha = c.alpha[idx]
    sub.beta = None if c.beta is None else c.beta[idx]
    sub.alpha_is_log = c.alpha_is_log
    return sub, idx


@pytest.mark.parametrize("which", ["gdn", "erase_free"])
def test_full_size_sampled(which):
    c = config_c3() if which == "gdn" else config_c2()
    S, o = gpu_run(c)
    seqs = [0, c.n_seqs - 1]
    sub, idx = _sampled(c, seqs)
    Sr, orf = oracle_run(sub)
    es = rel_fro(S[seqs], Sr)
    eo = rel_fro(o[idx], orf)
    print(f"    sampled rel S {es:.3e} rel o {eo:.3e}", flush=True)
    assert es <= TOL_BF16 and eo <= TOL_BF16
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(o))

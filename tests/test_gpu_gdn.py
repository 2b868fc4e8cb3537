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


@pytest.mark.parametrize("n_seqs,hk,hv", [(16, 32, 32), (12, 16, 32), (8, 16, 32),
                                          (4, 16, 32)])
@pytest.mark.parametrize("erase", [True, False])
def test_launch_shapes(n_seqs, hk, hv, erase):
    """The launch picks its workgroup shape from the number of (sequence,
    value head) chains: 512 chains with one value head per key head and 384
    chains take one head of 4 waves per workgroup; 256 chains one head of 8
    consumer waves beside 4 producer waves (which stage and tile the next
    chunk); 128 chains two workgroups per chain (value columns split), each
    4 consumer and 4 producer waves (pairs of heads are covered above).  Full
    parity with ragged lengths and an initial state, and state-only equals
    the full run."""
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


@pytest.mark.parametrize("keys", ["identical", "near"])
def test_repeated_keys_within_blocks(keys):
    """Keys repeated (or nearly) over runs of 16 tokens with beta = 1 and slow
    decay (alpha ~ U[0.90, 0.999]): the diagonal blocks of I + A are then
    close to all-ones lower triangles, the hardest case for the blocked
    inverse (its series terms are largest there; with identical keys and
    alpha = 1 the exact inverse is bidiagonal).  (With alpha = 1 exactly
    nothing is forgotten and the fp16 operand rounding of every chunk
    accumulates: 1.8e-3 on the state after 1000 tokens, growing with the
    length; the decaying gates of the workloads keep it at the per-chunk
    level.)"""
    from replay_inputs import to_bf16_bits
    c = gdn_case([1000, 130, 63], 2, 4, 128, "bf16", seed=43, alpha=("uniform", 0.90, 0.999),
                 beta="one", normalize_q=True)
    rng = np.random.default_rng(44)
    T = int(c.cu_seqlens[-1])
    base = rng.standard_normal((T // 16 + 1, c.h_k, 128))
    kf = base[np.arange(T) // 16]
    if keys == "near":
        kf = kf + 0.05 * rng.standard_normal(kf.shape)
    kf /= np.linalg.norm(kf, axis=-1, keepdims=True)
    c.k = to_bf16_bits(kf)
    check(c, TOL_BF16)


# ---------------------------------------------------------------------------
# full-size workloads in the launch configuration the benchmark times,
# compared with the oracle on every sequence and head
# ---------------------------------------------------------------------------
def worst_per_head(x, ref, idx_fn):
    """Largest relative Frobenius error over the (sequence, head) blocks that
    idx_fn(n, h) selects from x and ref."""
    worst, at = 0.0, None
    for key, sel in idx_fn():
        e = rel_fro(x[sel], ref[sel])
        if e > worst:
            worst, at = e, key
    return worst, at


def state_blocks(c):
    return lambda: (((n, h), (n, h)) for n in range(c.n_seqs) for h in range(c.h_v))


def output_blocks(c):
    cu = c.cu_seqlens
    return lambda: (((n, h), (slice(int(cu[n]), int(cu[n + 1])), h))
                    for n in range(c.n_seqs) for h in range(c.h_v) if cu[n + 1] > cu[n])


@pytest.mark.parametrize("which", ["gdn_16x3276", "erase_free_8x2048"])
def test_full_size_every_sequence(which):
    """16 x 3276 tokens, 16 key / 32 value heads (the benchmarked replay) and
    8 x 2048 tokens, 32 heads, scalar decay: states and outputs of every
    sequence and head against the oracle."""
    c = config_c3() if which == "gdn_16x3276" else config_c2()
    S, o, Sr, orf = check(c, TOL_BF16)
    ws, at_s = worst_per_head(S, Sr, state_blocks(c))
    wo, at_o = worst_per_head(o, orf, output_blocks(c))
    print(f"    worst (sequence, head): state {ws:.3e} at {at_s}, output {wo:.3e} at {at_o}",
          flush=True)
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(o))
    # every block on its own stays near the whole-tensor figure
    assert ws <= 2 * TOL_BF16 and wo <= 2 * TOL_BF16


@pytest.mark.parametrize("n_seqs", [16, 9, 8])
def test_packed_equals_solo_across_launch_shapes(n_seqs):
    """16 sequences x 32 value heads (512 chains: value-head pairs per
    workgroup), 9 x 32 (288 chains: one head of 4 waves) and 8 x 32 (256
    chains: 8 consumer and 4 producer waves) against each sequence replayed
    alone (32 chains: two producer/consumer workgroups per chain): bit-identical states and
    outputs, so no result depends on the launch shape or on a sequence's
    neighbours."""
    lens = (PAIR_LENS * 2)[:n_seqs]
    c = gdn_case(lens, 16, 32, 128, "bf16", seed=60 + n_seqs, normalize_q=True,
                 initial_state=True)
    S, o = gpu_run(c)
    cu = c.cu_seqlens
    for n in range(n_seqs):
        a, b = int(cu[n]), int(cu[n + 1])
        solo = gdn_case([b - a], 16, 32, 128, "bf16", seed=0)
        solo.q, solo.k, solo.v = c.q[a:b], c.k[a:b], c.v[a:b]
        solo.alpha, solo.beta = c.alpha[a:b], c.beta[a:b]
        solo.initial_state = c.initial_state[n:n + 1]
        Sn, on = gpu_run(solo)
        np.testing.assert_array_equal(Sn[0], S[n])
        np.testing.assert_array_equal(on, o[a:b])


# ---------------------------------------------------------------------------
# states beyond the fp16 range: the kernel's fp16 matrix-core copies of the
# state and of U are kept in range by a per-wave power-of-two exponent, so
# the replay holds for a state of any fp32 magnitude ("SuffixReplay", Eq. 4
# iterates from an arbitrary S)
# ---------------------------------------------------------------------------
def _large_state_case(which):
    from replay_inputs import to_bf16_bits, widen
    if which == "initial_1e5_fast_decay":
        # |S_0| ~ 1e5 decays away within a few chunks (mean alpha ~ 0.5): the
        # exponent rises at the first chunk and returns to zero
        c = gdn_case([300, 64, 1, 0], 2, 4, 128, "bf16", seed=51, normalize_q=True,
                     initial_state=True)
        c.initial_state = (c.initial_state * np.float32(1e5)).astype(np.float32)
    elif which == "initial_1e5_slow_decay":
        # alpha in [0.999, 1]: the state stays near 1e5 for the whole replay
        c = gdn_case([700, 129], 2, 4, 128, "bf16", seed=52, normalize_q=True,
                     alpha=("uniform", 0.999, 1.0), initial_state=True)
        c.initial_state = (c.initial_state * np.float32(1e5)).astype(np.float32)
    elif which == "erase_free_scaled_v":
        # scalar decay alpha in [0.999, 1], keys ~ N(0,1) (|k|^2 ~ 128) and
        # values x 1000: the state grows to ~1e5 and beyond from S_0 = 0
        c = gdn_case([2048, 700], 4, 4, 128, "bf16", seed=53, normalize_k=False,
                     alpha=("uniform", 0.999, 1.0), beta="none", erase=False)
        c.v = to_bf16_bits(widen(c.v) * 1000.0)
    else:
        raise ValueError(which)
    c.meta["name"] = which
    return c


@pytest.mark.parametrize("which", ["initial_1e5_fast_decay", "initial_1e5_slow_decay",
                                   "erase_free_scaled_v"])
def test_state_beyond_fp16_range(which):
    c = _large_state_case(which)
    S, o, Sr, orf = check(c, TOL_BF16)
    peak = float(np.max(np.abs(Sr)))
    print(f"    max |S_T| {peak:.3e}", flush=True)
    assert peak > 65504.0                # the case really leaves fp16's range
    assert np.all(np.isfinite(S)) and np.all(np.isfinite(o))
    S2, _ = gpu_run(c, want_o=False)
    np.testing.assert_array_equal(S, S2)


# ---------------------------------------------------------------------------
# device-side precondition checks (sr_check_replay_inputs and the SR_DEBUG
# path); the bad inputs only ever reach the validation kernels
# ---------------------------------------------------------------------------
def test_check_replay_inputs_flags_bad_data():
    import linear_attention_state_anchor_amd as sr
    print("[gdn] precondition checks", flush=True)
    c = gdn_case([50, 0, 70], 1, 2, 64, "bf16", seed=71)
    q, k, v, b = to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.beta)

    def run(alpha, cu, beta=b, log=True):
        sr.check_replay_inputs(q, k, v, to_dev(alpha), beta, to_dev(cu), alpha_is_log=log)

    run(c.alpha, c.cu_seqlens)                                  # valid
    run(np.exp(c.alpha), c.cu_seqlens, log=False)               # the same gates as alpha
    for cu in ([0, 60, 50, 120], [0, 50, 50, 119], [1, 50, 50, 120]):
        with pytest.raises(ValueError):
            run(c.alpha, np.asarray(cu, np.int32))
    for val, log in ((0.5, True), (np.nan, True), (1.5, False), (0.0, False), (np.nan, False)):
        a = (c.alpha if log else np.exp(c.alpha)).copy()
        a[77, 1] = val
        with pytest.raises(ValueError):
            run(a.astype(np.float32), c.cu_seqlens, log=log)
    bb = c.beta.copy()
    bb[3, 0] = 2.5
    with pytest.raises(ValueError):
        run(c.alpha, c.cu_seqlens, beta=to_dev(bb))


def test_sr_debug_replay_returns_before_enqueue(monkeypatch):
    """With SR_DEBUG=1 a replay with broken boundaries is rejected before the
    replay kernel is enqueued (the state output keeps its sentinel), and a
    valid call still matches the oracle."""
    import torch
    import linear_attention_state_anchor_amd as sr
    print("[gdn] SR_DEBUG", flush=True)
    monkeypatch.setenv("SR_DEBUG", "1")
    c = gdn_case([100, 30], 1, 2, 128, "bf16", seed=72, normalize_q=True)
    S = torch.full((2, 2, 128, 128), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        sr.gdn_replay_state(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.alpha),
                            to_dev(c.beta), to_dev(np.array([0, 131, 130], np.int32)),
                            alpha_is_log=True, final_state=S)
    torch.cuda.synchronize()
    assert bool((S == 3.0).all())
    check(c, TOL_BF16)

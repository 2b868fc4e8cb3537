"""GPU parity of the group replay (sr_pack_gdn_layer + sr_replay_group)
against the fp64 group oracle on the same seeded inputs.

The whole group runs on the GPU: pre-mixer RMSNorm, fused input projection
(fp16 matrix-core operands, fp32 accumulation), short conv + SiLU, L2 norms,
gates, the chunked gated delta rule, gated RMSNorm and the output projection
with the residual.  Tolerance: 2e-3 relative Frobenius on every layer's
state and conv window (the windows are pre-conv projections, carrying the
matrix-core rounding of the layer input; about 3e-4 at the first layer,
growing to about 9e-4 at the third of a hidden-2560 group).
"""
import numpy as np
import pytest

import oracle
from replay_inputs import (FA, GDN, GroupCase, PAGE, _group, config_c4, config_c5,
                           to_bf16_bits)
from tests.util import rel_fro, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = 2e-3


def pack_all(g):
    """Packed weights per GDN layer: the mixer, or (mixer, FFN) pairs."""
    import linear_attention_state_anchor_amd as sr
    out = []
    for w in g.weights:
        mix = sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), g.h_k, g.h_v,
                                g.d)
        if getattr(w, "w_gate", None) is not None:
            out.append((mix, sr.pack_ffn(to_dev(w.w_gate), to_dev(w.w_up), to_dev(w.w_down))))
        else:
            out.append(mix)
    return out


def ffn_dim(g):
    return (g.meta or {}).get("ffn_dim", 0) or 0


def gpu_group(g, anchors_dev=None, cu_dev=None, packed=None):
    import torch
    import linear_attention_state_anchor_amd as sr
    print(f"[group] {g.meta.get('name', '')} lens={g.meta.get('lens', [])[:6]} "
          f"hidden={g.hidden} hk={g.h_k} hv={g.h_v} d={g.d} kinds={g.layer_kind}",
          flush=True)
    packed = pack_all(g) if packed is None else packed
    anchors_dev = to_dev(g.anchors) if anchors_dev is None else anchors_dev
    cu_dev = to_dev(g.cu_seqlens) if cu_dev is None else cu_dev
    states, conv = sr.replay_group(anchors_dev, packed, cu_dev, g.layer_kind, g.h_k, g.h_v,
                                   g.d, conv_width=g.conv_width, want_conv_state=True,
                                   ffn_dim=ffn_dim(g))
    # without the conv windows the projection and the front end run as one
    # kernel (widths up to 4); every value must come out identical
    states_f = sr.replay_group(anchors_dev, packed, cu_dev, g.layer_kind, g.h_k, g.h_v,
                               g.d, conv_width=g.conv_width, want_conv_state=False,
                               ffn_dim=ffn_dim(g))
    torch.cuda.synchronize()
    states, states_f = to_np(states), to_np(states_f)
    np.testing.assert_array_equal(states_f, states)
    return states, to_np(conv)


def oracle_group(g, anchors=None, cu=None):
    return oracle.replay_group(g.anchors if anchors is None else anchors, g.weights,
                               g.cu_seqlens if cu is None else cu, g.layer_kind, g.h_k, g.h_v,
                               g.d)


def check(g):
    S, C = gpu_group(g)
    Sr, Cr = oracle_group(g)
    assert S.shape == Sr.shape and C.shape == Cr.shape
    for li in range(S.shape[0]):
        e = rel_fro(S[li], Sr[li])
        ec = rel_fro(C[li], Cr[li])
        worst = max(((rel_fro(S[li, n, h], Sr[li, n, h]), (n, h))
                     for n in range(S.shape[1]) for h in range(S.shape[2])
                     if np.any(Sr[li, n, h])), default=(0.0, None))
        print(f"    layer {li}: rel state {e:.3e}  rel conv state {ec:.3e}  worst (request, "
              f"head) state {worst[0]:.3e} at {worst[1]}", flush=True)
        # the gate is on the whole tensor; the worst (request, head) block is
        # reported (a one-token request's state is one rank-one product, with
        # no averaging of rounding errors)
        assert e <= TOL, (li, e)
        assert ec <= TOL, (li, ec)
    return S, C


@pytest.mark.parametrize("kinds", [[GDN, GDN, GDN, FA], [FA, GDN], [GDN]])
def test_small_group(kinds):
    g = _group([100, 37, 3, 0, 64], 11, 256, 2, 4, 64, kinds)
    check(g)


@pytest.mark.parametrize("d", [64, 128])
def test_sequence_starts_at_projection_tile_edges(d):
    """Sequences that start right at, and just after, the rows where the
    fused projection's overlapping M tiles meet (every 253 rows: each tile
    recomputes the 3 rows before its first emitted row), very short
    sequences, and a total that leaves a last tile of a few rows.  gpu_group
    asserts the fused and separate front ends agree bit for bit; the oracle
    checks the values."""
    lens = [253, 1, 2, 3, 247, 253, 255, 1, 40]   # starts at 253, 254, 256, 259, 506, ...
    g = _group(lens, 31, 256, 2, 4, d, [GDN, GDN, FA])
    check(g)


@pytest.mark.parametrize("width", [2, 6, 8])
def test_conv_widths(width):
    """Conv widths other than 4 (the wider ones take the 8-tap front end)."""
    g = _group([70, 5, 129], 14 + width, 256, 2, 4, 128, [GDN, GDN], conv_width=width)
    check(g)


def test_group_hidden_2560_short():
    g = _group([130, 65, 1], 12, 2560, 16, 32, 128, [GDN, GDN, GDN, FA])
    check(g)


def test_group_full_size():
    """3 GDN layers + a skipped full-attention layer, hidden 2560, 4 requests
    x 1638 anchors (5 % of a 32K prefix), random-init bf16 weights."""
    check(config_c4())


def _solo(g, i):
    a, b = int(g.cu_seqlens[i]), int(g.cu_seqlens[i + 1])
    return GroupCase(anchors=g.anchors[a:b], cu_seqlens=np.array([0, b - a], np.int32),
                     layer_kind=g.layer_kind, weights=g.weights, hidden=g.hidden, h_k=g.h_k,
                     h_v=g.h_v, d=g.d, conv_width=g.conv_width,
                     meta={"name": f"solo {i}", "ffn_dim": ffn_dim(g)})


def test_group_deterministic_and_solo():
    """Repeated calls are bit-identical, and a request replayed inside a packed
    batch gives exactly the states and conv windows it gives alone: every
    kernel of the group reduces a row in an order that does not depend on the
    row's position or its neighbours."""
    g = _group([90, 40], 13, 256, 2, 4, 128, [GDN, GDN])
    S1, C1 = gpu_group(g)
    S2, C2 = gpu_group(g)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(C1, C2)
    for i in range(2):
        S3, C3 = gpu_group(_solo(g, i))
        np.testing.assert_array_equal(S3[:, 0], S1[:, i])
        np.testing.assert_array_equal(C3[:, 0], C1[:, i])


def test_group_packed_equals_solo_across_launch_shapes():
    """16 requests x 32 value heads: the packed replay's GDN launches have 512
    (sequence, head) chains (value-head pairs per workgroup), each request
    alone has 32 (one head of 8 waves); projections tile the rows
    differently too.  States and conv windows must be bit-identical."""
    lens = [70, 1, 64, 129, 3, 200, 65, 17, 128, 90, 31, 63, 150, 5, 100, 77]
    g = _group(lens, 17, 256, 16, 32, 128, [GDN, GDN, FA])
    S, C = gpu_group(g)
    for i in (0, 1, 5, 15):
        Si, Ci = gpu_group(_solo(g, i))
        np.testing.assert_array_equal(Si[:, 0], S[:, i])
        np.testing.assert_array_equal(Ci[:, 0], C[:, i])


N_VARLEN_ORACLE = 16  # requests of the 64-hit batch the oracle replays


def test_varlen_from_paged_pool():
    """Varlen batch of 64 hits (m ~ U{8192..32768}, k = ceil(r m), r ~ U[0.05,
    0.10]) gathered from a 64-token paged pool and replayed through a 3-layer
    group, all 64 in one packed launch sequence.  The pool is filled on the
    device from a seeded generator; the oracle replays the first 16 requests
    (about a quarter of the batch: the fp64 projections of all 64 take
    minutes) from the pool pages copied to the host."""
    import torch
    import linear_attention_state_anchor_amd as sr
    pc, weights = config_c5()
    print(f"[group] varlen from pool: {int(pc.suffix_len.sum())} tokens", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(105)
    # bf16 ~ N(0,1) anchors
    pool = torch.randn((pc.n_pages, PAGE, pc.hidden), generator=gen, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)
    total = int(pc.suffix_len.sum())
    packed_anchors, cu = sr.gather_suffix(pool, to_dev(pc.page_table), to_dev(pc.matched_len),
                                          to_dev(pc.suffix_len), total)
    g = GroupCase(anchors=None, cu_seqlens=None, layer_kind=[GDN, GDN, GDN, FA],
                  weights=weights, hidden=pc.hidden, h_k=16, h_v=32, d=128, conv_width=4,
                  meta={"name": "varlen pool", "lens": list(pc.suffix_len[:6])})
    S, C = gpu_group(g, anchors_dev=packed_anchors, cu_dev=cu)
    sel = list(range(N_VARLEN_ORACLE))
    anchors, lens = [], []
    for i in sel:
        m, k = int(pc.matched_len[i]), int(pc.suffix_len[i])
        pages = pc.page_table[i][:(m + PAGE - 1) // PAGE]
        host = pool[torch.from_numpy(pages.astype(np.int64)).cuda()].view(torch.int16).cpu()
        host = host.numpy().view(np.uint16)           # [pages][64][hidden] bf16 bits
        sub_pt = np.arange(len(pages), dtype=np.int32)[None, :]
        a_i, _ = oracle.gather_suffix(host, sub_pt, [m], [k])
        anchors.append(a_i)
        lens.append(k)
    cu_o = np.zeros(len(sel) + 1, np.int32)
    cu_o[1:] = np.cumsum(lens)
    Sr, Cr = oracle.replay_group(np.concatenate(anchors), weights, cu_o, g.layer_kind,
                                 16, 32, 128)
    for li in range(3):
        e = rel_fro(S[li, sel], Sr[li])
        worst = max((rel_fro(S[li, i, h], Sr[li, j, h]), (i, h))
                    for j, i in enumerate(sel) for h in range(32))
        print(f"    layer {li}: rel state {e:.3e} over requests 0..{len(sel) - 1}; worst "
              f"(request, head) {worst[0]:.3e} at {worst[1]}", flush=True)
        assert e <= TOL
    assert rel_fro(C[:, sel], Cr) <= TOL
    assert np.all(np.isfinite(S))


def test_sr_debug_group_returns_before_enqueue(monkeypatch):
    import torch
    import linear_attention_state_anchor_amd as sr
    print("[group] SR_DEBUG", flush=True)
    monkeypatch.setenv("SR_DEBUG", "1")
    g = _group([40, 30], 19, 256, 2, 4, 64, [GDN, GDN])
    packed = pack_all(g)
    states = torch.full((2, 2, 4, 64, 64), 5.0, dtype=torch.float32, device="cuda")
    bad_cu = to_dev(np.array([0, 71, 70], np.int32))
    with pytest.raises(ValueError):
        sr.replay_group(to_dev(g.anchors), packed, bad_cu, g.layer_kind, 2, 4, 64, states=states)
    torch.cuda.synchronize()
    assert bool((states == 5.0).all())
    check(g)



# ---------------------------------------------------------------------------
# FFN blocks between the GDN layers (skipped after the last layer)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("hidden,hk,hv,d,F", [(256, 2, 4, 128, 512), (256, 2, 4, 64, 192),
                                               (2560, 16, 32, 128, 9728)])
def test_group_with_ffn(hidden, hk, hv, d, F):
    g = _group([130, 65, 1, 0], 27 + F, hidden, hk, hv, d, [GDN, GDN, GDN, FA], ffn_dim=F)
    check(g)


def test_group_with_ffn_packed_equals_solo():
    g = _group([90, 40, 7], 29, 256, 2, 4, 128, [GDN, GDN], ffn_dim=256)
    S, C = gpu_group(g)
    for i in range(3):
        Si, Ci = gpu_group(_solo(g, i))
        np.testing.assert_array_equal(Si[:, 0], S[:, i])
        np.testing.assert_array_equal(Ci[:, 0], C[:, i])

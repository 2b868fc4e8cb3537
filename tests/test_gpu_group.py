"""GPU parity of the group replay (sr_pack_gdn_layer + sr_replay_group)
against the fp64 group oracle on the same seeded inputs.

The whole group runs on the GPU: pre-mixer RMSNorm, fused input projection
(fp16 matrix-core operands, fp32 accumulation), short conv + SiLU, L2 norms,
gates, the chunked gated delta rule, gated RMSNorm and the output projection
with the residual.  Tolerance: 2e-3 relative Frobenius on every layer's
state; conv states are checked to 1e-3 (they are pre-conv projections,
carrying only the matrix-core rounding of the layer input).
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
    import linear_attention_state_anchor_amd as sr
    return [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), g.h_k,
                              g.h_v, g.d) for w in g.weights]


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
                                   g.d, conv_width=g.conv_width, want_conv_state=True)
    torch.cuda.synchronize()
    return to_np(states), to_np(conv)


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
        print(f"    layer {li}: rel state {e:.3e}  rel conv state {ec:.3e}", flush=True)
        assert e <= TOL, (li, e)
        assert ec <= 1e-3, (li, ec)
    return S, C


@pytest.mark.parametrize("kinds", [[GDN, GDN, GDN, FA], [FA, GDN], [GDN]])
def test_small_group(kinds):
    g = _group([100, 37, 3, 0, 64], 11, 256, 2, 4, 64, kinds)
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


def test_group_deterministic_and_solo():
    g = _group([90, 40], 13, 256, 2, 4, 128, [GDN, GDN])
    S1, C1 = gpu_group(g)
    S2, C2 = gpu_group(g)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(C1, C2)
    a, b = g.cu_seqlens[1], g.cu_seqlens[2]
    solo = GroupCase(anchors=g.anchors[a:b], cu_seqlens=np.array([0, b - a], np.int32),
                     layer_kind=g.layer_kind, weights=g.weights, hidden=g.hidden, h_k=g.h_k,
                     h_v=g.h_v, d=g.d, conv_width=g.conv_width, meta={})
    S3, C3 = gpu_group(solo)
    # the projections tile rows differently, so equal up to rounding only
    assert rel_fro(S3[:, 0], S1[:, 1]) < 1e-5


def test_varlen_from_paged_pool_sampled():
    """Varlen batch of 64 hits (m ~ U{8192..32768}, k = ceil(r m), r ~ U[0.05,
    0.10]) gathered from a 64-token paged pool and replayed through a 3-layer
    group.  The pool is filled on the device from a seeded generator; the
    oracle replays 3 of the requests from the pool pages copied to the host."""
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
    for i in (0, 31, 63):
        m, k = int(pc.matched_len[i]), int(pc.suffix_len[i])
        pages = pc.page_table[i][:(m + PAGE - 1) // PAGE]
        host = pool[torch.from_numpy(pages.astype(np.int64)).cuda()].view(torch.int16).cpu()
        host = host.numpy().view(np.uint16)           # [pages][64][hidden] bf16 bits
        sub_pt = np.arange(len(pages), dtype=np.int32)[None, :]
        anchors, cu_i = oracle.gather_suffix(host, sub_pt, [m], [k])
        Sr, Cr = oracle.replay_group(anchors, weights, cu_i, g.layer_kind, 16, 32, 128)
        for li in range(3):
            e = rel_fro(S[li, i], Sr[li, 0])
            print(f"    request {i} (k={k}) layer {li}: rel state {e:.3e}", flush=True)
            assert e <= TOL
        assert rel_fro(C[:, i], Cr[:, 0]) <= 1e-3

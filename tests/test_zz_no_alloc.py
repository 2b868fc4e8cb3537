"""Allocation-free group replay (sr_replay_group_noalloc: the workspace is the
library's static per-GPU array) against the workspace entry point
(sr_replay_group), both through the C ABI: bit-identical states and conv
windows on two calls in a row, the second with a smaller input, and a group
too large for the static array rejected before anything is enqueued."""
import numpy as np
import pytest

from replay_inputs import FA, GDN, _group
from tests.util import to_dev, to_np

pytestmark = pytest.mark.gpu

KINDS = [GDN, GDN, GDN, FA]


def _pack(g):
    import linear_attention_state_anchor_amd as sr
    return [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), g.h_k, g.h_v,
                              g.d) for w in g.weights]


def _both(g, packed):
    import torch
    import linear_attention_state_anchor_amd as sr
    anchors, cu = to_dev(g.anchors), to_dev(g.cu_seqlens)
    S1, C1 = sr.replay_group(anchors, packed, cu, g.layer_kind, g.h_k, g.h_v, g.d,
                             want_conv_state=True)
    S2 = torch.full_like(S1, 7.0)
    C2 = torch.full_like(C1, 7.0)
    sr.replay_group_noalloc(anchors, packed, cu, g.layer_kind, g.h_k, g.h_v, g.d,
                            want_conv_state=True, states=S2, conv_states=C2)
    torch.cuda.synchronize()
    return to_np(S1), to_np(C1), to_np(S2), to_np(C2)


@pytest.mark.parametrize("hidden,hk,hv,d", [(2560, 16, 32, 128), (256, 2, 4, 64)])
def test_noalloc_equals_workspace_entry_two_calls(hidden, hk, hv, d):
    import linear_attention_state_anchor_amd as sr
    print(f"[noalloc] hidden={hidden} hk={hk} hv={hv} d={d}", flush=True)
    big = _group([700, 129, 1, 600], 31, hidden, hk, hv, d, KINDS)
    small = _group([65, 3], 32, hidden, hk, hv, d, KINDS)
    small.weights = big.weights        # the same layers, a smaller batch second
    packed = _pack(big)
    for g in (big, small):
        need = sr.group_workspace_bytes(g.total_tokens, hidden, hk, hv, d, n_seqs=g.n_seqs,
                                        layer_kind=KINDS)
        assert 0 < need <= sr.noalloc_max_bytes()
        S1, C1, S2, C2 = _both(g, packed)
        print(f"    T={g.total_tokens}: workspace {need / 2 ** 20:.1f} MiB, states equal",
              flush=True)
        np.testing.assert_array_equal(S2, S1)
        np.testing.assert_array_equal(C2, C1)


def test_noalloc_rejects_a_group_beyond_the_static_workspace():
    import torch
    import linear_attention_state_anchor_amd as sr
    print("[noalloc] oversize", flush=True)
    g = _group([10], 33, 2560, 16, 32, 128, KINDS)
    packed = _pack(g)
    T = 4000
    assert sr.group_workspace_bytes(T, 2560, 16, 32, 128, n_seqs=2,
                                    layer_kind=KINDS) > sr.noalloc_max_bytes()
    anchors = torch.zeros((T, 2560), dtype=torch.bfloat16, device="cuda")
    cu = to_dev(np.array([0, 1000, T], np.int32))
    states = torch.full((3, 2, 32, 128, 128), 9.0, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        sr.replay_group_noalloc(anchors, packed, cu, KINDS, 16, 32, 128, states=states)
    torch.cuda.synchronize()
    assert bool((states == 9.0).all())

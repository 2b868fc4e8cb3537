"""Suffix-replay state reconstruction on MI355X (gfx950).

On a prefix-cache hit, a hybrid model's linear-attention states are rebuilt
by replaying the last k cached anchor hidden states of the matched prefix
through each group of Gated DeltaNet layers, from a zero state
("SuffixReplay", Eq. 1-4 and Algorithm Design; "Tail-Replay", section 3).

This module is a thin binding over the C ABI of libsr_replay.so
(include/sr_replay.h): it checks tensor metadata, allocates outputs with
torch on the current stream and passes raw device pointers.  Every step of
the computation runs in the library's HIP kernels; there is no other path.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import ReplayError, SR_BF16, SR_F16, SR_F32, SR_LAYER_FA, SR_LAYER_GDN

__all__ = ["gdn_replay_state", "gather_suffix", "pack_gdn_layer", "replay_group",
           "packed_layer_bytes", "version", "ReplayError", "SR_LAYER_GDN",
           "SR_LAYER_FA"]

_DT = {torch.bfloat16: SR_BF16, torch.float16: SR_F16, torch.float32: SR_F32}


def version() -> str:
    return _lib.load().sr_version().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def gdn_replay_state(q, k, v, alpha, beta=None, cu_seqlens=None, initial_state=None, *,
                     erase=True, alpha_is_log=False, scale=1.0, want_o=True,
                     o_dtype=None, final_state=None, o=None):
    """Gated-delta-rule replay of one layer (sr_gdn_replay_state).

    q, k: [T, h_k, d_k]; v: [T, h_v, d_v] (bf16, fp16 or fp32, one dtype);
    alpha (or log alpha with alpha_is_log): [T, h_v] fp32; beta: [T, h_v]
    fp32 or None (= 1); cu_seqlens: int32 [N+1] (None: one sequence);
    initial_state: fp32 [N, h_v, d_k, d_v] or None (= 0).
    Returns (final_state fp32 [N, h_v, d_k, d_v], o [T, h_v, d_v] or None).
    """
    _need(k, "k", ndim=3)
    _need(v, "v", dtype=k.dtype, ndim=3)
    if k.dtype not in _DT:
        raise ValueError(f"unsupported dtype {k.dtype}")
    T, h_k, d_k = k.shape
    Tv, h_v, d_v = v.shape
    if Tv != T:
        raise ValueError("k and v disagree on T")
    _need(alpha, "alpha", torch.float32, 2)
    if tuple(alpha.shape) != (T, h_v):
        raise ValueError("alpha must be [T, h_v]")
    if beta is not None:
        _need(beta, "beta", torch.float32, 2)
        if tuple(beta.shape) != (T, h_v):
            raise ValueError("beta must be [T, h_v]")
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=k.device)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    n = cu_seqlens.shape[0] - 1
    if want_o:
        _need(q, "q", dtype=k.dtype, ndim=3)
        if tuple(q.shape) != (T, h_k, d_k):
            raise ValueError("q must match k")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if tuple(initial_state.shape) != (n, h_v, d_k, d_v):
            raise ValueError("initial_state must be [N, h_v, d_k, d_v]")
    if final_state is None:
        final_state = torch.empty((n, h_v, d_k, d_v), dtype=torch.float32, device=k.device)
    else:
        _need(final_state, "final_state", torch.float32, 4)
    o_dtype = v.dtype if o_dtype is None else o_dtype
    if want_o and o is None:
        o = torch.empty((T, h_v, d_v), dtype=o_dtype, device=k.device)
    if not want_o:
        o = None
    elif o.dtype not in _DT:
        raise ValueError(f"unsupported output dtype {o.dtype}")
    desc = _lib.GdnDesc(n, T, h_k, h_v, d_k, d_v, _DT[k.dtype],
                        _DT[o.dtype] if o is not None else SR_F32, int(bool(erase)),
                        int(bool(alpha_is_log)), float(scale))
    io = _lib.GdnIO(_ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                    _ptr(cu_seqlens), _ptr(initial_state), _ptr(final_state), _ptr(o))
    st = _lib.load().sr_gdn_replay_state(ctypes.byref(desc), ctypes.byref(io), _stream())
    _lib.check("sr_gdn_replay_state", st)
    return final_state, o


def gather_suffix(pool, page_table, matched_len, suffix_len, total_tokens=None, *,
                  packed=None, cu_seqlens=None):
    """Gather the last k_i anchors of each hit from a paged pool and pack them
    varlen (sr_gather_suffix).

    pool: [P, 64, hidden] (2- or 4-byte elements); page_table: int32
    [N, max_pages]; matched_len, suffix_len: int32 [N].  total_tokens = sum
    of suffix_len (read back from the device when not given).
    Returns (packed [total, hidden], cu_seqlens int32 [N+1]).
    """
    _need(pool, "pool", ndim=3)
    if pool.shape[1] != 64:
        raise ValueError("pool pages must hold 64 tokens")
    _need(page_table, "page_table", torch.int32, 2)
    _need(matched_len, "matched_len", torch.int32, 1)
    _need(suffix_len, "suffix_len", torch.int32, 1)
    n = matched_len.shape[0]
    if total_tokens is None:
        total_tokens = int(suffix_len.sum().item())
    hidden = pool.shape[2]
    if packed is None:
        packed = torch.empty((total_tokens, hidden), dtype=pool.dtype, device=pool.device)
    if cu_seqlens is None:
        cu_seqlens = torch.empty((n + 1,), dtype=torch.int32, device=pool.device)
    st = _lib.load().sr_gather_suffix(
        _ptr(pool), hidden, pool.element_size(), pool.shape[0], _ptr(page_table),
        page_table.shape[1], _ptr(matched_len), _ptr(suffix_len), n, total_tokens,
        _ptr(packed), _ptr(cu_seqlens), _stream())
    _lib.check("sr_gather_suffix", st)
    return packed, cu_seqlens


def packed_layer_bytes(hidden, h_k, h_v, d, conv_width=4) -> int:
    return int(_lib.load().sr_packed_layer_bytes(hidden, h_k, h_v, d, conv_width))


def pack_gdn_layer(w_in, conv_w, w_out, h_k, h_v, d):
    """Pack one GDN layer's bf16 weights into the library's layout
    (sr_pack_gdn_layer).  w_in [hidden, n_in], conv_w [conv_dim, width],
    w_out [h_v*d, hidden] or None.  Returns a uint8 device tensor."""
    _need(w_in, "w_in", torch.bfloat16, 2)
    _need(conv_w, "conv_w", torch.bfloat16, 2)
    if w_out is not None:
        _need(w_out, "w_out", torch.bfloat16, 2)
    hidden = w_in.shape[0]
    width = conv_w.shape[1]
    nbytes = packed_layer_bytes(hidden, h_k, h_v, d, width)
    out = torch.empty((nbytes,), dtype=torch.uint8, device=w_in.device)
    st = _lib.load().sr_pack_gdn_layer(_ptr(w_in), _ptr(conv_w), _ptr(w_out), hidden, h_k,
                                       h_v, d, width, _ptr(out), _stream())
    _lib.check("sr_pack_gdn_layer", st)
    return out


def replay_group(anchors, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, *,
                 conv_width=4, rms_eps=1e-6, l2_eps=1e-6, max_seqlen=None,
                 want_conv_state=False, states=None, workspace=None):
    """Replay one group of linear-attention layers from its anchors
    (sr_replay_group).  Returns states fp32 [n_gdn, N, h_v, d, d] (and conv
    states fp32 [n_gdn, N, conv_dim, width-1] if asked)."""
    _need(anchors, "anchors", torch.bfloat16, 2)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    T, hidden = anchors.shape
    n = cu_seqlens.shape[0] - 1
    kinds = [int(x) for x in layer_kind]
    n_gdn = sum(1 for x in kinds if x == SR_LAYER_GDN)
    if len(packed_weights) != n_gdn:
        raise ValueError("one packed weight tensor per GDN layer")
    if max_seqlen is None:
        max_seqlen = T
    kind_arr = (ctypes.c_int32 * max(len(kinds), 1))(*kinds)
    desc = _lib.GroupDesc(len(kinds), ctypes.cast(kind_arr, ctypes.POINTER(ctypes.c_int32)),
                          hidden, h_k, h_v, d, conv_width, float(rms_eps), float(l2_eps),
                          n, T, int(max_seqlen))
    lib = _lib.load()
    ws_bytes = int(lib.sr_replay_group_workspace_bytes(ctypes.byref(desc)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=anchors.device)
    if states is None:
        states = torch.empty((n_gdn, n, h_v, d, d), dtype=torch.float32, device=anchors.device)
    conv = None
    if want_conv_state:
        conv_dim = 2 * h_k * d + h_v * d
        conv = torch.empty((n_gdn, n, conv_dim, conv_width - 1), dtype=torch.float32,
                           device=anchors.device)
    wts = (_lib.LayerWeights * max(n_gdn, 1))(*[_lib.LayerWeights(_ptr(w)) for w in packed_weights])
    st = lib.sr_replay_group(ctypes.byref(desc), wts, _ptr(anchors), _ptr(cu_seqlens),
                             _ptr(states), _ptr(conv), _ptr(workspace), ws_bytes, _stream())
    _lib.check("sr_replay_group", st)
    return (states, conv) if want_conv_state else states

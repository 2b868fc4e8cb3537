"""Suffix-replay state reconstruction on MI355X (gfx950).

On a prefix-cache hit, a hybrid model's linear-attention states are rebuilt
by replaying the last k cached anchor hidden states of the matched prefix
through each group of Gated DeltaNet layers, from a zero state
("SuffixReplay", Eq. 1-4 and Algorithm Design; "Tail-Replay", section 3).

This module is a thin binding over the C ABI of libsr_replay.so
(include/sr_replay.h): it checks tensor metadata (dtype, device, layout and
exact shape of every buffer, caller-supplied outputs included), allocates
outputs with torch on the current stream and passes raw device pointers.
Every step of the computation runs in the library's HIP kernels; there is no
other path.  Argument errors raise ValueError (ReplayArgumentError), launch
failures ReplayError.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (ReplayArgumentError, ReplayError, SR_BF16, SR_F16, SR_F32, SR_LAYER_FA,
                   SR_LAYER_GDN)

__all__ = ["gdn_replay_state", "gdn_decode_step", "extend_group", "check_replay_inputs",
           "gather_suffix", "gather_anchors",
           "check_gather_inputs", "replay_budget", "pack_gdn_layer", "replay_group",
           "packed_layer_bytes", "pack_ffn", "packed_ffn_bytes", "group_workspace_bytes",
           "replay_group_noalloc",
           "noalloc_max_bytes", "version", "ReplayError",
           "ReplayArgumentError", "SR_LAYER_GDN", "SR_LAYER_FA", "PAGE",
           "DENSE_NEAR_BOUNDARY_1_16", "UNIFORM_1_16"]

_DT = {torch.bfloat16: SR_BF16, torch.float16: SR_F16, torch.float32: SR_F32}

PAGE = 64  # tokens per KV page / anchor block
# in-page anchor offsets for density 1/16 ("SuffixReplay", Algorithm Design 2,
# Figure 3): concentrated next to the page boundary, or spread uniformly
DENSE_NEAR_BOUNDARY_1_16 = (60, 61, 62, 63)
UNIFORM_1_16 = (15, 31, 47, 63)


def version() -> str:
    return _lib.load().sr_version().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None, ndim=None, device=None):
    """Metadata check of a tensor handed to the library: device tensor,
    contiguous, and (when given) dtype, exact shape, rank and device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _gdn_call(q, k, v, alpha, beta, cu_seqlens, initial_state, erase, alpha_is_log, scale,
              want_o, o_dtype, final_state, o):
    _need(k, "k", ndim=3)
    dev = k.device
    if k.dtype not in _DT:
        raise ValueError(f"unsupported dtype {k.dtype}")
    T, h_k, d_k = k.shape
    _need(v, "v", dtype=k.dtype, ndim=3, device=dev)
    Tv, h_v, d_v = v.shape
    if Tv != T:
        raise ValueError("k and v disagree on T")
    if h_k < 1 or h_v % h_k != 0:
        raise ValueError("h_v must be a multiple of h_k")
    _need(alpha, "alpha", torch.float32, (T, h_v), device=dev)
    if beta is not None:
        _need(beta, "beta", torch.float32, (T, h_v), device=dev)
    if cu_seqlens is None:
        cu_seqlens = torch.tensor([0, T], dtype=torch.int32, device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, ndim=1, device=dev)
    n = cu_seqlens.shape[0] - 1
    if n < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if want_o:
        _need(q, "q", dtype=k.dtype, shape=(T, h_k, d_k), device=dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, h_v, d_k, d_v), device=dev)
    if final_state is None:
        final_state = torch.empty((n, h_v, d_k, d_v), dtype=torch.float32, device=dev)
    else:
        _need(final_state, "final_state", torch.float32, (n, h_v, d_k, d_v), device=dev)
    if not want_o:
        o = None
    elif o is None:
        o_dtype = v.dtype if o_dtype is None else o_dtype
        if o_dtype not in _DT:
            raise ValueError(f"unsupported output dtype {o_dtype}")
        o = torch.empty((T, h_v, d_v), dtype=o_dtype, device=dev)
    else:
        if o.dtype not in _DT:
            raise ValueError(f"unsupported output dtype {o.dtype}")
        _need(o, "o", shape=(T, h_v, d_v), device=dev)
    desc = _lib.GdnDesc(n, T, h_k, h_v, d_k, d_v, _DT[k.dtype],
                        _DT[o.dtype] if o is not None else SR_F32, int(bool(erase)),
                        int(bool(alpha_is_log)), float(scale))
    io = _lib.GdnIO(_ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                    _ptr(cu_seqlens), _ptr(initial_state), _ptr(final_state), _ptr(o))
    return desc, io, final_state, o


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
    desc, io, final_state, o = _gdn_call(q, k, v, alpha, beta, cu_seqlens, initial_state,
                                         erase, alpha_is_log, scale, want_o, o_dtype,
                                         final_state, o)
    lib = _lib.load()
    ws = int(lib.sr_gdn_workspace_bytes(ctypes.byref(desc)))
    if ws == ctypes.c_size_t(-1).value:
        raise ReplayArgumentError("sr_gdn_workspace_bytes", _lib.SR_ESHAPE)
    workspace = torch.empty((ws,), dtype=torch.uint8, device=k.device) if ws else None
    st = lib.sr_gdn_replay_state(ctypes.byref(desc), ctypes.byref(io), _ptr(workspace), ws,
                                 _stream())
    _lib.check("sr_gdn_replay_state", st)
    return final_state, o


def gdn_decode_step(q, k, v, alpha, beta=None, state=None, *, erase=True, alpha_is_log=False,
                    scale=1.0, want_o=True, o_dtype=None, out_state=None, o=None):
    """One decode token per sequence from a given state (sr_gdn_decode_step).

    q, k: [N, h_k, d]; v: [N, h_v, d] (row n: sequence n's token); alpha,
    beta: [N, h_v] fp32; state: fp32 [N, h_v, d, d] (the state before the
    token, transposed as gdn_replay_state returns it) or None (= 0).
    out_state may be `state` itself for an in-place update (the default when
    a state is given).  Returns (state after the token, o [N, h_v, d] or None).
    """
    _need(k, "k", ndim=3)
    N = k.shape[0]
    cu_dummy = torch.zeros((N + 1,), dtype=torch.int32, device=k.device)
    if out_state is None:
        out_state = state
    desc, io, out_state, o = _gdn_call(q, k, v, alpha, beta, cu_dummy, state, erase,
                                       alpha_is_log, scale, want_o, o_dtype, out_state, o)
    io.cu_seqlens = None
    st = _lib.load().sr_gdn_decode_step(ctypes.byref(desc), ctypes.byref(io), _stream())
    _lib.check("sr_gdn_decode_step", st)
    return out_state, o


def check_replay_inputs(q, k, v, alpha, beta=None, cu_seqlens=None, initial_state=None, *,
                        erase=True, alpha_is_log=False, want_o=True):
    """Run the device-side precondition check of one replay
    (sr_check_replay_inputs: cu_seqlens monotone with cu[0] = 0 and cu[N] = T,
    alpha in (0, 1] or log alpha <= 0, beta in [0, 2]); synchronises.
    Raises ReplayArgumentError (a ValueError) on a violation."""
    desc, io, _, _ = _gdn_call(q, k, v, alpha, beta, cu_seqlens, initial_state, erase,
                               alpha_is_log, 1.0, want_o, None, None, None)
    st = _lib.load().sr_check_replay_inputs(ctypes.byref(desc), ctypes.byref(io), _stream())
    _lib.check("sr_check_replay_inputs", st)


def _gather_common(pool, page_table, matched_len, suffix_len, rows):
    # the pool may sit in pinned host memory (read by the kernel over the
    # host link); everything else is device memory
    _need(page_table, "page_table", torch.int32, ndim=2)
    dev = page_table.device
    if pool.is_cuda:
        _need(pool, "pool", ndim=3, device=dev)
    else:
        if not isinstance(pool, torch.Tensor) or not pool.is_pinned():
            raise ValueError("a host pool must be a pinned (page-locked) tensor")
        if not pool.is_contiguous() or pool.dim() != 3:
            raise ValueError("pool must be a contiguous [P, rows, hidden] tensor")
    if pool.element_size() not in (2, 4):
        raise ValueError("pool elements must be 2 or 4 bytes")
    if pool.shape[1] != rows:
        raise ValueError(f"pool blocks must hold {rows} rows, got {pool.shape[1]}")
    _need(matched_len, "matched_len", torch.int32, ndim=1, device=dev)
    n = matched_len.shape[0]
    _need(suffix_len, "suffix_len", torch.int32, (n,), device=dev)
    if page_table.shape[0] != n or page_table.shape[1] < 1:
        raise ValueError(f"page_table must be [{n}, max_pages >= 1], got "
                         f"{tuple(page_table.shape)}")
    return n, dev


def _gather_outputs(pool, n, total_tokens, packed, cu_seqlens, dev):
    hidden = pool.shape[2]
    if packed is None:
        packed = torch.empty((total_tokens, hidden), dtype=pool.dtype, device=dev)
    else:
        _need(packed, "packed", dtype=pool.dtype, ndim=2, device=dev)
        if packed.shape[0] < total_tokens or packed.shape[1] != hidden:
            raise ValueError(f"packed must be [>= {total_tokens}, {hidden}], got "
                             f"{tuple(packed.shape)}")
    if cu_seqlens is None:
        cu_seqlens = torch.empty((n + 1,), dtype=torch.int32, device=dev)
    else:
        _need(cu_seqlens, "cu_seqlens", torch.int32, (n + 1,), device=dev)
    return packed, cu_seqlens


def gather_suffix(pool, page_table, matched_len, suffix_len, total_tokens=None, *,
                  packed=None, cu_seqlens=None):
    """Gather the last k_i anchors of each hit from a paged pool and pack them
    varlen (sr_gather_suffix).

    pool: [P, 64, hidden] (2- or 4-byte elements); page_table: int32
    [N, max_pages]; matched_len, suffix_len: int32 [N].  total_tokens = sum
    of suffix_len (read back from the device when not given).
    Returns (packed [total, hidden], cu_seqlens int32 [N+1]).
    """
    n, dev = _gather_common(pool, page_table, matched_len, suffix_len, PAGE)
    if total_tokens is None:
        total_tokens = int(suffix_len.sum().item())
    packed, cu_seqlens = _gather_outputs(pool, n, total_tokens, packed, cu_seqlens, dev)
    st = _lib.load().sr_gather_suffix(
        _ptr(pool), pool.shape[2], pool.element_size(), pool.shape[0], _ptr(page_table),
        page_table.shape[1], _ptr(matched_len), _ptr(suffix_len), n, total_tokens,
        _ptr(packed), _ptr(cu_seqlens), _stream())
    _lib.check("sr_gather_suffix", st)
    return packed, cu_seqlens


def _offsets(page_offsets):
    offs = [int(x) for x in page_offsets]
    if not 1 <= len(offs) <= PAGE:
        raise ValueError("1 to 64 anchors per page")
    return len(offs), (ctypes.c_int32 * len(offs))(*offs)


def gather_anchors(pool, page_offsets, page_table, matched_len, suffix_len, total_tokens=None,
                   *, packed=None, cu_seqlens=None, positions=True):
    """Gather the last k_i anchors of each hit with token-wise sparse anchors
    (sr_gather_anchors).

    pool: [P, A, hidden], block p holding the anchors of KV page p at the
    in-page positions page_offsets (A increasing values in [0, 64), e.g.
    DENSE_NEAR_BOUNDARY_1_16); matched_len: int32 [N] in tokens; suffix_len:
    int32 [N] in anchors.  Returns (packed [total, hidden], cu_seqlens
    int32 [N+1], positions int32 [total] or None)."""
    A, offs = _offsets(page_offsets)
    n, dev = _gather_common(pool, page_table, matched_len, suffix_len, A)
    if total_tokens is None:
        total_tokens = int(suffix_len.sum().item())
    packed, cu_seqlens = _gather_outputs(pool, n, total_tokens, packed, cu_seqlens, dev)
    pos = torch.empty((total_tokens,), dtype=torch.int32, device=dev) if positions else None
    st = _lib.load().sr_gather_anchors(
        _ptr(pool), pool.shape[2], pool.element_size(), pool.shape[0], A, offs,
        _ptr(page_table), page_table.shape[1], _ptr(matched_len), _ptr(suffix_len), n,
        total_tokens, _ptr(packed), _ptr(cu_seqlens), _ptr(pos), _stream())
    _lib.check("sr_gather_anchors", st)
    return packed, cu_seqlens, pos


def check_gather_inputs(n_blocks, page_table, matched_len, suffix_len, total_tokens,
                        page_offsets=None):
    """Device-side precondition check of a gather (sr_check_gather_inputs);
    synchronises; raises ReplayArgumentError (a ValueError) on a violation."""
    if page_offsets is None:
        A, offs = PAGE, None
    else:
        A, offs = _offsets(page_offsets)
    _need(matched_len, "matched_len", torch.int32, ndim=1)
    n = matched_len.shape[0]
    _need(suffix_len, "suffix_len", torch.int32, (n,))
    _need(page_table, "page_table", torch.int32, ndim=2)
    if page_table.shape[0] != n:
        raise ValueError("page_table needs one row per request")
    st = _lib.load().sr_check_gather_inputs(int(n_blocks), A, offs, _ptr(page_table),
                                            page_table.shape[1], _ptr(matched_len),
                                            _ptr(suffix_len), n, int(total_tokens), _stream())
    _lib.check("sr_check_gather_inputs", st)


def replay_budget(n_anchors, ratio=0.05, k_max=0):
    """Replay lengths k_i = min(ceil(ratio * n_i), k_max) (sr_replay_budget;
    k_max <= 0: no cap).  n_anchors: sequence of ints.  Returns a list."""
    ns = [int(x) for x in n_anchors]
    arr = (ctypes.c_int32 * max(len(ns), 1))(*ns)
    out = (ctypes.c_int32 * max(len(ns), 1))()
    total = _lib.load().sr_replay_budget(arr, len(ns), float(ratio), int(k_max), out)
    if total < 0:
        raise ReplayArgumentError("sr_replay_budget", _lib.SR_EINVAL)
    return [int(out[i]) for i in range(len(ns))]


def packed_ffn_bytes(hidden, ffn_dim) -> int:
    return int(_lib.load().sr_packed_ffn_bytes(hidden, ffn_dim))


def pack_ffn(w_gate, w_up, w_down):
    """Pack one FFN block's bf16 weights (sr_pack_ffn): w_gate, w_up [hidden,
    F], w_down [F, hidden].  Returns a uint8 device tensor."""
    _need(w_gate, "w_gate", torch.bfloat16, ndim=2)
    hidden, F = w_gate.shape
    _need(w_up, "w_up", torch.bfloat16, (hidden, F), device=w_gate.device)
    _need(w_down, "w_down", torch.bfloat16, (F, hidden), device=w_gate.device)
    nbytes = packed_ffn_bytes(hidden, F)
    if nbytes == 0:
        raise ValueError("unsupported FFN shape")
    out = torch.empty((nbytes,), dtype=torch.uint8, device=w_gate.device)
    st = _lib.load().sr_pack_ffn(_ptr(w_gate), _ptr(w_up), _ptr(w_down), hidden, F, _ptr(out),
                                 _stream())
    _lib.check("sr_pack_ffn", st)
    return out


def packed_layer_bytes(hidden, h_k, h_v, d, conv_width=4) -> int:
    return int(_lib.load().sr_packed_layer_bytes(hidden, h_k, h_v, d, conv_width))


def pack_gdn_layer(w_in, conv_w, w_out, h_k, h_v, d):
    """Pack one GDN layer's bf16 weights into the library's layout
    (sr_pack_gdn_layer).  w_in [hidden, 2 h_k d + 2 h_v d + 2 h_v], conv_w
    [2 h_k d + h_v d, width], w_out [h_v d, hidden] or None.  Returns a uint8
    device tensor."""
    _need(w_in, "w_in", torch.bfloat16, ndim=2)
    dev = w_in.device
    hidden = w_in.shape[0]
    n_in = 2 * h_k * d + 2 * h_v * d + 2 * h_v
    conv_dim = 2 * h_k * d + h_v * d
    if w_in.shape[1] != n_in:
        raise ValueError(f"w_in must be [{hidden}, {n_in}], got {tuple(w_in.shape)}")
    _need(conv_w, "conv_w", torch.bfloat16, ndim=2, device=dev)
    if conv_w.shape[0] != conv_dim:
        raise ValueError(f"conv_w must be [{conv_dim}, width], got {tuple(conv_w.shape)}")
    if w_out is not None:
        _need(w_out, "w_out", torch.bfloat16, (h_v * d, hidden), device=dev)
    width = conv_w.shape[1]
    nbytes = packed_layer_bytes(hidden, h_k, h_v, d, width)
    if nbytes == 0:
        raise ValueError("unsupported layer shape")
    out = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    st = _lib.load().sr_pack_gdn_layer(_ptr(w_in), _ptr(conv_w), _ptr(w_out), hidden, h_k,
                                       h_v, d, width, _ptr(out), _stream())
    _lib.check("sr_pack_gdn_layer", st)
    return out


def _event_handle(ev):
    """Raw hipEvent_t of a torch.cuda.Event (created on first use)."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()   # torch creates the event lazily, at its first record
    return ctypes.c_void_p(ev.cuda_event)


def _group_desc(kinds, hidden, h_k, h_v, d, conv_width, rms_eps, l2_eps, n, T, max_seqlen,
                layer_events=None, ffn_dim=0):
    kind_arr = (ctypes.c_int32 * max(len(kinds), 1))(*kinds)
    ev_arr = None
    if layer_events is not None:
        n_gdn = sum(1 for x in kinds if x == SR_LAYER_GDN)
        if len(layer_events) != n_gdn:
            raise ValueError("one event (or None) per GDN layer")
        ev_arr = (ctypes.c_void_p * max(n_gdn, 1))(*[_event_handle(e) for e in layer_events])
    desc = _lib.GroupDesc(len(kinds), ctypes.cast(kind_arr, ctypes.POINTER(ctypes.c_int32)),
                          hidden, h_k, h_v, d, conv_width, float(rms_eps), float(l2_eps),
                          n, T, int(max_seqlen),
                          ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p)) if ev_arr else None,
                          int(ffn_dim))
    return desc, (kind_arr, ev_arr)


def group_workspace_bytes(total_tokens, hidden, h_k, h_v, d, conv_width=4, n_seqs=1,
                          layer_kind=(SR_LAYER_GDN,), ffn_dim=0) -> int:
    """Workspace bytes of one replay_group call (sr_replay_group_workspace_bytes)."""
    kinds = [int(x) for x in layer_kind]
    desc, _keep = _group_desc(kinds, hidden, h_k, h_v, d, conv_width, 1e-6, 1e-6, n_seqs,
                              total_tokens, total_tokens, None, ffn_dim)
    return int(_lib.load().sr_replay_group_workspace_bytes(ctypes.byref(desc)))


def _group_prepare(anchors, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, conv_width,
                   rms_eps, l2_eps, max_seqlen, want_conv_state, states, conv_states,
                   layer_events=None, ffn_dim=0):
    _need(anchors, "anchors", torch.bfloat16, ndim=2)
    dev = anchors.device
    _need(cu_seqlens, "cu_seqlens", torch.int32, ndim=1, device=dev)
    T, hidden = anchors.shape
    n = cu_seqlens.shape[0] - 1
    if n < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    kinds = [int(x) for x in layer_kind]
    n_gdn = sum(1 for x in kinds if x == SR_LAYER_GDN)
    if len(packed_weights) != n_gdn:
        raise ValueError("one packed weight tensor per GDN layer")
    need_bytes = packed_layer_bytes(hidden, h_k, h_v, d, conv_width)
    if n_gdn and need_bytes == 0:
        raise ValueError("unsupported layer shape")
    ffn_bytes = packed_ffn_bytes(hidden, ffn_dim) if ffn_dim else 0
    pairs = []
    for i, w in enumerate(packed_weights):
        w_mix, w_ffn = (w if isinstance(w, (tuple, list)) else (w, None))
        _need(w_mix, f"packed_weights[{i}]", torch.uint8, ndim=1, device=dev)
        if w_mix.numel() < need_bytes:
            raise ValueError(f"packed_weights[{i}] holds {w_mix.numel()} bytes, the layer shape "
                             f"needs {need_bytes} (packed for another shape?)")
        if w_ffn is not None:
            if not ffn_dim:
                raise ValueError("FFN weights given but ffn_dim is 0")
            _need(w_ffn, f"packed FFN weights [{i}]", torch.uint8, ndim=1, device=dev)
            if w_ffn.numel() < ffn_bytes:
                raise ValueError(f"packed FFN weights [{i}] hold {w_ffn.numel()} bytes, "
                                 f"ffn_dim {ffn_dim} needs {ffn_bytes}")
        pairs.append((w_mix, w_ffn))
    if max_seqlen is None:
        max_seqlen = T
    desc, keep = _group_desc(kinds, hidden, h_k, h_v, d, conv_width, rms_eps, l2_eps, n, T,
                             max_seqlen, layer_events, ffn_dim)
    if states is None:
        states = torch.empty((n_gdn, n, h_v, d, d), dtype=torch.float32, device=dev)
    else:
        _need(states, "states", torch.float32, (n_gdn, n, h_v, d, d), device=dev)
    conv = None
    if want_conv_state:
        conv_dim = 2 * h_k * d + h_v * d
        shape = (n_gdn, n, conv_dim, conv_width - 1)
        if conv_states is None:
            conv = torch.empty(shape, dtype=torch.float32, device=dev)
        else:
            _need(conv_states, "conv_states", torch.float32, shape, device=dev)
            conv = conv_states
    wts = (_lib.LayerWeights * max(n_gdn, 1))(*[_lib.LayerWeights(_ptr(a), _ptr(b))
                                                 for a, b in pairs])
    return desc, keep, wts, states, conv, n_gdn, T


def replay_group(anchors, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, *,
                 conv_width=4, rms_eps=1e-6, l2_eps=1e-6, max_seqlen=None,
                 want_conv_state=False, states=None, conv_states=None, workspace=None,
                 layer_events=None, ffn_dim=0):
    """Replay one group of linear-attention layers from its anchors
    (sr_replay_group).  Returns states fp32 [n_gdn, N, h_v, d, d] (and conv
    states fp32 [n_gdn, N, conv_dim, width-1] if asked).  layer_events: one
    torch.cuda.Event (or None) per GDN layer, recorded as soon as that
    layer's state is written (layer-wise handoff).  packed_weights entries
    are pack_gdn_layer outputs, or (pack_gdn_layer, pack_ffn) pairs for
    layers followed by an FFN block of width ffn_dim."""
    desc, _keep, wts, states, conv, n_gdn, T = _group_prepare(
        anchors, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, conv_width, rms_eps,
        l2_eps, max_seqlen, want_conv_state, states, conv_states, layer_events, ffn_dim)
    lib = _lib.load()
    ws_bytes = int(lib.sr_replay_group_workspace_bytes(ctypes.byref(desc)))
    if ws_bytes == 0 and n_gdn and T > 0:
        raise ValueError("unsupported group shape")
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=anchors.device)
    else:
        _need(workspace, "workspace", torch.uint8, ndim=1, device=anchors.device)
        if workspace.numel() < ws_bytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, needs {ws_bytes}")
    st = lib.sr_replay_group(ctypes.byref(desc), wts, _ptr(anchors), _ptr(cu_seqlens),
                             _ptr(states), _ptr(conv), _ptr(workspace), workspace.numel(),
                             _stream())
    _lib.check("sr_replay_group", st)
    return (states, conv) if want_conv_state else states


def noalloc_max_bytes() -> int:
    """Size of the static per-GPU workspace of replay_group_noalloc."""
    return int(_lib.load().sr_replay_group_noalloc_max_bytes())


def replay_group_noalloc(anchors, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, *,
                         conv_width=4, rms_eps=1e-6, l2_eps=1e-6, max_seqlen=None,
                         want_conv_state=False, states=None, conv_states=None,
                         layer_events=None, ffn_dim=0):
    """replay_group without a workspace allocation (sr_replay_group_noalloc):
    the library's static per-GPU workspace is used.  Pass preallocated
    `states` (and `conv_states`) to keep the call free of allocations.
    Calls that overlap on one GPU race."""
    desc, _keep, wts, states, conv, n_gdn, T = _group_prepare(
        anchors, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, conv_width, rms_eps,
        l2_eps, max_seqlen, want_conv_state, states, conv_states, layer_events, ffn_dim)
    st = _lib.load().sr_replay_group_noalloc(ctypes.byref(desc), wts, _ptr(anchors),
                                             _ptr(cu_seqlens), _ptr(states), _ptr(conv),
                                             _stream())
    _lib.check("sr_replay_group_noalloc", st)
    return (states, conv) if want_conv_state else states


def extend_group(tokens, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, *,
                 initial_states=None, initial_conv_states=None, want_hidden=True,
                 conv_width=4, rms_eps=1e-6, l2_eps=1e-6, max_seqlen=None, states=None,
                 conv_states=None, workspace=None, layer_events=None, ffn_dim=0):
    """Continue a group from given per-layer states and conv windows over new
    tokens (sr_extend_group).  Returns (states, conv_states, hidden_out fp32
    [T, hidden] or None)."""
    desc, _keep, wts, states, conv, n_gdn, T = _group_prepare(
        tokens, packed_weights, cu_seqlens, layer_kind, h_k, h_v, d, conv_width, rms_eps,
        l2_eps, max_seqlen, True, states, conv_states, layer_events, ffn_dim)
    dev = tokens.device
    n = cu_seqlens.shape[0] - 1
    if initial_states is not None:
        _need(initial_states, "initial_states", torch.float32, (n_gdn, n, h_v, d, d), device=dev)
        if initial_states.data_ptr() == states.data_ptr():
            raise ValueError("states must not alias initial_states")
    if initial_conv_states is not None:
        _need(initial_conv_states, "initial_conv_states", torch.float32, tuple(conv.shape),
              device=dev)
        if initial_conv_states.data_ptr() == conv.data_ptr():
            raise ValueError("conv_states must not alias initial_conv_states")
    hidden = None
    if want_hidden:
        hidden = torch.empty((T, tokens.shape[1]), dtype=torch.float32, device=dev)
    lib = _lib.load()
    ws_bytes = int(lib.sr_replay_group_workspace_bytes(ctypes.byref(desc)))
    if ws_bytes == 0 and n_gdn and T > 0:
        raise ValueError("unsupported group shape")
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, ndim=1, device=dev)
        if workspace.numel() < ws_bytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, needs {ws_bytes}")
    st = lib.sr_extend_group(ctypes.byref(desc), wts, _ptr(tokens), _ptr(cu_seqlens),
                             _ptr(initial_states), _ptr(initial_conv_states), _ptr(states),
                             _ptr(conv), _ptr(hidden), _ptr(workspace), workspace.numel(),
                             _stream())
    _lib.check("sr_extend_group", st)
    return states, conv, hidden

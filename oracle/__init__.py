"""fp64 CPU oracle of the suffix-replay hot path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``linear_attention_state_anchor_amd``) and imports
nothing from it.  Inputs come from ``replay_inputs`` as stored bytes and are
widened exactly to fp64; every step runs in fp64.

Functions and the passages they follow:
  gdn            -- the per-token recurrence S_t = A_t(S_{t-1}) + B_t
                    ("SuffixReplay", Eq. 4; "Tail-Replay", section 2), in C
                    (gdn_oracle.c), erase and erase-free modes.
  gather_suffix  -- the last k_i anchors of each hit, packed varlen
                    ("SuffixReplay", Algorithm Design 2 and Pipelined Replay
                    Path: 64-token pages, one packed variable-length batch).
  anchor_positions, gather_anchors
                 -- token-wise sparse anchors: each 64-token page keeps the
                    anchors at a fixed set of in-page positions (density
                    1/16, concentrated next to the page boundary or spread
                    uniformly; "SuffixReplay", Algorithm Design 2, Figure 3),
                    and the replay takes the last k_i anchors.
  replay_budget  -- k = min(0.05 n, k_max) anchors ("SuffixReplay",
                    Algorithm Design 3), ceil of the exact decimal ratio.
  frontend, output_path, replay_group
                 -- one replay group run from its anchors, skipping
                    full-attention layers, from a zero state, the last
                    layer state-only ("SuffixReplay", Algorithm Design 1;
                    "Tail-Replay", section 3).  The layer internals (norms,
                    short conv, gates) are not written out on the pages;
                    the readings taken are listed at each function.
  rel_fro        -- relative Frobenius error in fp64.

Parity pins live in tests/test_oracle_*.py.  The layer-internal readings
(RMSNorm with unit weight, conv on q|k|v only, L2 norm, softplus/sigmoid
gates, gated RMSNorm, no FFN) have no page to pin them against real models:
for them parity is pinned only to their textbook definitions, not to a model.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None
_lock = threading.Lock()

GDN, FA = 0, 1


def build(force: bool = True) -> str:
    """Compile the C part of the oracle with gcc (fp64, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.oracle_gdn_f64.restype = ctypes.c_int
        lib.oracle_gdn_f64.argtypes = [i32, P, i32, i32, i32, i32, P, P, P, P,
                                       i32, P, i32, ctypes.c_double, P, P, P, i32]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(x):
    """Exact float64 copy of a stored tensor (bf16 bits, fp16, fp32 or fp64)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float16, np.float32, np.float64):
        return np.ascontiguousarray(x, dtype=np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def gdn(q, k, v, alpha, beta, cu_seqlens, h_k, h_v, *, alpha_is_log, erase=True,
        scale=1.0, initial_state=None, want_o=True, n_threads=0):
    """Gated-delta-rule replay in fp64, token by token (see gdn_oracle.c).

    q, k: [T][h_k][d_k]; v: [T][h_v][d_v] (bf16 bits, fp16, fp32 or fp64);
    alpha (or log alpha), beta: [T][h_v] (beta None means 1);
    cu_seqlens: [N+1] int32.  Returns (final_state [N][h_v][d_k][d_v] fp64,
    o [T][h_v][d_v] fp64 or None).
    """
    lib = _load()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    n = cu.shape[0] - 1
    kk = _f64(k)
    vv = _f64(v)
    T = int(cu[-1]) if cu.shape[0] else 0
    d_k = kk.shape[-1]
    d_v = vv.shape[-1]
    qq = _f64(q) if (want_o and q is not None) else None
    a = _f64(alpha)
    b = None if beta is None else _f64(beta)
    s0 = None if initial_state is None else _f64(initial_state)
    if kk.shape[0] < T or vv.shape[0] < T or a.shape[0] < T:
        raise ValueError("inputs shorter than cu_seqlens[-1]")
    final = np.zeros((max(n, 0), h_v, d_k, d_v), dtype=np.float64)
    o = np.zeros((T, h_v, d_v), dtype=np.float64) if qq is not None else None
    rc = lib.oracle_gdn_f64(n, _ptr(cu), h_k, h_v, d_k, d_v, _ptr(qq), _ptr(kk),
                            _ptr(vv), _ptr(a), int(bool(alpha_is_log)), _ptr(b),
                            int(bool(erase)), float(scale), _ptr(s0), _ptr(final),
                            _ptr(o), int(n_threads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_f64 failed ({rc})")
    return final, o


# ---------------------------------------------------------------------------
# anchor gather ("SuffixReplay", Algorithm Design 2: 64-token pages; System
# Design, Pipelined Replay Path: hits packed into one variable-length batch)
# ---------------------------------------------------------------------------
def gather_suffix(pool, page_table, matched_len, suffix_len, page=64):
    """Packed replay input: for hit i, anchors m_i-k_i .. m_i-1 of its prefix.

    pool: [P][page][hidden]; page_table[i][j] = physical page holding the
    prefix's tokens j*page .. j*page+page-1.  Returns (packed [T][hidden],
    cu_seqlens [N+1] int32) by plain fancy indexing.
    """
    m = np.asarray(matched_len, dtype=np.int64)
    k = np.asarray(suffix_len, dtype=np.int64)
    cu = np.zeros(m.shape[0] + 1, dtype=np.int64)
    cu[1:] = np.cumsum(k)
    rows = []
    for i in range(m.shape[0]):
        pos = np.arange(m[i] - k[i], m[i])
        rows.append(np.asarray(pool)[page_table[i][pos // page], pos % page])
    hidden = np.asarray(pool).shape[-1]
    packed = (np.concatenate(rows, axis=0) if rows else
              np.zeros((0, hidden), dtype=np.asarray(pool).dtype))
    return packed, cu.astype(np.int32)


def anchor_positions(m, page_offsets, page=64):
    """Prefix positions that hold an anchor, in increasing order, for a
    matched prefix of m tokens whose pages keep the anchors at the in-page
    positions page_offsets."""
    offs = sorted(int(o) for o in page_offsets)
    return [p * page + o for p in range((int(m) + page - 1) // page) for o in offs
            if p * page + o < int(m)]


def gather_anchors(pool, page_offsets, page_table, matched_len, suffix_len, page=64):
    """Packed replay input with token-wise sparse anchors.

    pool: [P][A][hidden]; block page_table[i][p] holds, in row j, request
    i's anchor at position p*page + page_offsets[j].  Anchor a of request i
    (counting its anchors in position order) therefore sits in block
    page_table[i][a // A], row a % A.  The packed rows are the last k_i
    anchors of each request.  Returns (packed [T][hidden], cu_seqlens [N+1]
    int32, positions [T] int32).
    """
    pool = np.asarray(pool)
    A = len(page_offsets)
    rows, positions = [], []
    cu = [0]
    for i in range(len(matched_len)):
        pos = anchor_positions(matched_len[i], page_offsets, page)
        k = int(suffix_len[i])
        if k > len(pos):
            raise ValueError(f"request {i}: {k} anchors asked, {len(pos)} held")
        for a in range(len(pos) - k, len(pos)):
            rows.append(pool[page_table[i][a // A], a % A])
            positions.append(pos[a])
        cu.append(cu[-1] + k)
    packed = (np.stack(rows) if rows else np.zeros((0, pool.shape[-1]), dtype=pool.dtype))
    return packed, np.asarray(cu, dtype=np.int32), np.asarray(positions, dtype=np.int32)


def replay_budget(n_anchors, ratio, k_max):
    """k_i = min(ceil(ratio * n_i), k_max) with the ratio taken as the exact
    decimal it is written as (k_max <= 0: no cap)."""
    from fractions import Fraction
    r = Fraction(str(ratio))
    out = []
    for n in n_anchors:
        k = -((-r.numerator * int(n)) // r.denominator)   # ceil(r n), exact
        if k_max > 0:
            k = min(k, int(k_max))
        out.append(int(k))
    return out


# ---------------------------------------------------------------------------
# replay group ("SuffixReplay", Algorithm Design 1; "Tail-Replay", section 3)
# ---------------------------------------------------------------------------
def rmsnorm_rows(x, eps):
    """x / sqrt(mean(x^2) + eps) per row, unit weight."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def l2norm_rows(x, eps):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def silu(x):
    with np.errstate(over="ignore"):  # exp overflow gives the exact limit 0
        return x / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, x)


def sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def causal_conv_silu(u, conv_w, cu_seqlens, initial_state=None):
    """Depthwise causal conv per sequence, then SiLU.

    y_t[c] = SiLU(sum_j w[c][j] * u_{t-W+1+j}[c]), with tap W-1 on the
    current token and, before each sequence start, the W-1 rows of
    initial_state [N][C][W-1] (oldest first) -- zeros when it is None, the
    replay case (an empty history).  Returns (y, conv_state [N][C][W-1]: the
    last W-1 rows of the history followed by the sequence, oldest first).
    """
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(conv_w, dtype=np.float64)
    W = w.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    y = np.zeros_like(u)
    n = cu.shape[0] - 1
    state = np.zeros((n, u.shape[1], W - 1))
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        hist = (np.zeros((W - 1, u.shape[1])) if initial_state is None else
                np.asarray(initial_state[s], dtype=np.float64).T)
        seg = np.concatenate([hist, u[a:b]], axis=0)
        acc = np.zeros((b - a, u.shape[1]))
        for j in range(W):
            acc += w[:, j][None, :] * seg[j:j + (b - a)]
        y[a:b] = silu(acc)
        state[s] = seg[seg.shape[0] - (W - 1):].T
    return y, state


def frontend(x, w_in, conv_w, cu_seqlens, h_k, h_v, d, rms_eps=1e-6,
             l2_eps=1e-6, conv_initial=None):
    """Pre-mixer RMSNorm, fused input projection, short conv + SiLU on q|k|v,
    per-head L2 norm of q and k, and the gates.

    Column order of w_in: q (h_k*d) | k (h_k*d) | v (h_v*d) | z (h_v*d) |
    a (h_v) | b (h_v).  log alpha = -softplus(a); beta = sigmoid(b).
    """
    x = np.asarray(x, dtype=np.float64)
    W = _f64(w_in)
    xh = rmsnorm_rows(x, rms_eps)
    p = xh @ W
    nq = h_k * d
    conv_dim = 2 * nq + h_v * d
    c, conv_state = causal_conv_silu(p[:, :conv_dim], _f64(conv_w), cu_seqlens,
                                     conv_initial)
    T = x.shape[0]
    q = l2norm_rows(c[:, :nq].reshape(T, h_k, d), l2_eps)
    k = l2norm_rows(c[:, nq:2 * nq].reshape(T, h_k, d), l2_eps)
    v = c[:, 2 * nq:conv_dim].reshape(T, h_v, d)
    z = p[:, conv_dim:conv_dim + h_v * d].reshape(T, h_v, d)
    a = p[:, conv_dim + h_v * d:conv_dim + h_v * d + h_v]
    b = p[:, conv_dim + h_v * d + h_v:conv_dim + h_v * d + 2 * h_v]
    return dict(q=q, k=k, v=v, z=z, log_alpha=-softplus(a), beta=sigmoid(b),
                conv_state=conv_state, u=p[:, :conv_dim], c=c)


def output_path(o, z, w_out, eps=1e-6):
    """Gated RMSNorm per value head (unit weight), then the output
    projection: returns y @ w_out with y = rms(o) * SiLU(z)."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    T = o.shape[0]
    y = rmsnorm_rows(o, eps) * silu(z)
    return y.reshape(T, -1) @ _f64(w_out)


def ffn_block(x, w_gate, w_up, w_down, eps=1e-6):
    """Pre-norm feed-forward block: x + (SiLU(x^ W_gate) * (x^ W_up)) W_down
    with x^ = RMSNorm(x), unit weight.  The pages give no FFN form; a SwiGLU
    FFN of the family the pages evaluate is taken."""
    xh = rmsnorm_rows(np.asarray(x, dtype=np.float64), eps)
    return x + (silu(xh @ _f64(w_gate)) * (xh @ _f64(w_up))) @ _f64(w_down)


def replay_group(anchors, weights, cu_seqlens, layer_kind, h_k, h_v, d,
                 rms_eps=1e-6, l2_eps=1e-6, return_trace=False):
    """Replay one group of linear-attention layers from its entry anchors.

    Full-attention entries are skipped (they carry no state into the replay;
    "SuffixReplay", Algorithm Design 1).  Every GDN layer starts from a zero
    state ("Tail-Replay", section 3).  Each intermediate layer is a pre-norm
    residual block x <- x + mixer(x); the last GDN layer of the group only
    produces its state, since the next group restarts from a cached
    full-attention hidden ("Tail-Replay", section 3, final-FFN skip).

    Returns (states [n_gdn][N][h_v][d][d], conv_states [n_gdn][N][conv][W-1]).
    """
    out = extend_group(anchors, weights, cu_seqlens, layer_kind, h_k, h_v, d, rms_eps=rms_eps,
                       l2_eps=l2_eps, want_hidden=False, return_trace=return_trace)
    return (out[0], out[1], out[3]) if return_trace else (out[0], out[1])


def extend_group(tokens, weights, cu_seqlens, layer_kind, h_k, h_v, d, initial_states=None,
                 initial_conv_states=None, rms_eps=1e-6, l2_eps=1e-6, want_hidden=True,
                 return_trace=False):
    """Run new tokens through one group from given per-layer states and conv
    windows ("Tail-Replay", section 3: the unmatched tokens continue from the
    reconstructed states).  With no initial states this is the replay above;
    with want_hidden the last layer also forms its mixer output and the
    group's output hidden states are returned.

    Returns (states, conv_states, hidden [T][hidden] or None, trace or None).
    """
    x = _f64(tokens)
    gdn_layers = [i for i, kind in enumerate(layer_kind) if kind == GDN]
    states, conv_states, trace = [], [], []
    hidden = None
    for li, idx in enumerate(gdn_layers):
        w = weights[li]
        last = li == len(gdn_layers) - 1
        full = not last or want_hidden
        fe = frontend(x, w.w_in, w.conv_w, cu_seqlens, h_k, h_v, d, rms_eps, l2_eps,
                      None if initial_conv_states is None else initial_conv_states[li])
        S, o = gdn(fe["q"], fe["k"], fe["v"], fe["log_alpha"], fe["beta"],
                   cu_seqlens, h_k, h_v, alpha_is_log=True, erase=True,
                   initial_state=None if initial_states is None else initial_states[li],
                   want_o=full)
        states.append(S)
        conv_states.append(fe["conv_state"])
        if return_trace:
            trace.append(dict(x=x, **fe, o=o))
        if full:
            x = x + output_path(o, fe["z"], w.w_out, rms_eps)
            # the FFN after the mixer ("Tail-Replay", section 3: replay omits
            # the group's final FFN -- it runs for the last layer only when
            # the group's output is asked for)
            if getattr(w, "w_gate", None) is not None:
                x = ffn_block(x, w.w_gate, w.w_up, w.w_down, rms_eps)
        if last and want_hidden:
            hidden = x
    st = np.stack(states) if states else np.zeros((0,))
    cs = np.stack(conv_states) if conv_states else np.zeros((0,))
    return st, cs, hidden, (trace if return_trace else None)


def rel_fro(x, ref):
    """||x - ref||_F / ||ref||_F in fp64 (||x||_F when ref is all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)

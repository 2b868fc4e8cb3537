"""Seeded synthetic inputs for the suffix-replay workloads.

This module only draws random tensors and rounds them to their storage types.
It holds none of the replay method's arithmetic, so both the fp64 oracle and
the HIP library can be fed from it without sharing code with each other.

Shapes and distributions follow the workloads the pages evaluate: matched
prefixes of 8K-32K tokens, replay budgets of 5-10 % of the prefix, 64-token
anchor pages ("SuffixReplay", Algorithm Design 2-3; "Tail-Replay" section 3
and 4).  The pages evaluate on LongBench/RULER/ShareGPT/ToolMind; none of those
is used here: every tensor is drawn from a fixed-seed NumPy PCG64 generator.

Storage conventions (shared by the oracle and the library, which both read
the same bytes):
  * bf16 tensors are numpy ``uint16`` arrays holding the bf16 bit patterns,
    rounded once from fp64 with round-to-nearest-even;
  * fp32 tensors are numpy ``float32`` arrays rounded once from fp64;
  * ``cu_seqlens`` is int32 with N+1 entries, cu[0] = 0, cu[N] = T.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "to_bf16_bits", "bf16_bits_to_f32", "widen", "GdnCase", "gdn_case",
    "config_c1", "config_c2", "config_c3", "GroupCase", "group_weights",
    "config_c4", "config_c5", "PoolCase", "suffix_pool_case", "CONFIG_SEEDS", "FFN_DIM",
]

CONFIG_SEEDS = {1: 101, 2: 102, 3: 103, 4: 104, 5: 105}


# --------------------------------------------------------------------------
# storage-type rounding
# --------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """Round an fp64/fp32 array to bf16 (round to nearest, ties to even).

    Rounds first to fp32 (exact for every value drawn here, which are far from
    fp32 ties) and then keeps the upper 16 bits with RNE on the lower 16.
    NaN is not produced by any generator here and is not handled specially.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def widen(x) -> np.ndarray:
    """Exact float64 view of a stored tensor (bf16 bits or float32)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# one GDN layer's recurrence inputs
# --------------------------------------------------------------------------
@dataclass
class GdnCase:
    """Inputs of one gated-delta-rule replay launch (packed varlen)."""
    q: np.ndarray            # [T][h_k][d_k]  bf16 bits or float32
    k: np.ndarray            # [T][h_k][d_k]
    v: np.ndarray            # [T][h_v][d_v]
    alpha: np.ndarray        # [T][h_v] float32: alpha, or log(alpha) if alpha_is_log
    beta: np.ndarray | None  # [T][h_v] float32, or None (= 1)
    cu_seqlens: np.ndarray   # [N+1] int32
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    dtype: str               # "bf16" | "f32"
    alpha_is_log: bool
    erase: bool
    initial_state: np.ndarray | None = None  # [N][h_v][d_k][d_v] float32
    meta: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        if self.n_seqs == 0:
            return 0
        return int(np.max(np.diff(self.cu_seqlens)))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _unit_rows(x: np.ndarray) -> np.ndarray:
    # Input recipe only: the configurations draw keys (and in some cases
    # queries) with unit L2 norm per head.  Normalised in fp64 before the
    # single rounding to the storage type.
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def gdn_case(lens, h_k, h_v, d, dtype="bf16", seed=0, *, normalize_q=False,
             normalize_k=True, alpha="softplus", beta="sigmoid", erase=True,
             initial_state=False, d_v=None) -> GdnCase:
    """Draw one packed varlen batch of GDN replay inputs.

    alpha: "softplus" -> log(alpha) = -softplus(N(0,1)) stored as log alpha;
           ("uniform", lo, hi) -> alpha ~ U[lo, hi] stored as alpha;
           "one" -> alpha = 1 (stored as alpha).
    beta:  "sigmoid" -> sigmoid(N(0,1)); "none" -> None (= 1);
           "zero" -> 0; "one" -> 1.
    Tensor draw order: q, k, v, alpha, beta, initial state.
    """
    lens = [int(x) for x in lens]
    d_k = int(d)
    d_v = int(d if d_v is None else d_v)
    T = int(sum(lens))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, h_k, d_k))
    k = rng.standard_normal((T, h_k, d_k))
    v = rng.standard_normal((T, h_v, d_v))
    if normalize_q:
        q = _unit_rows(q)
    if normalize_k:
        k = _unit_rows(k)
    if alpha == "softplus":
        a = -np.logaddexp(0.0, rng.standard_normal((T, h_v)))
        alpha_is_log = True
    elif alpha == "one":
        a = np.ones((T, h_v))
        alpha_is_log = False
    elif isinstance(alpha, tuple) and alpha[0] == "uniform":
        a = rng.uniform(alpha[1], alpha[2], size=(T, h_v))
        alpha_is_log = False
    else:
        raise ValueError(f"unknown alpha recipe {alpha!r}")
    if beta == "sigmoid":
        b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, h_v))))
    elif beta == "none":
        b = None
    elif beta == "zero":
        b = np.zeros((T, h_v))
    elif beta == "one":
        b = np.ones((T, h_v))
    else:
        raise ValueError(f"unknown beta recipe {beta!r}")
    s0 = None
    if initial_state:
        s0 = np.ascontiguousarray(
            rng.standard_normal((len(lens), h_v, d_k, d_v)), dtype=np.float32)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    if lens:
        cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64)).astype(np.int32)
    return GdnCase(
        q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
        alpha=np.ascontiguousarray(a, dtype=np.float32),
        beta=None if b is None else np.ascontiguousarray(b, dtype=np.float32),
        cu_seqlens=cu, h_k=int(h_k), h_v=int(h_v), d_k=d_k, d_v=d_v,
        dtype=dtype, alpha_is_log=alpha_is_log, erase=bool(erase),
        initial_state=s0, meta={"seed": seed, "lens": lens})


def config_c1(seed=CONFIG_SEEDS[1]) -> GdnCase:
    """1 sequence x 256 tokens, 4 heads, d = 64, fp32, unit keys."""
    c = gdn_case([256], 4, 4, 64, "f32", seed, normalize_q=False,
                 normalize_k=True)
    c.meta["name"] = "gdn 1x256 h4 d64 fp32"
    return c


def config_c2(seed=CONFIG_SEEDS[2], n_seqs=8, seqlen=2048, heads=32) -> GdnCase:
    """Erase-free (scalar decay) replay: 8 x 2048, 32 heads, d = 128, bf16,
    alpha ~ U[0.90, 0.999], no write gate."""
    c = gdn_case([seqlen] * n_seqs, heads, heads, 128, "bf16", seed,
                 normalize_q=False, normalize_k=False,
                 alpha=("uniform", 0.90, 0.999), beta="none", erase=False)
    c.meta["name"] = f"erase-free {n_seqs}x{seqlen} h{heads} d128 bf16"
    return c


def config_c3(seed=CONFIG_SEEDS[3], n_seqs=16, seqlen=3276) -> GdnCase:
    """GDN replay kernel alone: 16 x 3276 (10 % of a 32K prefix), 16 key /
    32 value heads, d = 128, bf16, unit q and k."""
    c = gdn_case([seqlen] * n_seqs, 16, 32, 128, "bf16", seed,
                 normalize_q=True, normalize_k=True)
    c.meta["name"] = f"gdn {n_seqs}x{seqlen} hk16 hv32 d128 bf16"
    return c


# --------------------------------------------------------------------------
# a replay group from anchors
# --------------------------------------------------------------------------
GDN, FA = 0, 1


@dataclass
class GroupWeights:
    """bf16 weights of one GDN layer (bit patterns), with an optional FFN
    block after it."""
    w_in: np.ndarray    # [hidden][n_in]  columns q | k | v | z | a | b
    conv_w: np.ndarray  # [conv_dim][width]  over the q|k|v channels
    w_out: np.ndarray   # [h_v*d_v][hidden]
    w_gate: np.ndarray | None = None  # [hidden][ffn]
    w_up: np.ndarray | None = None    # [hidden][ffn]
    w_down: np.ndarray | None = None  # [ffn][hidden]


@dataclass
class GroupCase:
    anchors: np.ndarray          # [T][hidden] bf16 bits
    cu_seqlens: np.ndarray       # [N+1] int32
    layer_kind: list             # GDN / FA per layer
    weights: list                # GroupWeights per GDN layer
    hidden: int
    h_k: int
    h_v: int
    d: int
    conv_width: int
    meta: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def group_weights(rng, hidden, h_k, h_v, d, conv_width=4, w_std=0.02,
                  conv_std=0.5, ffn_dim=0) -> GroupWeights:
    """Random-init bf16 weights of one GDN layer.

    Projection columns: q (h_k*d) | k (h_k*d) | v (h_v*d) | z (h_v*d) |
    a (h_v) | b (h_v), all N(0, w_std^2).  Conv taps N(0, conv_std^2) over the
    q|k|v channels.  Output projection N(0, w_std^2).  With ffn_dim > 0,
    FFN gate, up and down weights N(0, w_std^2) are drawn after the others.
    """
    n_in = 2 * h_k * d + 2 * h_v * d + 2 * h_v
    conv_dim = 2 * h_k * d + h_v * d
    w_in = to_bf16_bits(rng.standard_normal((hidden, n_in), dtype=np.float32)
                        * np.float32(w_std))
    conv_w = to_bf16_bits(rng.standard_normal((conv_dim, conv_width),
                                              dtype=np.float32)
                          * np.float32(conv_std))
    w_out = to_bf16_bits(rng.standard_normal((h_v * d, hidden),
                                             dtype=np.float32)
                         * np.float32(w_std))
    gw = GroupWeights(w_in=w_in, conv_w=conv_w, w_out=w_out)
    if ffn_dim:
        draw = lambda shape: to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)
                                          * np.float32(w_std))
        gw.w_gate = draw((hidden, ffn_dim))
        gw.w_up = draw((hidden, ffn_dim))
        gw.w_down = draw((ffn_dim, hidden))
    return gw


def _group(lens, seed, hidden, h_k, h_v, d, layer_kind, conv_width=4, ffn_dim=0):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    anchors = to_bf16_bits(rng.standard_normal((T, hidden), dtype=np.float32))
    weights = [group_weights(rng, hidden, h_k, h_v, d, conv_width, ffn_dim=ffn_dim)
               for kind in layer_kind if kind == GDN]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    if lens:
        cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64)).astype(np.int32)
    return GroupCase(anchors=anchors, cu_seqlens=cu, layer_kind=list(layer_kind),
                     weights=weights, hidden=hidden, h_k=h_k, h_v=h_v, d=d,
                     conv_width=conv_width, meta={"seed": seed, "lens": list(lens),
                                                  "ffn_dim": ffn_dim})


FFN_DIM = 9728  # FFN width taken for the hidden-2560 layers (see the group oracle)


def config_c4(seed=CONFIG_SEEDS[4], n_seqs=4, suffix=1638, hidden=2560,
              h_k=16, h_v=32, d=128, ffn_dim=0) -> GroupCase:
    """Replay group: 3 GDN layers then a skipped full-attention layer,
    hidden 2560, 4 requests x 1638 anchors (5 % of 32K); with ffn_dim, an
    FFN block after each GDN layer."""
    g = _group([suffix] * n_seqs, seed, hidden, h_k, h_v, d, [GDN, GDN, GDN, FA],
               ffn_dim=ffn_dim)
    g.meta["name"] = f"group {n_seqs}x{suffix} D{hidden} 3xGDN+FA"
    return g


# --------------------------------------------------------------------------
# paged anchor pool for the varlen gather
# --------------------------------------------------------------------------
PAGE = 64  # tokens per anchor page ("SuffixReplay", Algorithm Design 2)


@dataclass
class PoolCase:
    """A paged pool of cached anchors and one batch of prefix-cache hits."""
    n_pages: int
    hidden: int
    page_table: np.ndarray    # [n_req][max_pages] int32 physical page ids
    matched_len: np.ndarray   # [n_req] int32  m_i
    suffix_len: np.ndarray    # [n_req] int32  k_i
    seed: int
    meta: dict = field(default_factory=dict)

    def pool_pages(self, page_ids) -> np.ndarray:
        """bf16 bits of the listed physical pages, [len][64][hidden].

        Page p is drawn from its own generator seeded with (seed, p), so any
        subset of the pool can be produced without the rest.
        """
        out = np.empty((len(page_ids), PAGE, self.hidden), dtype=np.uint16)
        for i, p in enumerate(page_ids):
            rng = np.random.default_rng([self.seed, 7, int(p)])
            out[i] = to_bf16_bits(
                rng.standard_normal((PAGE, self.hidden), dtype=np.float32))
        return out

    def pool(self) -> np.ndarray:
        return self.pool_pages(range(self.n_pages))


def suffix_pool_case(n_req, m_lo, m_hi, r_lo, r_hi, hidden, seed,
                     spare_pages=0) -> PoolCase:
    """Draw n_req cache hits: matched length m ~ U{m_lo..m_hi}, replay ratio
    r ~ U[r_lo, r_hi], replay length k = ceil(r*m) ("Tail-Replay", section 3).

    Each request owns ceil(m/64) pages; the physical page ids of all
    requests are one random permutation of the pool, so gathers are
    non-contiguous.
    """
    rng = np.random.default_rng(seed)
    m = rng.integers(m_lo, m_hi, endpoint=True, size=n_req).astype(np.int64)
    r = rng.uniform(r_lo, r_hi, size=n_req)
    k = np.array([min(int(mi), max(1, math.ceil(ri * mi))) for ri, mi in zip(r, m)],
                 dtype=np.int64)
    pages_per = (m + PAGE - 1) // PAGE
    n_pages = int(pages_per.sum()) + int(spare_pages)
    perm = rng.permutation(n_pages).astype(np.int32)
    max_pages = int(pages_per.max()) if n_req else 0
    pt = np.full((n_req, max(max_pages, 1)), -1, dtype=np.int32)
    off = 0
    for i in range(n_req):
        pt[i, :pages_per[i]] = perm[off:off + pages_per[i]]
        off += int(pages_per[i])
    return PoolCase(n_pages=n_pages, hidden=hidden, page_table=pt,
                    matched_len=m.astype(np.int32), suffix_len=k.astype(np.int32),
                    seed=seed, meta={"r": r})


def config_c5(seed=CONFIG_SEEDS[5], n_req=64, hidden=2560):
    """Varlen batched replay: 64 hits, m ~ U{8192..32768}, k = ceil(r m) with
    r ~ U[0.05, 0.10]; the replay group has the layer shapes of config_c4.

    Returns (pool case, per-layer weights as a GroupCase without anchors)."""
    pc = suffix_pool_case(n_req, 8192, 32768, 0.05, 0.10, hidden, seed)
    rng = np.random.default_rng([seed, 1])
    weights = [group_weights(rng, hidden, 16, 32, 128) for _ in range(3)]
    return pc, weights

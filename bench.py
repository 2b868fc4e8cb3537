"""Benchmark of the suffix-replay hot path on one MI355X.

Default workload: the gated-delta-rule replay of one GDN layer for 16 hits of
a 32K-token matched prefix with a 10 % replay budget (k = 3276 anchors each),
16 key / 32 value heads, d = 128, bf16 inputs, chunk 64 -- the configuration
the headline metric (replayed tokens/s per GDN layer and the fraction of the
roofline) is quoted on.  A step is one replay of that batch through
sr_gdn_replay_state (states + per-token outputs), inputs resident in HBM.

Prints one JSON line.  `--gpus N` with N > 1 exits: this build runs on one
GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0  # dense fp16/bf16 matrix cores


def gdn_algorithmic(n_seqs, seqlen, h_k, h_v, d, in_bytes=2, out_bytes=2, chunk=64,
                    want_o=True, erase=True):
    """Algorithmic bytes (each input read once, each output written once) and
    nominal matrix-core FLOPs of the chunked algorithm for one launch."""
    T = n_seqs * seqlen
    byts = T * h_k * d * in_bytes                    # k
    byts += T * h_v * d * in_bytes                   # v
    byts += T * h_v * 4 * (2 if erase else 1)        # alpha (+ beta)
    byts += n_seqs * h_v * d * d * 4                 # final state
    if want_o:
        byts += T * h_k * d * in_bytes               # q
        byts += T * h_v * d * out_bytes              # o
    C = chunk
    if erase and want_o:
        per = 10 * C * d + 6 * d * d + C * C / 3
    elif erase:
        per = 6 * C * d + 4 * d * d + C * C / 3
    elif want_o:
        per = 4 * C * d + 4 * d * d
    else:
        per = 2 * d * d
    flops = T * h_v * per
    return byts, flops


def kernel_source_hash():
    p = os.path.join(ROOT, "linear_attention_state_anchor_amd", "csrc", "gdn_chunk.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def read_traffic(bytes_alg):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "gdn_chunk_gdn16x3276_pmc.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on whole sequences of the same
    workload, as many as fit about budget_s of host time on all host threads,
    and on one sequence with a single thread.  Returns (baseline entry,
    sequences timed, oracle final states, oracle outputs) -- the outputs let
    the benchmarked launch be checked against the oracle."""
    import numpy as np
    import oracle
    from replay_inputs import gdn_case

    cu = case.cu_seqlens

    def sub(seqs):
        idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
        c = gdn_case([int(cu[s + 1] - cu[s]) for s in seqs], case.h_k, case.h_v, case.d_k,
                     case.dtype, seed=0, erase=case.erase)
        c.q, c.k, c.v, c.alpha = case.q[idx], case.k[idx], case.v[idx], case.alpha[idx]
        c.beta = None if case.beta is None else case.beta[idx]
        c.alpha_is_log = case.alpha_is_log
        return c

    def run(c, threads=0):
        t0 = time.perf_counter()
        S, o = oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, c.h_k, c.h_v,
                          alpha_is_log=c.alpha_is_log, erase=c.erase, n_threads=threads)
        return time.perf_counter() - t0, S, o

    threads = oracle.max_threads()
    first = sub([0])
    t1, _, _ = run(first)
    n = int(max(1, min(case.n_seqs, budget_s // max(t1, 1e-3))))
    seqs = list(range(n))
    c = sub(seqs)
    t, S, o = run(c)
    t_one, _, _ = run(first, threads=1)
    toks = c.total_tokens
    entry = {"value": toks / t, "unit": "replayed tokens/s per GDN layer", "cores": threads,
             "kind": "oracle", "cpu_model": cpu_model(),
             "one_core_value": first.total_tokens / t_one,
             "sample": f"{n} of {case.n_seqs} sequences ({toks} tokens, all {case.h_v} value "
                       f"heads), fp64 token loop, {t:.2f} s on {threads} threads; one "
                       f"sequence ({first.total_tokens} tokens) on 1 thread in {t_one:.2f} s"}
    return entry, seqs, S, o


def parity_vs_oracle(S_gpu, o_gpu, case, seqs, S_ref, o_ref):
    """Relative Frobenius error of the benchmarked launch's states and outputs
    against the oracle on the sequences it ran, and the worst (sequence, head)
    block of each."""
    import numpy as np
    import torch
    cu = case.cu_seqlens
    S = S_gpu[seqs].double().cpu().numpy()
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    o = o_gpu[torch.from_numpy(rows).to(o_gpu.device)].float().cpu().numpy()

    def rel(x, r):
        return float(np.linalg.norm(x - r) / np.linalg.norm(r))
    worst_S = max(rel(S[i, h], S_ref[i, h]) for i in range(len(seqs)) for h in range(case.h_v))
    worst_o, off = 0.0, 0
    for s in seqs:
        L = int(cu[s + 1] - cu[s])
        for h in range(case.h_v):
            worst_o = max(worst_o, rel(o[off:off + L, h], o_ref[off:off + L, h]))
        off += L
    return {"rel_S": rel(S, S_ref), "rel_o": rel(o, o_ref), "worst_head_S": worst_S,
            "worst_head_o": worst_o, "sequences": f"{len(seqs)} of {case.n_seqs}",
            "tolerance": 2e-3}


def group_flops(T, hidden, h_k, h_v, d, n_gdn, chunk=64):
    """Nominal matrix-core FLOPs of one group replay: projections, the chunked
    recurrence (outputs for all but the last layer) and output projections."""
    n_in = 2 * h_k * d + 2 * h_v * d + 2 * h_v
    n_last = (h_k + h_v) * d + 2 * h_v
    f = 0.0
    for li in range(n_gdn):
        last = li == n_gdn - 1
        f += 2.0 * T * hidden * (n_last if last else n_in)
        _, fl = gdn_algorithmic(1, T, h_k, h_v, d, want_o=not last)
        f += fl
        if not last:
            f += 2.0 * T * h_v * d * hidden
    return f


def time_steps(fn, steps, warmup):
    """Time `steps` calls of fn after `warmup` untimed ones.  The timed region
    is bracketed by device synchronisations; a HIP event on the current
    stream (the stream the library launches on) follows every call, so both
    the whole-run mean and the per-call distribution are measured.  Returns
    milliseconds: mean (total / steps), median, p10, p90, min, max."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))

    def pct(q):
        return per[min(len(per) - 1, int(round(q * (len(per) - 1))))]
    return {"mean_ms": ev[0].elapsed_time(ev[-1]) / steps, "median_ms": pct(0.5),
            "p10_ms": pct(0.1), "p90_ms": pct(0.9), "min_ms": per[0], "max_ms": per[-1]}


def time_cold(fn, reps=20, scrub_mib=512):
    """Median time of fn with a 512 MiB read-only sweep before each call,
    which fills the 256 MB infinity cache (MALL) and the L2s with other,
    clean lines, so the call reads its inputs from HBM and evicts nothing
    that needs writing back: the cold counterpart of time_steps' warm
    figure.  Only the call is inside the events."""
    import torch
    scrub = torch.ones(((scrub_mib << 20) // 4,), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(reps):
        scrub.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    del scrub
    per.sort()
    return per[len(per) // 2]


def replay_entry(t, T, byts, flops):
    ms = t["mean_ms"]
    sec = ms / 1e3
    return {"ms_per_step": ms, "median_ms": t["median_ms"], "p10_ms": t["p10_ms"],
            "p90_ms": t["p90_ms"], "replayed_tokens_per_s": T / sec,
            "hbm_gbs": byts / sec / 1e9, "hbm_frac": byts / sec / 1e9 / HBM_PEAK_GBS,
            "mfma_tflops": flops / sec / 1e12,
            "mfma_frac": flops / sec / 1e12 / MFMA_F16_PEAK_TFS,
            "bytes_per_launch": byts, "flop_per_launch": flops}


def bench_replay_variants(steps, warmup, to_dev, q, k, v, alpha, beta, cu, S):
    """Secondary single-layer replay measurements: the headline workload in
    state-only mode (no q, no o: the last layer of a group), and the
    erase-free (scalar-decay) 8 x 2048, 32-head workload with outputs."""
    import torch
    import linear_attention_state_anchor_amd as sr
    from replay_inputs import config_c2

    n, L, hk, hv, d = S.shape[0], 3276, k.shape[1], v.shape[1], k.shape[2]
    T = k.shape[0]
    t = time_steps(lambda: sr.gdn_replay_state(None, k, v, alpha, beta, cu, None,
                                               alpha_is_log=True, want_o=False,
                                               final_state=S), steps, warmup)
    byts, flops = gdn_algorithmic(n, L, hk, hv, d, want_o=False)
    out = {"state_only": dict(workload="headline replay without q and o (state only)",
                              **replay_entry(t, T, byts, flops))}
    c = config_c2()
    q2, k2, v2, a2, cu2 = (to_dev(x) for x in (c.q, c.k, c.v, c.alpha, c.cu_seqlens))
    S2 = torch.empty((c.n_seqs, c.h_v, c.d_k, c.d_v), dtype=torch.float32, device=k.device)
    o2 = torch.empty((c.total_tokens, c.h_v, c.d_v), dtype=torch.bfloat16, device=k.device)
    t = time_steps(lambda: sr.gdn_replay_state(q2, k2, v2, a2, None, cu2, None, erase=False,
                                               alpha_is_log=c.alpha_is_log,
                                               final_state=S2, o=o2), steps, warmup)
    byts, flops = gdn_algorithmic(c.n_seqs, c.total_tokens // c.n_seqs, c.h_k, c.h_v, c.d_k,
                                  erase=False)
    out["erase_free"] = dict(workload="erase-free (scalar decay) replay, 8 x 2048, 32 heads, "
                                      "d=128, bf16 in/out, beta = 1",
                             **replay_entry(t, c.total_tokens, byts, flops))
    out["erase_free"]["cold_median_ms"] = time_cold(
        lambda: sr.gdn_replay_state(q2, k2, v2, a2, None, cu2, None, erase=False,
                                    alpha_is_log=c.alpha_is_log, final_state=S2, o=o2))
    return out


def bench_group(steps, warmup, to_dev):
    """3-layer replay group (hidden 2560) from 4 x 1638 anchors; the varlen
    path: 64 hits gathered from a paged pool of full prefixes and replayed
    through the same group shapes; and the sparse-anchor path: the same 64
    hits with anchors kept at density 1/16 next to each page boundary and a
    replay of k = min(ceil(0.05 n), 512) anchors."""
    import numpy as np
    import torch
    import linear_attention_state_anchor_amd as sr
    from replay_inputs import PAGE, config_c4, config_c5

    out = {}
    g = config_c4()
    packed = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32, 128)
              for w in g.weights]
    anchors, cu = to_dev(g.anchors), to_dev(g.cu_seqlens)
    T = g.total_tokens
    states = torch.empty((3, g.n_seqs, 32, 128, 128), dtype=torch.float32, device="cuda:0")
    ws = torch.empty((sr.group_workspace_bytes(T, 2560, 16, 32, 128, n_seqs=g.n_seqs,
                                               layer_kind=g.layer_kind),),
                     dtype=torch.uint8, device="cuda:0")
    t = time_steps(lambda: sr.replay_group(anchors, packed, cu, g.layer_kind, 16, 32, 128,
                                           states=states, workspace=ws), steps, warmup)
    fl = group_flops(T, 2560, 16, 32, 128, 3)
    ms = t["mean_ms"]
    out["group"] = {
        "workload": "3 GDN layers + skipped FA, hidden 2560, 4 requests x 1638 anchors "
                    "(5% of 32K), bf16 anchors and weights",
        "ms_per_step": ms, "median_ms": t["median_ms"], "p10_ms": t["p10_ms"],
        "p90_ms": t["p90_ms"], "replayed_tokens_per_s_per_layer": 3 * T / (ms / 1e3),
        "tflops": fl / (ms / 1e3) / 1e12, "mfma_frac": fl / (ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS,
    }
    del ws
    # the same group with an FFN block after each intermediate layer
    from replay_inputs import FFN_DIM
    gf = config_c4(ffn_dim=FFN_DIM)
    packed_f = [(sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32,
                                   128),
                 sr.pack_ffn(to_dev(w.w_gate), to_dev(w.w_up), to_dev(w.w_down)))
                for w in gf.weights]
    wsf = torch.empty((sr.group_workspace_bytes(T, 2560, 16, 32, 128, n_seqs=g.n_seqs,
                                                layer_kind=g.layer_kind, ffn_dim=FFN_DIM),),
                      dtype=torch.uint8, device="cuda:0")
    af = to_dev(gf.anchors)
    t = time_steps(lambda: sr.replay_group(af, packed_f, cu, g.layer_kind, 16, 32, 128,
                                           states=states, workspace=wsf, ffn_dim=FFN_DIM),
                   steps, warmup)
    flf = fl + 2 * 3 * 2.0 * T * 2560 * FFN_DIM
    ms = t["mean_ms"]
    out["group_ffn"] = {
        "workload": f"the 4 x 1638 group with a SwiGLU FFN (width {FFN_DIM}) after the two "
                    f"intermediate GDN layers (the last layer's FFN is skipped)",
        "ms_per_step": ms, "median_ms": t["median_ms"],
        "replayed_tokens_per_s_per_layer": 3 * T / (ms / 1e3),
        "tflops": flf / (ms / 1e3) / 1e12, "mfma_frac": flf / (ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS,
    }
    del wsf, packed_f
    # varlen: gather + group
    pc, wts = config_c5()
    packed5 = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32, 128)
               for w in wts]
    gen = torch.Generator(device="cuda:0").manual_seed(105)
    pool = torch.randn((pc.n_pages, PAGE, 2560), generator=gen, device="cuda:0",
                       dtype=torch.float32).to(torch.bfloat16)
    pt, ml, sl = to_dev(pc.page_table), to_dev(pc.matched_len), to_dev(pc.suffix_len)
    T5 = int(pc.suffix_len.sum())
    packed_anchors = torch.empty((T5, 2560), dtype=torch.bfloat16, device="cuda:0")
    cu5 = torch.empty((65,), dtype=torch.int32, device="cuda:0")
    ws5 = torch.empty((sr.group_workspace_bytes(T5, 2560, 16, 32, 128, n_seqs=64),),
                      dtype=torch.uint8, device="cuda:0")
    states5 = torch.empty((3, 64, 32, 128, 128), dtype=torch.float32, device="cuda:0")
    gather = lambda: sr.gather_suffix(pool, pt, ml, sl, T5, packed=packed_anchors, cu_seqlens=cu5)
    tg = time_steps(gather, steps, warmup)

    def path():
        gather()
        sr.replay_group(packed_anchors, packed5, cu5, [0, 0, 0, 1], 16, 32, 128,
                        max_seqlen=int(pc.suffix_len.max()), states=states5, workspace=ws5)
    tp = time_steps(path, max(2, steps // 5), 1)
    fl5 = group_flops(T5, 2560, 16, 32, 128, 3)
    gb = 2 * T5 * 2560 * 2 / 1e9
    ms_p, ms_g = tp["mean_ms"], tg["mean_ms"]
    out["varlen"] = {
        "workload": f"64 hits, m ~ U{{8192..32768}}, k = ceil(r m), r ~ U[0.05,0.10] "
                    f"(T = {T5}), gather from 64-token pages + 3-layer group, hidden 2560",
        "ms_per_step": ms_p, "median_ms": tp["median_ms"],
        "replayed_tokens_per_s_per_layer": 3 * T5 / (ms_p / 1e3),
        "tflops": fl5 / (ms_p / 1e3) / 1e12, "mfma_frac": fl5 / (ms_p / 1e3) / 1e12 / MFMA_F16_PEAK_TFS,
        "gather_ms": ms_g, "gather_median_ms": tg["median_ms"], "gather_gbs": gb / (ms_g / 1e3),
        "gather_hbm_frac": gb / (ms_g / 1e3) / HBM_PEAK_GBS,
    }
    del pool, ws5, packed_anchors
    # sparse anchors: 4 of every 64 positions (next to the page boundary)
    offs = sr.DENSE_NEAR_BOUNDARY_1_16
    m = [int(x) for x in pc.matched_len]
    n_anchor = [len(offs) * (x // PAGE) + sum(o < x % PAGE for o in offs) for x in m]
    k_sp = sr.replay_budget(n_anchor, 0.05, 512)
    Ts = sum(k_sp)
    spool = torch.randn((pc.n_pages, len(offs), 2560), generator=gen, device="cuda:0",
                        dtype=torch.float32).to(torch.bfloat16)
    ksp = to_dev(np.asarray(k_sp, np.int32))
    sp_anchors = torch.empty((Ts, 2560), dtype=torch.bfloat16, device="cuda:0")
    cus = torch.empty((65,), dtype=torch.int32, device="cuda:0")
    wss = torch.empty((sr.group_workspace_bytes(Ts, 2560, 16, 32, 128, n_seqs=64),),
                      dtype=torch.uint8, device="cuda:0")
    sgather = lambda: sr.gather_anchors(spool, offs, pt, ml, ksp, Ts, packed=sp_anchors,
                                        cu_seqlens=cus, positions=False)
    tsg = time_steps(sgather, steps, warmup)

    def spath():
        sgather()
        sr.replay_group(sp_anchors, packed5, cus, [0, 0, 0, 1], 16, 32, 128,
                        max_seqlen=max(k_sp), states=states5, workspace=wss)
    tsp = time_steps(spath, steps, warmup)
    fls = group_flops(Ts, 2560, 16, 32, 128, 3)
    ms_s = tsp["mean_ms"]
    out["sparse_anchors"] = {
        "workload": f"the same 64 hits with anchors at density 1/16 next to each page "
                    f"boundary, k = min(ceil(0.05 n), 512) anchors (T = {Ts}), gather + "
                    f"3-layer group, hidden 2560",
        "ms_per_step": ms_s, "median_ms": tsp["median_ms"],
        "replayed_anchors_per_s_per_layer": 3 * Ts / (ms_s / 1e3),
        "tflops": fls / (ms_s / 1e3) / 1e12,
        "gather_ms": tsg["mean_ms"],
        "gather_gbs": 2 * Ts * 2560 * 2 / 1e9 / (tsg["mean_ms"] / 1e3),
    }
    return out


def bench_continuation_and_handoff(steps, warmup, to_dev):
    """Single-token decode from reconstructed states (64 sequences x 32
    heads, d = 128: each state read and written once), the sparse-anchor
    gather from a pinned host-memory pool (over the host link) and its
    overlap with a replay on another stream, and a small batch through the
    group as an eager call against its bucketed HIP graph."""
    import numpy as np
    import torch
    import linear_attention_state_anchor_amd as sr
    from linear_attention_state_anchor_amd.graphs import GroupReplayGraphs
    from replay_inputs import PAGE, config_c5, gdn_case

    out = {}
    # decode step
    c = gdn_case([1] * 64, 16, 32, 128, "bf16", seed=7, normalize_q=True)
    q, k, v, a, b = (to_dev(x) for x in (c.q, c.k, c.v, c.alpha, c.beta))
    S = torch.randn((64, 32, 128, 128), dtype=torch.float32, device="cuda:0") * 0.1
    o = torch.empty((64, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    t = time_steps(lambda: sr.gdn_decode_step(q, k, v, a, b, S, alpha_is_log=True, o=o),
                   steps, warmup)
    byts = 2 * S.numel() * 4 + 64 * (2 * 16 + 2 * 32) * 128 * 2 + 64 * 32 * 8
    out["decode_step"] = {
        "workload": "one decode token for 64 sequences from their states, 16 key / 32 value "
                    "heads, d=128, fp32 state in place, bf16 in/out",
        "ms_per_step": t["mean_ms"], "median_ms": t["median_ms"],
        "tokens_per_s": 64 / (t["mean_ms"] / 1e3),
        "hbm_gbs": byts / (t["mean_ms"] / 1e3) / 1e9,
        "hbm_frac": byts / (t["mean_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": byts}
    tc = time_cold(lambda: sr.gdn_decode_step(q, k, v, a, b, S, alpha_is_log=True, o=o))
    out["decode_step"].update({"cold_median_ms": tc,
                               "cold_hbm_frac": byts / (tc / 1e3) / 1e9 / HBM_PEAK_GBS})
    del S
    # sparse anchors kept in pinned host memory, gathered over the host link
    pc, wts = config_c5()
    offs = sr.DENSE_NEAR_BOUNDARY_1_16
    m = [int(x) for x in pc.matched_len]
    n_anchor = [len(offs) * (x // PAGE) + sum(o_ < x % PAGE for o_ in offs) for x in m]
    k_sp = sr.replay_budget(n_anchor, 0.05, 512)
    Ts = sum(k_sp)
    hpool = torch.empty((pc.n_pages, len(offs), 2560), dtype=torch.bfloat16).pin_memory()
    hpool.view(torch.int16).random_(-16000, 16000)
    pt, ml = to_dev(pc.page_table), to_dev(pc.matched_len)
    ksp = to_dev(np.asarray(k_sp, np.int32))
    sp = torch.empty((Ts, 2560), dtype=torch.bfloat16, device="cuda:0")
    cus = torch.empty((65,), dtype=torch.int32, device="cuda:0")
    hg = lambda: sr.gather_anchors(hpool, offs, pt, ml, ksp, Ts, packed=sp, cu_seqlens=cus,
                                   positions=False)
    tg = time_steps(hg, steps, warmup)
    # overlap: the host gather on a copy stream next to a replay on this one
    packed5 = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32, 128)
               for w in wts]
    anchors_prev = torch.randn((Ts, 2560), device="cuda:0").to(torch.bfloat16)
    cu_prev = cus.clone()
    hg()
    torch.cuda.synchronize()
    cu_prev.copy_(cus)
    st = torch.empty((3, 64, 32, 128, 128), dtype=torch.float32, device="cuda:0")
    ws = torch.empty((sr.group_workspace_bytes(Ts, 2560, 16, 32, 128, n_seqs=64),),
                     dtype=torch.uint8, device="cuda:0")
    replay = lambda: sr.replay_group(anchors_prev, packed5, cu_prev, [0, 0, 0, 1], 16, 32, 128,
                                     states=st, workspace=ws)
    tr = time_steps(replay, max(3, steps // 4), 2)
    copy_stream = torch.cuda.Stream()

    def both():
        copy_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(copy_stream):
            hg()
        replay()
        torch.cuda.current_stream().wait_stream(copy_stream)
    tb = time_steps(both, max(3, steps // 4), 2)
    gb = Ts * 2560 * 2 / 1e9
    out["host_pool_gather"] = {
        "workload": f"sparse anchors (1/16, next to the page boundary) of the 64 varlen hits in "
                    f"pinned host memory, k = min(ceil(0.05 n), 512) (T = {Ts}), gathered over "
                    f"the host link; next to a 3-layer group replay of a previous batch on "
                    f"another stream",
        "gather_ms": tg["mean_ms"], "host_link_gbs": gb / (tg["mean_ms"] / 1e3),
        "replay_ms": tr["mean_ms"], "gather_and_replay_overlapped_ms": tb["mean_ms"],
        "serial_sum_ms": tg["mean_ms"] + tr["mean_ms"]}
    del hpool, ws, st
    # small batches, where launching about two dozen kernels one by one
    # costs host time: eager library call against the graph of its bucket
    g4 = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32, 128)
          for w in wts]
    graphs = GroupReplayGraphs(g4, [0, 0, 0, 1], 16, 32, 128, 2560, buckets=(64, 512),
                               max_requests=4)
    for n_tok in (64, 512):
        small = torch.randn((n_tok, 2560), device="cuda:0").to(torch.bfloat16)
        cu4 = to_dev(np.arange(0, n_tok + 1, n_tok // 4, dtype=np.int32))
        st4 = torch.empty((3, 4, 32, 128, 128), dtype=torch.float32, device="cuda:0")
        ws4 = torch.empty((sr.group_workspace_bytes(n_tok, 2560, 16, 32, 128, n_seqs=4),),
                          dtype=torch.uint8, device="cuda:0")
        te = time_steps(lambda: sr.replay_group(small, g4, cu4, [0, 0, 0, 1], 16, 32, 128,
                                                states=st4, workspace=ws4), steps, warmup)
        graphs.run(small, cu4)
        tgr = time_steps(lambda: graphs.run(small, cu4), steps, warmup)
        out[f"graph_bucket_{n_tok}"] = {
            "workload": f"4 requests x {n_tok // 4} anchors through the 3-layer hidden-2560 "
                        f"group: eager library call against run() of its {n_tok}-token bucket "
                        f"graph (input copies included)",
            "eager_ms": te["mean_ms"], "graph_ms": tgr["mean_ms"]}
    return out


def error_vs_k(to_dev, n_req=8, ks=(16, 32, 64, 128, 256, 512)):
    """Replay error against the replay length (untimed report).

    For n_req hits of the varlen workload, the full-prefix state of every GDN
    layer (Eq. 1: the state is a function of all m inputs) is rebuilt from all
    m anchors, and compared with the suffix replay of the last k anchors (Eq. 2)
    for k in ks and k = ceil(0.05 m), ceil(0.10 m).  Relative Frobenius error
    per layer, over all heads of the n_req requests."""
    import math
    import numpy as np
    import torch
    import linear_attention_state_anchor_amd as sr
    from replay_inputs import PAGE, config_c5

    pc, wts = config_c5()
    packed = [sr.pack_gdn_layer(to_dev(w.w_in), to_dev(w.conv_w), to_dev(w.w_out), 16, 32, 128)
              for w in wts]
    gen = torch.Generator(device="cuda:0").manual_seed(105)
    pool = torch.randn((pc.n_pages, PAGE, 2560), generator=gen, device="cuda:0",
                       dtype=torch.float32).to(torch.bfloat16)
    sel = list(range(n_req))
    m = pc.matched_len[sel].astype(np.int32)
    pt = to_dev(np.ascontiguousarray(pc.page_table[sel]))
    ml = to_dev(m)

    def states_for(klist):
        kk = np.minimum(np.asarray(klist, np.int32), m)
        anchors, cu = sr.gather_suffix(pool, pt, ml, to_dev(kk), int(kk.sum()))
        S = sr.replay_group(anchors, packed, cu, [0, 0, 0, 1], 16, 32, 128,
                            max_seqlen=int(kk.max()))
        return S.double()

    full = states_for(m)
    rows = []
    for label, klist in ([(str(k), [k] * n_req) for k in ks] +
                         [("ceil(0.05m)", [math.ceil(0.05 * int(x)) for x in m]),
                          ("ceil(0.10m)", [math.ceil(0.10 * int(x)) for x in m])]):
        S = states_for(klist)
        err = [float(torch.linalg.vector_norm(S[l] - full[l]) / torch.linalg.vector_norm(full[l]))
               for l in range(full.shape[0])]
        rows.append({"k": label, "rel_fro_per_layer": err})
    out = {"group": {"workload": f"{n_req} hits of the varlen workload (m = "
                                 f"{list(map(int, m))}), 3-layer group, random-init gates "
                                 f"(mean alpha about 0.5), full-prefix vs suffix replay, all "
                                 f"on the GPU",
                     "rows": rows}}
    out["slow_decay"] = error_vs_k_slow_decay(to_dev, ks)
    return out


def error_vs_k_slow_decay(to_dev, ks, n_seqs=4, m=16384, h_k=4, h_v=8):
    """Replay error against k for one GDN layer whose gates forget slowly:
    alpha ~ U[0.90, 0.999] per token and head (the scalar-decay recipe), so
    the product of the replayed alphas spans about 0.4 (k = 16) to below
    1e-6 (k = 256).  Gated delta rule (unit keys, beta = sigmoid(N(0,1))) and
    scalar decay (beta = 1, keys N(0,1)).  Per k: the relative Frobenius
    error of the suffix state against the full-prefix state, and the bound
    (product of the replayed alphas) x |S_(m-k)| / |S_m| the recurrence
    gives (an equality without the erase term)."""
    import numpy as np
    import torch
    import linear_attention_state_anchor_amd as sr
    from replay_inputs import gdn_case

    res = {}
    for name, kw in (("gated_delta_rule", dict(normalize_k=True, beta="sigmoid", erase=True)),
                     ("scalar_decay", dict(normalize_k=False, beta="none", erase=False))):
        c = gdn_case([m] * n_seqs, h_k, h_v, 128, "bf16", seed=77, alpha=("uniform", 0.90, 0.999),
                     **kw)
        k_all, v_all, a_all = to_dev(c.k), to_dev(c.v), to_dev(c.alpha)
        b_all = None if c.beta is None else to_dev(c.beta)
        la = np.log(c.alpha.astype(np.float64)).reshape(n_seqs, m, h_v)

        def state(lo, hi):
            idx = torch.cat([torch.arange(i * m + lo, i * m + hi, device="cuda:0")
                             for i in range(n_seqs)])
            cu = to_dev(np.arange(0, n_seqs * (hi - lo) + 1, hi - lo, dtype=np.int32))
            S, _ = sr.gdn_replay_state(None, k_all[idx], v_all[idx], a_all[idx],
                                       None if b_all is None else b_all[idx], cu, erase=c.erase,
                                       alpha_is_log=False, want_o=False)
            return S.double()

        full = state(0, m)
        nf = float(torch.linalg.vector_norm(full))
        rows = []
        for kk in list(ks) + [int(np.ceil(0.05 * m)), int(np.ceil(0.10 * m))]:
            S = state(m - kk, m)
            err = float(torch.linalg.vector_norm(S - full)) / nf
            head = state(0, m - kk)
            # bound per (sequence, head): prod(alpha over the suffix) |S_(m-k)|
            pa = np.exp(la[:, m - kk:, :].sum(axis=1))               # [n_seqs][h_v]
            hn = torch.linalg.vector_norm(head, dim=(2, 3)).cpu().numpy()
            bound = float(np.sqrt(np.sum((pa * hn) ** 2))) / nf
            rows.append({"k": kk, "rel_fro": err, "bound": bound,
                         "mean_prod_alpha": float(pa.mean())})
        res[name] = {"workload": f"{n_seqs} x {m} tokens, {h_k} key / {h_v} value heads, d=128, "
                                 f"bf16, alpha ~ U[0.90, 0.999]", "rows": rows}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-group", action="store_true")
    ap.add_argument("--error-vs-k", action="store_true",
                    help="print the replay-error-vs-k report (untimed) instead of the benchmark")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after timing, run one 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the replay "
              "path has no cross-GPU part in this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import linear_attention_state_anchor_amd as sr
    from replay_inputs import config_c3

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:  # bf16 bit patterns
            return torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16)
        return torch.from_numpy(x).to("cuda:0")

    if args.error_vs_k:
        print(json.dumps({"error_vs_k": error_vs_k(to_dev)}), flush=True)
        return

    case = config_c3()
    n, L, hk, hv, d = case.n_seqs, 3276, case.h_k, case.h_v, case.d_k
    T = case.total_tokens
    dev = torch.device("cuda:0")
    q, k, v = to_dev(case.q), to_dev(case.k), to_dev(case.v)
    alpha, beta, cu = to_dev(case.alpha), to_dev(case.beta), to_dev(case.cu_seqlens)
    S = torch.empty((n, hv, d, d), dtype=torch.float32, device=dev)
    o = torch.empty((T, hv, d), dtype=torch.bfloat16, device=dev)

    def step():
        sr.gdn_replay_state(q, k, v, alpha, beta, cu, None, alpha_is_log=True,
                            final_state=S, o=o)

    t = time_steps(step, args.steps, args.warmup)
    ms = t["mean_ms"]
    assert bool(torch.isfinite(S).all()), "non-finite state"

    byts, flops = gdn_algorithmic(n, L, hk, hv, d)
    sec = ms / 1e3
    achieved = byts / sec / 1e9
    traffic = read_traffic(byts)
    line = {
        "metric": "replayed tokens/s per GDN layer (+ % of MI355X HBM / bf16-fp16 MFMA "
                  "roofline), 32K prefix, 10% suffix",
        "value": T / sec,
        "unit": "replayed tokens/s per GDN layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "median_ms": t["median_ms"], "p10_ms": t["p10_ms"], "p90_ms": t["p90_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "gated-delta-rule replay, 16 hits x 3276 anchors (10% of a 32K "
                        "prefix), 16 key / 32 value heads, d=128, chunk 64, bf16 in/out, "
                        "fp32 state",
            "n_seqs": n, "suffix": L, "h_k": hk, "h_v": hv, "d": d, "chunk": 64,
            "kernel": "gdn_chunk_kernel (fp16 MFMA operands, fp32 accumulate)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "mfma": {
            "achieved_tflops": flops / sec / 1e12,
            "peak_tflops": MFMA_F16_PEAK_TFS,
            "frac": flops / sec / 1e12 / MFMA_F16_PEAK_TFS,
            "flop_per_launch": flops,
            "bytes_per_launch": byts,
            "flop_count": "chunked algorithm with the C x C tile products counted dense",
        },
    }
    line.update(bench_replay_variants(min(50, args.steps), 10, to_dev, q, k, v, alpha, beta,
                                      cu, S))
    if not args.no_group:
        line.update(bench_group(min(20, max(3, args.steps // 5)), 3, to_dev))
        line.update(bench_continuation_and_handoff(min(50, args.steps), 5, to_dev))
    if not args.no_cpu_baseline:
        # the benchmarked launch's S and o, against the oracle
        step()
        torch.cuda.synchronize()
        entry, seqs, S_ref, o_ref = cpu_baseline(case, args.cpu_budget)
        line["cpu_baseline"] = entry
        line["parity"] = parity_vs_oracle(S, o, case, seqs, S_ref, o_ref)
    # cold: the headline launch with the caches flushed before each call
    tc = time_cold(step)
    line["cold"] = {"note": "headline launch, median of 20 calls each after a 512 MiB read "
                            "sweep that refills the infinity cache and L2s with clean lines",
                    "median_ms": tc, "hbm_frac": byts / (tc / 1e3) / 1e9 / HBM_PEAK_GBS}
    if not args.no_group:
        # the same headline launch once more at the end of the run, after
        # seconds of other GPU work, as a check that `value` (timed first,
        # after its warm-up launches) is not an artefact of the GPU's state
        ts = time_steps(step, args.steps, 10)
        line["steady_state"] = {
            "note": "headline launch re-timed at the end of the run, after the other lines' "
                    "GPU work",
            "ms_per_step": ts["mean_ms"], "median_ms": ts["median_ms"],
            "replayed_tokens_per_s": T / (ts["mean_ms"] / 1e3),
            "hbm_frac": byts / (ts["mean_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS}
    if args.copy_calib:
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

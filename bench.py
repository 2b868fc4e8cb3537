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


def cpu_baseline(case, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on whole sequences of the same
    workload, as many as fit about budget_s of host time."""
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

    def run(c):
        t0 = time.perf_counter()
        oracle.gdn(c.q, c.k, c.v, c.alpha, c.beta, c.cu_seqlens, c.h_k, c.h_v,
                   alpha_is_log=c.alpha_is_log, erase=c.erase)
        return time.perf_counter() - t0

    threads = oracle.max_threads()
    first = sub([0])
    t1 = run(first)
    n = int(max(1, min(case.n_seqs, budget_s // max(t1, 1e-3))))
    seqs = list(range(n))
    c = sub(seqs)
    t = run(c)
    toks = c.total_tokens
    return {"value": toks / t, "unit": "replayed tokens/s per GDN layer", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {case.n_seqs} sequences ({toks} tokens, all {case.h_v} value "
                      f"heads), fp64 token loop, {t:.2f} s"}


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


def timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_launches(fn, steps, warmup):
    """Average milliseconds per call of fn over `steps` calls, HIP events on
    the current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def replay_entry(ms, T, byts, flops):
    sec = ms / 1e3
    return {"ms_per_step": ms, "replayed_tokens_per_s": T / sec,
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
    ms = time_launches(lambda: sr.gdn_replay_state(None, k, v, alpha, beta, cu, None,
                                                   alpha_is_log=True, want_o=False,
                                                   final_state=S), steps, warmup)
    byts, flops = gdn_algorithmic(n, L, hk, hv, d, want_o=False)
    out = {"state_only": dict(workload="headline replay without q and o (state only)",
                              **replay_entry(ms, T, byts, flops))}
    c = config_c2()
    q2, k2, v2, a2, cu2 = (to_dev(x) for x in (c.q, c.k, c.v, c.alpha, c.cu_seqlens))
    S2 = torch.empty((c.n_seqs, c.h_v, c.d_k, c.d_v), dtype=torch.float32, device=k.device)
    o2 = torch.empty((c.total_tokens, c.h_v, c.d_v), dtype=torch.bfloat16, device=k.device)
    ms = time_launches(lambda: sr.gdn_replay_state(q2, k2, v2, a2, None, cu2, None, erase=False,
                                                   alpha_is_log=c.alpha_is_log,
                                                   final_state=S2, o=o2), steps, warmup)
    byts, flops = gdn_algorithmic(c.n_seqs, c.total_tokens // c.n_seqs, c.h_k, c.h_v, c.d_k,
                                  erase=False)
    out["erase_free"] = dict(workload="erase-free (scalar decay) replay, 8 x 2048, 32 heads, "
                                      "d=128, bf16 in/out, beta = 1",
                             **replay_entry(ms, c.total_tokens, byts, flops))
    return out


def bench_group(steps, warmup, to_dev):
    """3-layer replay group (hidden 2560) from 4 x 1638 anchors, and the
    varlen path: 64 hits gathered from a paged pool of full prefixes and
    replayed through the same group shapes."""
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
    ws = torch.empty((1 << 20,), dtype=torch.uint8, device="cuda:0")
    sr.replay_group(anchors, packed, cu, g.layer_kind, 16, 32, 128, states=states)
    import ctypes
    from linear_attention_state_anchor_amd import _lib
    kinds = (ctypes.c_int32 * 4)(*g.layer_kind)
    desc = _lib.GroupDesc(4, ctypes.cast(kinds, ctypes.POINTER(ctypes.c_int32)), 2560, 16, 32,
                          128, 4, 1e-6, 1e-6, g.n_seqs, T, T)
    wsb = int(_lib.load().sr_replay_group_workspace_bytes(ctypes.byref(desc)))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda:0")
    ms = timed(lambda: sr.replay_group(anchors, packed, cu, g.layer_kind, 16, 32, 128,
                                       states=states, workspace=ws), steps, warmup)
    fl = group_flops(T, 2560, 16, 32, 128, 3)
    out["group"] = {
        "workload": "3 GDN layers + skipped FA, hidden 2560, 4 requests x 1638 anchors "
                    "(5% of 32K), bf16 anchors and weights",
        "ms_per_step": ms, "replayed_tokens_per_s_per_layer": 3 * T / (ms / 1e3),
        "tflops": fl / (ms / 1e3) / 1e12, "mfma_frac": fl / (ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFS,
    }
    del ws
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
    desc5 = _lib.GroupDesc(4, ctypes.cast(kinds, ctypes.POINTER(ctypes.c_int32)), 2560, 16, 32,
                           128, 4, 1e-6, 1e-6, 64, T5, int(pc.suffix_len.max()))
    ws5 = torch.empty((int(_lib.load().sr_replay_group_workspace_bytes(ctypes.byref(desc5))),),
                      dtype=torch.uint8, device="cuda:0")
    states5 = torch.empty((3, 64, 32, 128, 128), dtype=torch.float32, device="cuda:0")
    gather = lambda: sr.gather_suffix(pool, pt, ml, sl, T5, packed=packed_anchors, cu_seqlens=cu5)
    ms_g = timed(gather, steps, warmup)
    def path():
        gather()
        sr.replay_group(packed_anchors, packed5, cu5, [0, 0, 0, 1], 16, 32, 128,
                        states=states5, workspace=ws5)
    ms_p = timed(path, max(2, steps // 5), 1)
    fl5 = group_flops(T5, 2560, 16, 32, 128, 3)
    gb = 2 * T5 * 2560 * 2 / 1e9
    out["varlen"] = {
        "workload": f"64 hits, m ~ U{{8192..32768}}, k = ceil(r m), r ~ U[0.05,0.10] "
                    f"(T = {T5}), gather from 64-token pages + 3-layer group, hidden 2560",
        "ms_per_step": ms_p, "replayed_tokens_per_s_per_layer": 3 * T5 / (ms_p / 1e3),
        "tflops": fl5 / (ms_p / 1e3) / 1e12,
        "gather_ms": ms_g, "gather_gbs": gb / (ms_g / 1e3),
        "gather_hbm_frac": gb / (ms_g / 1e3) / HBM_PEAK_GBS,
    }
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
    return {"workload": f"{n_req} hits of the varlen workload (m = {list(map(int, m))}), "
                        "3-layer group, full-prefix vs suffix replay, all on the GPU",
            "rows": rows}


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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
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
        },
    }
    line.update(bench_replay_variants(min(50, args.steps), 10, to_dev, q, k, v, alpha, beta,
                                      cu, S))
    if not args.no_group:
        line.update(bench_group(min(20, max(3, args.steps // 5)), 3, to_dev))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    if args.copy_calib:
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

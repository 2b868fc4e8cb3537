"""Build the HIP library (gfx950) in-tree.

Each source under csrc/ is compiled to an object in _build/ and linked into
linear_attention_state_anchor_amd/libsr_replay.so with hipcc.  Packed fp32
VALU instructions are disabled for every device compile.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsr_replay.so")
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def headers():
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    hs += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return hs


def _compile(src, force):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    newest_dep = max([os.path.getmtime(src)] + [os.path.getmtime(h) for h in headers()])
    if not force and os.path.exists(obj) and os.path.getmtime(obj) >= newest_dep:
        return obj
    # -save-temps keeps the gfx950 assembly the object is assembled from, so
    # the generated code can be checked (below) exactly as it will run
    cmd = ["hipcc", *CXXFLAGS, "-save-temps=obj", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    stem = os.path.splitext(os.path.basename(src))[0]
    temps = [os.path.join(BUILD, f) for f in os.listdir(BUILD)
             if f.startswith((stem + "-hip-", stem + "-host-", stem + ".hip-hip-"))]
    try:
        asm = os.path.join(BUILD, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")
        bad = check_mfma_chains(open(asm).read())
    finally:
        for t in temps:
            os.remove(t)
    if bad:
        os.remove(obj)
        raise RuntimeError(f"{src}: MFMA accumulation chains that mix shapes without enough "
                           f"wait states (stale accumulators on gfx950):\n" + "\n".join(bad))
    return obj


_MFMA = re.compile(r"(v_mfma_\w+)\s+([va]\[\d+:\d+\]|[va]\d+),\s*([va]\[\d+:\d+\]|[va]\d+),\s*"
                   r"([va]\[\d+:\d+\]|[va]\d+),\s*([va]\[\d+:\d+\]|[va]\d+|[-\w.]+)")
_REGS = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)\b")
_NOP = re.compile(r"s_nop\s+(\d+)")
MFMA_CHAIN_WAIT_STATES = 8


def _regs(tok: str) -> set:
    out = set()
    for m in _REGS.finditer(tok):
        if m.group(1):
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def check_mfma_chains(asm: str, min_wait_states: int = MFMA_CHAIN_WAIT_STATES) -> list:
    """Lines of `asm` where an MFMA accumulates (SrcC) onto the result of an
    earlier MFMA of a different shape with fewer than `min_wait_states` wait
    states between them.

    On gfx950 such a pair (e.g. 16x16x32 f16 then 16x16x16 f16 on the same
    accumulator) reads two stale accumulator registers unless about five
    wait states separate the two; the compiler inserts one.  Chains of one
    shape are safe.  The kernels avoid mixed chains; this scan makes the build
    fail if one appears.  Wait states: one per instruction, N + 1 per s_nop N;
    a VALU/memory write to the accumulator in between ends the chain."""
    bad, func = [], "?"
    last = []  # (opcode, dst regs, wait states since), most recent last
    for line in asm.splitlines():
        if line and not line[0].isspace() and line.endswith(":") and not line.startswith("."):
            func, last = line[:-1], []
            continue
        ins = line.strip()
        if not ins or ins.startswith((";", ".")) or ins.endswith(":"):
            continue
        m = _MFMA.match(ins)
        n = _NOP.match(ins)
        step = int(n.group(1)) + 1 if n else 1
        if m:
            op, dst, src_c = m.group(1), _regs(m.group(2)), _regs(m.group(5))
            for pop, pdst, ws in last:
                if pop != op and pdst & src_c and ws < min_wait_states:
                    bad.append(f"{func}: {ins}  (accumulates onto {pop} {ws} wait states earlier)")
            last = [(o, d - dst, w) for o, d, w in last if d - dst]
            last = [(o, d, w + 1) for o, d, w in last] + [(op, dst, 0)]
        else:
            written = _regs(ins.split(",")[0].split(None, 1)[1]) if ("," in ins and ins.startswith(("v_", "ds_read", "global_load", "buffer_load", "scratch_load", "flat_load"))) else set()
            last = [(o, d - written, w + step) for o, d, w in last if d - written]
    return bad


def build(force: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libsr_replay.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), srcs))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))

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
        bad = check_transpose_reads(open(asm).read())
    finally:
        for t in temps:
            os.remove(t)
    if bad:
        os.remove(obj)
        raise RuntimeError(f"{src}: LDS transpose reads whose destination overlaps the "
                           f"address register (kept out of the kernels):\n" + "\n".join(bad))
    return obj


_TR = re.compile(r"ds_read_b64_tr_b(?:16|8|4)\s+v\[(\d+):(\d+)\],\s*v(\d+)")


def check_transpose_reads(asm: str) -> list:
    """Lines of `asm` where a ds_read_b64_tr_* writes its own address VGPR.

    A build with that form gave wrong results in one kernel variant (the
    cause is not established: an isolated test of the form did not show it).
    The kernels keep their transpose-read bases live across the reads so the
    form does not arise, and this check makes the build fail if it does."""
    bad, func = [], "?"
    for line in asm.splitlines():
        if line and not line[0].isspace() and line.endswith(":") and not line.startswith("."):
            func = line[:-1]
        m = _TR.search(line)
        if m and int(m.group(1)) <= int(m.group(3)) <= int(m.group(2)):
            bad.append(f"{func}: {line.strip()}")
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

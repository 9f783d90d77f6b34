"""Build libvegas_attn.so for gfx950 with hipcc (in-tree, next to this file).

Every .hip file under csrc/ is one translation unit (the host side of the
C-ABI, and one per attention kernel family); they compile in parallel into
_build/ and link into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "vegas_attn")
LIB = os.path.join(HERE, "libvegas_attn.so")
ARCH = os.environ.get("VG_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def units():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def sources():
    return [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [
        os.path.join(ROOT, "include", "vegas_attn.h")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(verbose: bool = False, jobs: int = 0) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmds, objs = [], []
    for u in units():
        o = os.path.join(OBJ, u[:-4] + ".o")
        objs.append(o)
        cmds.append([hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, u), "-o", o])
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            sys.stderr.write(out)
            raise RuntimeError(f"hipcc failed on {cmd[-3]}")
    tmp = LIB + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp])
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("hipcc failed to link libvegas_attn.so")
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in sources())


if __name__ == "__main__":
    print(build(verbose=True))

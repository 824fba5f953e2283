"""Build the HIP library liblsa.so for gfx950 (hipcc, in-tree)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblsa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip to an object in parallel, then link liblsa.so."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        jobs.append([hipcc, *compile_flags, "-c", "-o", obj, src])
    workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        errs = list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + f".tmp{os.getpid()}"
    errs.append(_run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
                      *[j[-2] for j in jobs]], verbose))
    if verbose:
        for e in errs:
            if e.strip():
                print(e, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

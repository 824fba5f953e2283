"""Host-side sanitizer run: builds the CPU oracle and the host code of the
HIP library with AddressSanitizer and UndefinedBehaviorSanitizer, then runs
the CPU tests that exercise them -- the oracle's pins (every oracle function
on golden, brute-force and property cases) and the C ABI's host validation
(every refused call) -- against those builds.  Device code is compiled as
usual (the sanitizers apply to the host side only).  Needs no GPU.

    python -m learned_kv_chunk_amd.sanitize [--skip-hip]

Builds go to learned_kv_chunk_amd/_build/san/.  Exits non-zero if a build or
a test run fails or a sanitizer reports an error."""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "_build", "san")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]


def _run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, env=env)
    if r.returncode != 0:
        sys.exit(f"failed ({r.returncode}): {' '.join(cmd)}")


def build_oracle() -> str:
    lib = os.path.join(OUT, "liblsa_oracle_san.so")
    _run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", *SAN,
          "-o", lib, os.path.join(ROOT, "oracle", "lsa_oracle.c"), "-lm"])
    return lib


def build_hip() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib = os.path.join(OUT, "liblsa_san.so")
    host = [x for f in SAN for x in ("-Xarch_host", f)]
    flags = ["-O1", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *host]
    objs, jobs = [], []
    for src in sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip"))):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        objs.append(obj)
        jobs.append([hipcc, *flags, "-c", "-o", obj, src])
    with ThreadPoolExecutor(max(1, min(len(jobs), len(os.sched_getaffinity(0))))) as ex:
        res = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs))
    for c, r in zip(jobs, res):
        if r.returncode != 0:
            sys.exit(f"hipcc failed: {' '.join(c)}\n{r.stderr}")
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan",
          "-fsanitize=address", "-fsanitize=undefined", "-o", lib, *objs])
    return lib


def clang_asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        sys.exit("clang's AddressSanitizer runtime not found under /opt/rocm/llvm")
    return hits[-1]


def run_tests(files, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    # the interpreter's own allocations are not under test
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    _run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
          *files], env=env)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--skip-hip", action="store_true", help="oracle only")
    args = ap.parse_args()
    os.makedirs(OUT, exist_ok=True)
    oracle_lib = build_oracle()
    gcc_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                            text=True, check=True).stdout.strip()
    run_tests([os.path.join(ROOT, "tests", "test_oracle_pins.py")],
              {"LSA_ORACLE_LIBRARY": oracle_lib}, gcc_rt)
    if not args.skip_hip:
        hip_lib = build_hip()
        run_tests([os.path.join(ROOT, "tests", "test_abi.py")], {"LSA_LIBRARY": hip_lib},
                  clang_asan_runtime())
    print("sanitizer runs clean", flush=True)


if __name__ == "__main__":
    main()

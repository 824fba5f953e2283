"""The library's device-side precondition checks (csrc/table_check.hpp)
built for the host with g++ under the address and undefined-behaviour
sanitizers and run on tables that break one precondition at a time: each
reports exactly its bits, and no check reads outside the arrays' documented
sizes (every array is its own heap block, so such a read aborts the run)."""
import os
import shutil
import subprocess

import pytest

from tests.table_cases import CASES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "table_check_host.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("tc") / "table_check_host")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "learned_kv_chunk_amd", "csrc"),
                    "-o", exe, SRC], check=True)
    return exe


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_host_table_checks_under_sanitizers(driver, case):
    tc, tk = case.totals()
    lines = [f"{case.B} {case.C} {case.max_chunks} {case.max_k} {tc} {tk} "
             f"{int(case.uniform)} {int(case.ascending)} 1 1",
             " ".join(map(str, case.tok_off)), " ".join(map(str, case.chunk_off)),
             " ".join(map(str, case.sel_off)), " ".join(map(str, case.sel_idx))]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       env=env, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    bits = [int(x) for x in r.stdout.split()]
    assert bits[-1] == case.expect, (case.name, bits)

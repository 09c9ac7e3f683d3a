"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

The planner (csrc/plan.cpp), the host argument and page-table checks (csrc/checks.cpp) and the
CPU oracle (oracle/attention_ref.c) are rebuilt with -fsanitize=address,undefined and driven by
tests/sanitize/fuzz_host.cpp: randomised batches, head dims, page sizes (ragged included),
kv dtypes, GQA groups, workspace caps and planner modes, with malformed batches mixed in,
every accepted plan checked against its contract, and the oracle run on small random batches
with row subsets, key ranges and merges. The sanitizers abort on the first finding.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "deterministic_paged_prefill_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc")
def test_host_code_under_asan_and_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    objs = []
    for src, cc, std in ((os.path.join(CSRC, "plan.cpp"), "g++", "-std=c++17"),
                         (os.path.join(CSRC, "checks.cpp"), "g++", "-std=c++17"),
                         (os.path.join(ROOT, "tests", "sanitize", "fuzz_host.cpp"), "g++", "-std=c++17"),
                         (os.path.join(ROOT, "oracle", "attention_ref.c"), "gcc", "-std=c11")):
        obj = os.path.join(tmp_path, os.path.basename(src) + ".o")
        subprocess.run([cc, std, *san, "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    exe = os.path.join(tmp_path, "fuzz_host")
    subprocess.run(["g++", *san, "-o", exe, *objs, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe, "300"], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failed checks" in res.stdout, res.stdout

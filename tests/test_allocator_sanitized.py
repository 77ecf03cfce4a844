"""The host block allocator under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/alloc_fuzz.cpp drives paged_kv_cache_106_amd/csrc/pa_allocator.cpp
through random operation sequences (allocate, append one token or a batch,
share a prefix, fork, free, prompts with prefix caching on and off, calls
that must fail) and checks the allocator's invariants after every one; this
test builds it with g++ (host code only, no device code involved) and runs
a few seeds.  The fuzzer reports how often the out-of-memory, copy-on-write
and prefix-cache-hit paths ran, and each must have run.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"   # pa.h names HIP's runtime types


def _build(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path / "alloc_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "paged_kv_cache_106_amd", "csrc"),
           "-I" + ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "alloc_fuzz.cpp"),
           os.path.join(ROOT, "paged_kv_cache_106_amd", "csrc", "pa_allocator.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower():
        pytest.skip("the sanitizer runtimes are not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_allocator_fuzz_sanitized(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    totals = {"oom": 0, "cow": 0, "prefix_hits": 0}
    for seed in (1, 2, 3, 4):
        r = subprocess.run([exe, str(seed), "1500"], capture_output=True, text=True, env=env,
                           timeout=300)
        assert r.returncode == 0, f"seed {seed}:\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
        m = re.search(r"ok oom=(\d+) cow=(\d+) prefix_hits=(\d+)", r.stdout)
        assert m, r.stdout
        for k, v in zip(totals, m.groups()):
            totals[k] += int(v)
    assert all(v > 0 for v in totals.values()), totals

"""The library's host-side argument checks and launch planning under
AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_fuzz.cpp drives mrr_validate, mrr_describe_plan,
mrr_workspace_size and mrr_status_string with random and extreme arguments
(sizes at and beyond every limit, INT64_MIN/MAX, null and misaligned fake
pointers, overlapping buffers) and with consistent argument sets that must be
accepted. It links mrr_validate.cpp alone, built for the host with g++; no HIP
code and no device are involved, and no pointer is dereferenced.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    out = str(tmp_path_factory.mktemp("host_fuzz") / "host_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "moe_token_re_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_fuzz.cpp"),
           os.path.join(ROOT, "moe_token_re_amd", "csrc", "mrr_validate.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "asan" in res.stderr.lower():
        pytest.skip(f"sanitizer runtime unavailable: {res.stderr[-300:]}")
    assert res.returncode == 0, res.stderr
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_checks_sanitized(fuzz_binary, seed):
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    # the plan's tuning overrides stay at their defaults
    for k in ("MRR_STREAM", "MRR_FUSED", "MRR_OFFSETS", "MRR_ROWS_PER_WG", "MRR_LOG"):
        env.pop(k, None)
    res = subprocess.run([fuzz_binary, str(seed), "200000"], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout, res.stdout
    assert "runtime error" not in res.stderr, res.stderr

"""The host half of the library (block pool, prefix indexes, planner) under
AddressSanitizer and UndefinedBehaviorSanitizer: tests/host_fuzz.cpp drives
random operation sequences through the public C API and checks the block
accounting after each one; any memory error, undefined behaviour, accounting
mismatch or undocumented status fails the test.  CPU only (g++)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_cache_12_amd", "csrc")


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("host_fuzz") / "host_fuzz")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "pa_pool.cpp"), os.path.join(CSRC, "pa_prefix.cpp"),
           os.path.join(HERE, "host_fuzz.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def test_host_api_under_sanitizers(fuzz_binary):
    env = dict(os.environ)
    # the sanitizer runtime must not object to a preloaded library it does not know
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([fuzz_binary, "1000", "400"], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ok 1000 runs" in r.stdout
    cov = dict(kv.split("=") for kv in r.stdout.split("coverage ")[1].split("\n")[0].split())
    # the failure paths and both caches were reached, so the run is not vacuous
    for key in ("no_blocks", "cow_pairs", "cached_hits", "evicted", "swaps", "beam_steps",
                "plans_with_groups"):
        assert int(cov[key]) > 0, (key, cov)

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle (C)
and the expert-slot cache's LRU (cache_core.cpp, the library's host-side policy),
each built with gcc/g++ into its own small driver under tests/sanitize/ and run
over random shapes, edge cases, refused arguments, miss splits, failed fills and
resizes.  Any sanitizer report makes the driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_and_run(compiler, args, exe):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    r = subprocess.run([compiler] + SAN + args + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-4000:])


def test_oracle_under_sanitizers(tmp_path):
    _build_and_run("gcc", ["-std=c11", "-I", os.path.join(ROOT, "oracle"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_stress.c"),
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"], str(tmp_path / "oracle_stress"))


def test_cache_core_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "routed_expert_ffn_layer_amd", "csrc")
    _build_and_run("g++", ["-std=c++17", "-I", csrc, os.path.join(ROOT, "tests", "sanitize", "cache_core_stress.cpp"),
                           os.path.join(csrc, "cache_core.cpp")], str(tmp_path / "cache_core_stress"))

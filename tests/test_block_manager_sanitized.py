"""The host block manager (csrc/block_manager.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer, driven by the differential tests of
tests/test_block_manager.py (random operations against the oracle manager,
swaps, refusals, the copy-on-write cases). The sanitized library is built
here with g++ and loaded in a child Python process that preloads the ASan
runtime; any report aborts the child. CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_kv_cache_440_amd", "csrc", "block_manager.cpp")

CHILD = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import paged_kv_cache_440_amd.block_manager as bm
san = ctypes.CDLL({lib!r})
bm.library = lambda: san            # the manager's symbols come from the sanitized build
import pytest
sys.exit(pytest.main([{tests!r}, "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu"]))
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_manager_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    lib = str(tmp_path / "libpkv_bm_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D_GLIBCXX_SANITIZE_VECTOR",
                    "-I", os.path.join(ROOT, "include"), SRC, "-o", lib], check=True)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (asan, env.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, lib=lib,
                        tests=os.path.join(ROOT, "tests", "test_block_manager.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]

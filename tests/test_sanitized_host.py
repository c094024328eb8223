"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``attn_decode.cpp`` (argument checks, plans, workspace layout) is compiled for
the host with g++ and ``-fsanitize=address,undefined``, linked against stand-ins
for the kernel launchers (``tests/sanitize/launch_stubs.cpp``), and
``tests/test_abi.py``'s checks of argument handling, plans and helpers (all but
the export check: the allocation-free entry point lives in a HIP source) are run
against that library in a child process with the sanitizer runtime preloaded.
Any out-of-bounds access, overflow or other undefined behaviour aborts the
child; the test also requires that no check reached a launch.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_kv_cache_amd", "csrc")
GXX = shutil.which("g++")
ROCM_INC = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(GXX is None or not os.path.isdir(ROCM_INC),
                                reason="g++ or the ROCm headers are not available")


def _runtime(name: str) -> str:
    return subprocess.run([GXX, f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libattn_decode_san.so"
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "attn_decode.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan = _runtime("libasan.so")
    if not os.path.exists(asan):
        pytest.skip("libasan runtime not found")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "ATTN_ABI_TEST_LIB": str(lib),
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-s", "-p", "no:cacheprovider", "-k", "not python_helper and not exports_every"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert "sanitized library: 0 launches reached" in out, out[-2000:]

"""The C ABI's argument checks (api.cpp and host_plan.cpp: sizes, alignment, overlap of byte
ranges, return codes) built for the host alone with AddressSanitizer, and the host tests of
test_capi_host.py run against that build in a child process.

The kernel launchers are replaced by stubs that abort (tests/capi_host_stubs.cpp): every
call those tests make must be rejected before any HIP call.  No GPU is used.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "online_softmax_09_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


def _asan_runtime(cxx):
    out = subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_argument_checks_under_asan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(HIP_INCLUDE):
        pytest.skip("needs g++ and the HIP headers")
    runtime = _asan_runtime(cxx)
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    lib = tmp_path / "libmi355attn_asan.so"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_plan.cpp"),
           os.path.join(ROOT, "tests", "capi_host_stubs.cpp"), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, MI355ATTN_LIB_PATH=str(lib), LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_capi_host.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout

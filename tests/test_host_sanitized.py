"""The library's host-only code (split planner, workspace and counter sizing,
descriptor check, status strings: csrc/attn_host.cpp) built by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer, and driven by
tests/host_fuzz.py in a child process with the ASan runtime preloaded.
Any out-of-bounds access, overflow or other undefined behaviour aborts the
child; every plan is also checked against the invariants the kernels rely
on.  (Host code only: the kernels are not built or run here.)
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_kv_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I/opt/rocm/include"]


def _toolchain():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the ASan runtime is not installed")
    return gxx, asan


def _build(gxx, src, out):
    r = subprocess.run([gxx, *FLAGS, src, "-o", out], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]


def _run(args, asan):
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


@pytest.fixture(scope="module")
def sanitized_host_lib(tmp_path_factory):
    gxx, asan = _toolchain()
    out = str(tmp_path_factory.mktemp("san") / "libattn_host_san.so")
    _build(gxx, os.path.join(CSRC, "attn_host.cpp"), out)
    return out, asan


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    """The set-up itself: a one-element heap overflow in a throwaway library
    built and loaded the same way must abort the child."""
    gxx, asan = _toolchain()
    src = tmp_path / "overflow.cpp"
    src.write_text('#include <vector>\nextern "C" int poke(int n) {\n'
                   '  std::vector<int> v(n);\n  int* p = v.data();\n  p[n] = 1;\n  return p[0];\n}\n')
    lib = str(tmp_path / "liboverflow.so")
    _build(gxx, str(src), lib)
    r = _run(["-c", f"import ctypes; ctypes.CDLL({lib!r}).poke(8)"], asan)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


@pytest.mark.parametrize("seed", [11, 12])
def test_planner_fuzz_under_sanitizers(sanitized_host_lib, seed):
    lib, asan = sanitized_host_lib
    r = _run(["-m", "tests.host_fuzz", lib, "400", str(seed)], asan)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "plans checked" in r.stdout

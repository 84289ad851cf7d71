"""The host side of the library under AddressSanitizer, on the CPU.

Every source of the library is compiled as for the library itself, with
AddressSanitizer on the host pass only (the device code is built as usual and
never runs here), and linked into a library of its own; the CPU tests of the C
ABI
(tests/test_abi_cpu.py: argument validation and the refusals before any launch,
workspace sizing over many shapes, the state layout, the hooks) then run in a
child process against that library, with the sanitizer's runtime preloaded.  Any
out-of-bounds access, use after free or double free in that host code makes the
child fail.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "recurrent_state_phi_amd"))
import build as libbuild  # noqa: E402  (the library's own source list and flags)

HIPCC = libbuild.HIPCC


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_cpu_tests_pass_under_address_sanitizer():
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("no hipcc or AddressSanitizer runtime")
    flags = [f for f in libbuild.FLAGS if f != "-O3"]
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, "-x", "hip", *flags, *libbuild.EXTRA.get(src, []), "-O1", "-Xarch_host", "-g",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-c",
                   os.path.join(libbuild.CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            return obj

        with cf.ThreadPoolExecutor(max_workers=8) as ex:
            objs = list(ex.map(compile_one, libbuild.SOURCES))
        lib = os.path.join(tmp, "libtaylor_attn_asan.so")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                            *objs, "-o", lib],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        env = dict(os.environ, TAYLOR_ATTN_LIB=lib, LD_PRELOAD=rt,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                            os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        out = r.stdout + r.stderr
        assert "AddressSanitizer" not in out, out[-4000:]
        assert r.returncode == 0, out[-4000:]
        assert " passed" in out
        # control: the same set-up reports a planted heap overflow in a library
        # built the same way
        src = os.path.join(tmp, "overflow.cpp")
        with open(src, "w") as f:
            f.write('extern "C" int overflow(int i) { int* p = new int[4]; p[i] = 1; int r = p[0]; delete[] p; return r; }\n')
        bad = os.path.join(tmp, "liboverflow.so")
        r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-fPIC", "-shared", "-O1", "-Xarch_host",
                            "-fsanitize=address", src, "-o", bad], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({bad!r}).overflow(4)"],
                           env=env, capture_output=True, text=True, timeout=120)
        assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

"""Host AddressSanitizer / UndefinedBehaviorSanitizer run of the C-ABI layer (CPU only).

api.cpp (argument validation, workspace carving, launch sequencing) is compiled with the host
sanitizers (hipcc, each -fsanitize= given to the host side only) and linked with the regular
kernel objects into a second library; the host API tests then run against it in a child
process with the compiler's ASan runtime preloaded.  No GPU code is sanitized."""
import glob
import os
import subprocess
import sys

import pytest

from block_sparse_video_reblock_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build():
    os.makedirs(OUT, exist_ok=True)
    objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o")
            for s in sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = os.path.join(OUT, "api.cpp.o")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([B.HIPCC, *flags, *SAN, "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = os.path.join(OUT, "libbsattn.so")
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib,
                        api_o, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def test_host_api_under_address_sanitizer():
    rt = _asan_runtime()
    if rt is None or not os.path.exists(B.HIPCC):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    lib = _build()
    env = dict(os.environ, BSATTN_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child proves the sanitizer runtime is live, then runs the host API tests
    probe = "import ctypes; ctypes.CDLL(None).__asan_init; print('asan live')"
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and "asan live" in r.stdout, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_api.py")], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr

"""The host side of the C ABI under AddressSanitizer and UndefinedBehavior-
Sanitizer: api.cpp (argument validation, status strings, device checks) is
recompiled with host-only sanitizers, linked with the library's other
objects into a separate libqgemm, and tests/test_boundary.py runs against
that build in a subprocess with the ASan runtime preloaded.  Any
out-of-bounds access, signed overflow, invalid enum load or other undefined
behaviour on a validation path fails the run.  No GPU is needed; the device
code is the normal build's."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def test_boundary_under_asan_and_ubsan(tmp_path):
    from conv_qgemm_amd import build

    rt = _asan_runtime()
    if rt is None or not os.path.exists(build.HIPCC):
        pytest.skip("no clang sanitizer runtime or hipcc here")
    objdir = build.OBJ
    others = [os.path.join(objdir, s + ".o") for s in build.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in others):
        build.build()
    # host-only sanitizers: each -fsanitize option follows -Xarch_host, so the
    # gfx950 device code of this translation unit is built as usual
    san = ["-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in build.CFLAGS if f != "-O3"] + ["-O1", "-g"]
    api_o = tmp_path / "api_san.o"
    subprocess.run([build.HIPCC, *flags, *san, "-c",
                    os.path.join(build.CSRC, "api.cpp"), "-o", str(api_o)],
                   check=True, capture_output=True)
    lib = tmp_path / "libqgemm_san.so"
    subprocess.run([build.HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address,undefined", "-shared-libsan",
                    str(api_o), *others, "-o", str(lib), "-Wl,-rpath,/opt/rocm/lib"],
                   check=True, capture_output=True)
    env = dict(os.environ, QG_LIB=str(lib), LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "passed" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]

"""The C ABI from plain C (tests/c/abi_check.c): a C11 program, compiled
with gcc against include/qgemm.h and the HIP runtime API only, allocates
device buffers with hipMalloc, calls the library's entry points with raw
pointers and compares every output with the oracle's C functions.  The CPU
test checks that it compiles and links (the header is valid C, every symbol
it names resolves); the GPU test runs it: the tile and ring GEMM kernels,
the skinny W4A8 kernel (one and two token blocks), the int4 tile path, both
conv kernels, and a rejected call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_check.c")
LIBDIR = os.path.join(ROOT, "conv_qgemm_amd")
ORCDIR = os.path.join(ROOT, "oracle")


def _compile(out):
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no gcc or ROCm headers")
    for lib in (os.path.join(LIBDIR, "libqgemm.so"), os.path.join(ORCDIR, "liboracle.so")):
        if not os.path.exists(lib):
            pytest.skip(f"{lib} is not built")
    cmd = ["gcc", "-O1", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), SRC,
           "-L" + LIBDIR, "-lqgemm", "-L" + ORCDIR, "-loracle", "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + ORCDIR, "-Wl,-rpath,/opt/rocm/lib",
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


def test_c_program_builds(tmp_path):
    _compile(tmp_path / "abi_check")


@pytest.mark.gpu
def test_c_program_matches_oracle(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = tmp_path / "abi_check"
    _compile(exe)
    print("running", exe, flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=180)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert "every output matches the oracle" in r.stdout

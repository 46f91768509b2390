"""Guards on the generated gfx950 code of the large-GEMM kernel (compiled
here to AMD assembly; no GPU needed).  Two silent regressions these catch:
the accumulator array demoted to scratch memory (private segment), and the
compiler waiting for every direct-to-LDS load (vmcnt(0)) inside the main
loop, which serialises the 4-stage ring."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "conv_qgemm_amd", "csrc", "k_gemm_dma.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "k_gemm_dma.s"
    from conv_qgemm_amd import build
    cmd = [build.HIPCC, *build.CFLAGS, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _kernels(asm):
    """name -> body text for each k_gemm_dma instantiation."""
    out = {}
    for m in re.finditer(r"^(_Z\S*k_gemm_dma\S*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end]
    return out


# s8s8 requantize, s4s4 raw int32, s8s8 asymmetric requantize, s4s4 binary16,
# w4a8 requantize (int4 weights low or high nibble first)
N_INSTANTIATIONS = 6


def _nonempty(ks):
    assert len(ks) == N_INSTANTIATIONS, list(ks)
    return ks


def _main_loop(body):
    lines = [ln.strip() for ln in body.splitlines() if ln.strip() and not ln.strip().startswith(";")]
    mf = [i for i, ln in enumerate(lines) if "v_mfma" in ln]
    start = max(i for i in range(mf[0]) if lines[i].startswith(".LBB"))
    return lines[start:mf[-1] + 1]


def test_no_scratch(asm):
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes
    ks = _nonempty(_kernels(asm))
    for name, body in ks.items():
        loop = _main_loop(body)
        assert not any("scratch_" in ln for ln in loop), name


def test_main_loop_shape(asm):
    for name, body in _nonempty(_kernels(asm)).items():
        loop = _main_loop(body)
        waits = [ln for ln in loop if ln.startswith("s_waitcnt")]
        assert not any(re.search(r"vmcnt\(0\)", w) for w in waits), (name, waits)
        assert sum("s_barrier" in ln for ln in loop) == 1, name
        # operand kind: 8 int8 x int8, 4 int4 x int4, 3 / 5 int8 x int4
        kind = int(re.search(r"k_gemm_dmaILi(\d)E", name).group(1))
        loads = 12 if kind in (3, 5) else 8
        assert sum("global_load_lds_dwordx4" in ln for ln in loop) == loads, name
        assert sum("v_mfma_i32_32x32x32_i8" in ln for ln in loop) == (32 if kind == 8 else 64), name


def test_accumulators_not_spilled(asm):
    for name, body in _nonempty(_kernels(asm)).items():
        # every accumulator stays in registers: no acc-sized private segment
        m = re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", body)
        if m:
            assert int(m.group(1)) < 256, name


@pytest.mark.parametrize("src", ["k_gemm_dma.hip", "k_tile_gemm.hip"])
def test_binary16_output_rounds_twice(tmp_path, src):
    """The binary16 epilogue rounds the scaled product to binary32 and then
    to binary16.  A mixed-precision FMA (v_fma_mix*/v_mad_mix*) would round
    once and differ from the definition in rare cases."""
    from conv_qgemm_amd import build
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC, *build.CFLAGS, "--cuda-device-only", "-S",
           os.path.join(ROOT, "conv_qgemm_amd", "csrc", src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    assert "v_cvt_f16_f32" in text
    assert not re.search(r"v_(fma|mad)_mix", text)

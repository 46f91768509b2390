"""Guards on the generated gfx950 code of the large-GEMM kernel (compiled
here to AMD assembly; no GPU needed).  Two silent regressions these catch:
the accumulator array demoted to scratch memory (private segment), and the
compiler waiting for every direct-to-LDS load (vmcnt(0)) inside the main
loop, which serialises the 4-stage ring.  The loop is also checked to issue
its loads as buffer loads with no per-lane address arithmetic."""
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
    cmd = [build.HIPCC, *build.flags_for(SRC), "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _kernels(asm):
    """name -> body text for each k_gemm_dma instantiation."""
    out = {}
    for m in re.finditer(r"^(_Z\S*k_gemm_dma\S*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end]
    return out


# s8s8 requantize, s4s4 raw int32, s8s8 asymmetric requantize, s4s4 binary16
# (each stage by stage and in pairs of stages), w4a8 requantize (int4
# weights low or high nibble first; stage by stage only)
N_INSTANTIATIONS = 10


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
        # operand kind: 8 int8 x int8, 4 int4 x int4, 3 / 5 int8 x int4;
        # pairs: one loop iteration multiplies two 64-byte K stages
        kind, epi, pairs, nw = re.search(r"k_gemm_dmaILi(\d)ELi(\d)ELb(\d)ELi(\d)E", name).groups()
        kind, pairs, nw = int(kind), pairs == "1", int(nw)
        rows = 256 // nw  # A and B rows each wave loads per stage
        row_a = 128 if kind in (3, 5) else 64
        loads = 2 * rows * 128 // 1024 if pairs else rows * (row_a + 64) // 1024
        vm = [w for w in waits if "vmcnt" in w]
        barriers = sum("s_barrier" in ln for ln in loop)
        if pairs and nw == 4:
            # early form: a second barrier frees the pair's slot mid-pair;
            # the pair's last barrier leaves the first half of the pair
            # after next in flight (its second half goes out in the next
            # pair's first stage)
            assert barriers == 2, name
            assert len(vm) == 1 and re.search(rf"vmcnt\({loads // 2}\)", vm[0]), (name, waits)
        elif pairs:
            # the pair's loads are waited for once, at its barrier
            assert barriers == 1, name
            assert len(vm) == 1 and re.search(r"vmcnt\(0\)", vm[0]), (name, waits)
        else:
            # the ring keeps the later stages' loads in flight at the barrier
            assert barriers == 1, name
            assert not any(re.search(r"vmcnt\(0\)", w) for w in waits), (name, waits)
        assert sum(re.search(r"buffer_load_dwordx4 .* offen lds", ln) is not None
                   for ln in loop) == loads, name
        # no per-lane address arithmetic for the loads: the loop's only
        # 64-bit VALU ops would be address adds
        assert not any(ln.startswith(("v_lshl_add_u64", "v_add_co_u32")) for ln in loop), name
        # a stage is 8x8 tiles of 16x16x64 per wave: 64 MFMAs for int8, two
        # K steps (128) when a 64-byte fragment row holds packed int4
        # a wave owns 128 x (512 / nw) outputs: 8 x (32 / nw) tiles, one
        # MFMA each per K step, one step per stage for int8, two for int4
        per_stage = 8 * (32 // nw) * (1 if kind == 8 else 2)
        assert sum("v_mfma_i32_16x16x64_i8" in ln for ln in loop) == per_stage * (2 if pairs else 1), name
        assert not any("v_mfma_i32_32x32" in ln for ln in loop), name
        # every MFMA accumulates in place: no accumulator copies in the loop
        assert not any(ln.startswith("v_accvgpr") for ln in loop), name


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
    cmd = [build.HIPCC, *build.flags_for(src), "--cuda-device-only", "-S",
           os.path.join(ROOT, "conv_qgemm_amd", "csrc", src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    assert "v_cvt_f16_f32" in text
    assert not re.search(r"v_(fma|mad)_mix", text)


def test_skinny_staged_readback_waits_for_the_copies_only(tmp_path):
    """The skinny W4A8 kernel stages its first token block's activations
    through LDS and reads them back before its first barrier.  That read-back
    must wait only for the staging copies (vmcnt(8): the first unit's eight
    weight loads per wave stay in flight), not for every load (vmcnt(0)),
    which would put the weights' HBM latency in front of it.  Checked on the
    one-chunk kernels, one and two token blocks, both nibble orders."""
    from conv_qgemm_amd import build
    out = tmp_path / "k_skinny_w4a8.s"
    cmd = [build.HIPCC, *build.flags_for("k_skinny_w4a8.hip"), "--cuda-device-only", "-S",
           os.path.join(ROOT, "conv_qgemm_amd", "csrc", "k_skinny_w4a8.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    names = re.findall(r"^(_Z\S*k_skinny_w4a8ILb1E\S*):", text, re.M)
    assert len(names) == 4, names  # one chunk: (one or two blocks) x 2 nibble orders
    for name in names:
        start = text.index("\n" + name + ":")
        body = text[start:text.index(".Lfunc_end", start)]
        ops = [ln.strip() for ln in body.splitlines()
               if ln.startswith("\t") and not ln.strip().startswith((".", ";"))]
        first_bar = next(i for i, ln in enumerate(ops) if ln.startswith("s_barrier"))
        pro = ops[:first_bar]
        first_read = next(i for i, ln in enumerate(pro) if ln.startswith("ds_read_b128"))
        dma = [i for i, ln in enumerate(pro[:first_read]) if ln.startswith("global_load_lds_dwordx4")]
        # the staged branch: 16 copies, then the unit's 8 weight loads
        assert len(dma) >= 24, (name, len(dma))
        waits = [ln for ln in pro[dma[-1]:first_read] if ln.startswith("s_waitcnt")]
        assert waits and all("vmcnt(0)" not in w for w in waits), (name, waits)
        assert any("vmcnt(8)" in w for w in waits), (name, waits)

"""The C-ABI library on the host: it loads, exports every function declared in
include/qgemm.h, and rejects every invalid argument before any HIP call (so
these run with no GPU).  Pointers here are fake, aligned addresses: a call
that passes validation is only made where no GPU is present, where it must
stop at the device check."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")


@pytest.fixture(scope="module")
def qg():
    from conv_qgemm_amd import qgemm
    return qgemm


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+)\s*\(", text)))


def test_exports_every_declared_symbol(qg):
    names = _declared_functions()
    assert set(names) >= {"qgemm_s8s8_requant", "qgemm_s4s4_i32", "qgemm_w4a8_requant",
                          "qconv2d_nhwc_s8_requant", "qdwconv2d_nhwc_s8_requant",
                          "qquant_per_token", "qgemm_s8s8_requant_zp", "qgemm_w4a8_requant_msb",
                          "qgemm_s4s4_f16",
                          "qconv2d_nhwc_s8_requant_zp", "qdwconv2d_nhwc_s8_requant_zp",
                          "qg_status_string", "qg_version"}
    raw = ctypes.CDLL(qg._LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(qg.EXPORTS) == set(names)


def test_status_strings(qg):
    for code in range(5):
        s = qg.status_string(code)
        assert s.startswith("QG_")
    assert qg.status_string(99) == "unknown qg_status"
    assert qg.version() >= 100


def test_header_constants_match_binding(qg):
    text = open(HEADER).read()
    assert int(re.search(r"QG_S4S4_MAX_K (\d+)", text).group(1)) == qg.QG_S4S4_MAX_K
    assert int(re.search(r"QG_W4A8_MAX_K (\d+)", text).group(1)) == qg.QG_W4A8_MAX_K
    # 256 * 64 * K and 16 * 1024 * K stay below 2^31 at the bound
    assert 256 * 64 * qg.QG_S4S4_MAX_K < 2 ** 31
    assert 16 * 128 * 8 * qg.QG_W4A8_MAX_K < 2 ** 31
    assert qg.QG_S4S4_MAX_K % 32 == 0
    for name in ("QG_DT_F32", "QG_DT_F16", "QG_DT_BF16"):
        assert int(re.search(name + r" (\d+)", text).group(1)) == getattr(qg, name)


P = 0x10000  # fake, 16-byte aligned device addresses
NULL = None


def s8(qg, A=P, lda=64, B=P, ldb=64, bias=P, mult=P, shift=P, C=P, ldc=64, M=32, N=64, K=64):
    return qg.lib.qgemm_s8s8_requant(A, lda, B, ldb, bias, mult, shift, C, ldc, M, N, K, None)


def s4(qg, A=P, lda=64, B=P, ldb=64, C=P, ldc=64, M=32, N=64, K=64):
    return qg.lib.qgemm_s4s4_i32(A, lda, B, ldb, C, ldc, M, N, K, None)


def s4h(qg, A=P, lda=64, B=P, ldb=64, sa=P, sb=P, C=P, ldc=64, M=32, N=64, K=64):
    return qg.lib.qgemm_s4s4_f16(A, lda, B, ldb, sa, sb, C, ldc, M, N, K, None)


def w4(qg, A=P, lda=64, B=P, ldb=64, bias=P, mult=P, shift=P, C=P, ldc=64, M=16, N=64, K=64):
    return qg.lib.qgemm_w4a8_requant(A, lda, B, ldb, bias, mult, shift, C, ldc, M, N, K, None)


def w4m(qg, A=P, lda=64, B=P, ldb=64, bias=P, mult=P, shift=P, C=P, ldc=64, M=16, N=64, K=64):
    return qg.lib.qgemm_w4a8_requant_msb(A, lda, B, ldb, bias, mult, shift, C, ldc, M, N, K,
                                         None)


def cv(qg, X=P, W=P, bias=P, mult=P, shift=P, Y=P, batch=1, H=8, Wd=8, C_in=16, C_out=16,
       KH=3, KW=3, sh=1, sw=1, ph=1, pw=1):
    return qg.lib.qconv2d_nhwc_s8_requant(X, W, bias, mult, shift, Y, batch, H, Wd, C_in, C_out,
                                          KH, KW, sh, sw, ph, pw, None)


def dw(qg, X=P, W=P, bias=P, mult=P, shift=P, Y=P, batch=1, H=8, Wd=8, C=16, KH=3, KW=3,
       sh=1, sw=1, ph=1, pw=1):
    return qg.lib.qdwconv2d_nhwc_s8_requant(X, W, bias, mult, shift, Y, batch, H, Wd, C, KH, KW,
                                            sh, sw, ph, pw, None)


def qt(qg, X=P, dtype=0, ldx=64, Q=P, ldq=64, scale=P, M=8, K=64, clip=1.0, bits=8):
    return qg.lib.qquant_per_token(X, dtype, ldx, Q, ldq, scale, M, K, clip, bits, None)


WS = 0x20000  # fake workspace address


def s8z(qg, A=P, lda=64, B=P, ldb=64, bias=P, mult=P, shift=P, za=3, zb=-4, zo=5, lo=-128,
        hi=127, C=P, ldc=64, M=32, N=64, K=64, ws=WS, wsb=1 << 20):
    return qg.lib.qgemm_s8s8_requant_zp(A, lda, B, ldb, bias, mult, shift, za, zb, zo, lo, hi, C,
                                        ldc, M, N, K, ws, wsb, None)


def s8n(qg, A=P, lda=64, B=P, ldb=64, bias=P, mult=P, shift=P, za=3, zb=-4, zo=5, lo=-128,
        hi=127, C=P, ldc=64, M=32, N=64, K=64):
    return qg.lib.qgemm_s8s8_requant_zp_noalloc(A, lda, B, ldb, bias, mult, shift, za, zb, zo, lo,
                                                hi, C, ldc, M, N, K, None)


def cvz(qg, X=P, W=P, bias=P, mult=P, shift=P, za=3, zb=-4, zo=5, lo=-128, hi=127, Y=P, batch=1,
        H=8, Wd=8, C_in=16, C_out=16, KH=3, KW=3, sh=1, sw=1, ph=1, pw=1, ws=WS, wsb=1 << 20):
    return qg.lib.qconv2d_nhwc_s8_requant_zp(X, W, bias, mult, shift, za, zb, zo, lo, hi, Y,
                                             batch, H, Wd, C_in, C_out, KH, KW, sh, sw, ph, pw,
                                             ws, wsb, None)


def dwz(qg, X=P, W=P, bias=P, mult=P, shift=P, za=3, zb=-4, zo=5, lo=-128, hi=127, Y=P, batch=1,
        H=8, Wd=8, C=16, KH=3, KW=3, sh=1, sw=1, ph=1, pw=1, ws=WS, wsb=1 << 20):
    return qg.lib.qdwconv2d_nhwc_s8_requant_zp(X, W, bias, mult, shift, za, zb, zo, lo, hi, Y,
                                               batch, H, Wd, C, KH, KW, sh, sw, ph, pw, ws, wsb,
                                               None)


def test_nullptr(qg):
    E = qg.QG_ERR_NULLPTR
    for kw in ("A", "B", "C", "mult", "shift"):
        assert s8(qg, **{kw: NULL}) == E, kw
        assert w4(qg, **{kw: NULL}) == E, kw
        assert w4m(qg, **{kw: NULL}) == E, kw
    for kw in ("A", "B", "C"):
        assert s4(qg, **{kw: NULL}) == E, kw
        assert s4h(qg, **{kw: NULL}) == E, kw
    for kw in ("X", "W", "Y", "mult", "shift"):
        assert cv(qg, **{kw: NULL}) == E, kw
        assert dw(qg, **{kw: NULL}) == E, kw
    for kw in ("X", "Q", "scale"):
        assert qt(qg, **{kw: NULL}) == E, kw
    for kw in ("A", "B", "C", "mult", "shift", "ws"):
        assert s8z(qg, **{kw: NULL}) == E, kw
    for kw in ("X", "W", "Y", "mult", "shift", "ws"):
        assert cvz(qg, **{kw: NULL}) == E, kw
        assert dwz(qg, **{kw: NULL}) == E, kw


def test_invalid_gemm_sizes(qg):
    E = qg.QG_ERR_INVALID
    for f in (s8, s4, s4h, w4, w4m):
        assert f(qg, M=0) == E
        assert f(qg, N=0) == E
        assert f(qg, K=0) == E
        assert f(qg, M=-1) == E
        assert f(qg, M=2 ** 31) == E        # rows past the int32 headroom
        assert f(qg, lda=32, K=64) == E     # lda < K
        assert f(qg, ldb=32, K=64) == E     # ldb < K
        assert f(qg, ldc=48, N=64) == E     # ldc < N
    # K must fill whole 16-byte rows: K % 16 for int8, K % 32 with any int4 operand
    assert s8(qg, K=40, lda=64, ldb=64) == E
    assert s4(qg, K=48, lda=64, ldb=64) == E
    assert w4(qg, K=48, lda=64, ldb=64) == E
    assert w4m(qg, K=48, lda=64, ldb=64) == E
    # row strides: multiples of 16 bytes
    assert s8(qg, lda=72) == E
    assert s4(qg, lda=80) == E              # 80 nibbles = 40 bytes
    assert w4(qg, ldb=80) == E
    # int4 K bounds keep the scaled int32 sums exact
    big = qg.QG_S4S4_MAX_K + 32
    assert s4(qg, K=big, lda=big, ldb=big) == E
    assert s4h(qg, K=big, lda=big, ldb=big) == E
    assert s4h(qg, K=48, lda=64, ldb=64) == E
    assert s4h(qg, sa=P + 4) == E           # scales 16-byte aligned
    assert s4h(qg, sb=P + 8) == E
    assert s4h(qg, C=P + 2) == E
    assert w4(qg, K=big, lda=big, ldb=big) == E
    assert w4m(qg, K=big, lda=big, ldb=big) == E


def test_invalid_alignment(qg):
    E = qg.QG_ERR_INVALID
    for kw in ("A", "B", "C"):
        assert s8(qg, **{kw: P + 8}) == E, kw
        assert s4(qg, **{kw: P + 4}) == E, kw
        assert w4(qg, **{kw: P + 1}) == E, kw
    for kw in ("bias", "mult", "shift"):
        assert s8(qg, **{kw: P + 4}) == E, kw
        assert w4(qg, **{kw: P + 4}) == E, kw
    for kw in ("X", "W", "Y", "mult"):
        assert cv(qg, **{kw: P + 4}) == E, kw
        assert dw(qg, **{kw: P + 4}) == E, kw


def test_invalid_conv(qg):
    E = qg.QG_ERR_INVALID
    for kw in ("batch", "H", "Wd", "C_in", "C_out", "KH", "KW", "sh", "sw"):
        assert cv(qg, **{kw: 0}) == E, kw
    assert cv(qg, ph=-1) == E
    assert cv(qg, pw=-1) == E
    assert cv(qg, C_in=24) == E             # C_in % 16
    assert cv(qg, C_out=8) == E             # C_out % 16
    assert cv(qg, H=2, KH=5, ph=1) == E     # H_out < 1
    assert cv(qg, Wd=1, KW=4, pw=1) == E    # W_out < 1
    assert cv(qg, batch=2 ** 20, H=2 ** 10, Wd=2 ** 10) == E  # too many pixels


def test_invalid_dwconv(qg):
    E = qg.QG_ERR_INVALID
    for kw in ("batch", "H", "Wd", "C", "KH", "KW", "sh", "sw"):
        assert dw(qg, **{kw: 0}) == E, kw
    assert dw(qg, ph=-1) == E
    assert dw(qg, pw=-1) == E
    assert dw(qg, C=24) == E                # C % 16
    assert dw(qg, H=2, KH=5, ph=1) == E     # H_out < 1
    assert dw(qg, Wd=1, KW=4, pw=1) == E    # W_out < 1
    assert dw(qg, batch=2 ** 20, H=2 ** 10, Wd=2 ** 10) == E  # too many pixels


def test_invalid_quant(qg):
    E = qg.QG_ERR_INVALID
    assert qt(qg, dtype=3) == E
    assert qt(qg, dtype=-1) == E
    for bits in (0, 2, 16):
        assert qt(qg, bits=bits) == E
    for clip in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert qt(qg, clip=clip) == E, clip
    assert qt(qg, M=0) == E
    assert qt(qg, K=0) == E
    assert qt(qg, K=8, ldx=64) == E             # K < 16
    assert qt(qg, K=40, ldx=64, ldq=64) == E    # K % 16
    assert qt(qg, ldx=48, K=64) == E            # ldx < K
    assert qt(qg, ldq=48, K=64) == E            # ldq < K
    assert qt(qg, ldx=68, K=64, dtype=1) == E   # half rows must be 16-byte multiples
    assert qt(qg, ldx=66, K=64, dtype=0) == E   # float rows must be 16-byte multiples
    assert qt(qg, ldq=72, K=64) == E            # ldq % 16
    assert qt(qg, M=2 ** 31) == E
    for kw in ("X", "Q"):
        assert qt(qg, **{kw: P + 8}) == E, kw
    assert qt(qg, scale=P + 2) == E


def test_invalid_zero_point_forms(qg):
    E = qg.QG_ERR_INVALID
    for f in (s8z, cvz, dwz):
        for kw in ("za", "zb", "zo"):
            assert f(qg, **{kw: 128}) == E, (f.__name__, kw)
            assert f(qg, **{kw: -129}) == E, (f.__name__, kw)
        assert f(qg, ws=WS + 8) == E             # misaligned workspace
        assert f(qg, lo=10, hi=9) == E           # empty clamp range
        assert f(qg, lo=-129) == E
        assert f(qg, hi=128) == E
    # workspace smaller than the size function asks for
    need = qg.lib.qgemm_s8s8_requant_zp_workspace_size(32, 64)
    assert need == 256 + 256
    assert s8z(qg, wsb=need - 1) == E
    need = qg.lib.qconv2d_nhwc_s8_requant_zp_workspace_size(1, 8, 8, 16, 3, 3, 1, 1, 1, 1)
    assert need == 256 + 256                    # 16 channels, 64 pixels
    assert cvz(qg, wsb=need - 4) == E
    need = qg.lib.qdwconv2d_nhwc_s8_requant_zp_workspace_size(16)
    assert need == 256
    assert dwz(qg, wsb=need - 1) == E
    # the symmetric calls' own rules still apply
    assert s8z(qg, K=40) == E
    assert cvz(qg, C_in=24) == E
    assert dwz(qg, C=24) == E
    # size functions reject what the calls reject
    assert qg.lib.qgemm_s8s8_requant_zp_workspace_size(0, 5) == 0
    assert qg.lib.qconv2d_nhwc_s8_requant_zp_workspace_size(1, 2, 8, 16, 5, 3, 1, 1, 1, 1) == 0
    assert qg.lib.qdwconv2d_nhwc_s8_requant_zp_workspace_size(0) == 0


def test_invalid_noalloc_form(qg):
    """The allocation-free asymmetric GEMM checks what qgemm_s8s8_requant_zp
    checks, and rejects shapes whose compensation sums exceed its 1 MiB
    per-GPU array: 4 * (ceil(M/64) + ceil(N/64)) * 64 bytes."""
    for kw in ("A", "B", "C", "mult", "shift"):
        assert s8n(qg, **{kw: NULL}) == qg.QG_ERR_NULLPTR, kw
    E = qg.QG_ERR_INVALID
    for kw in ("za", "zb", "zo"):
        assert s8n(qg, **{kw: 128}) == E, kw
        assert s8n(qg, **{kw: -129}) == E, kw
    assert s8n(qg, lo=10, hi=9) == E
    assert s8n(qg, K=40) == E
    assert s8n(qg, M=0) == E
    assert s8n(qg, A=P + 8) == E
    assert s8n(qg, M=131072, N=131073, ldc=131088) == E
    assert s8n(qg, M=262081, N=64) == E
    import torch
    if torch.cuda.is_available():
        return
    # exactly at the limit the call passes validation and stops at the device
    assert s8n(qg, M=131072, N=131072, ldc=131072) == qg.QG_ERR_NO_DEVICE
    assert s8n(qg, M=262080, N=64) == qg.QG_ERR_NO_DEVICE
    assert s8n(qg, bias=NULL) == qg.QG_ERR_NO_DEVICE


def test_valid_call_without_gpu_reports_no_device(qg):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case is only meaningful without one")
    assert s8(qg) == qg.QG_ERR_NO_DEVICE
    assert s4(qg) == qg.QG_ERR_NO_DEVICE
    assert w4(qg) == qg.QG_ERR_NO_DEVICE
    assert w4m(qg) == qg.QG_ERR_NO_DEVICE
    assert s4h(qg) == qg.QG_ERR_NO_DEVICE
    assert s4h(qg, sa=NULL, sb=NULL, ldc=66) == qg.QG_ERR_NO_DEVICE  # scales optional
    assert cv(qg) == qg.QG_ERR_NO_DEVICE
    assert dw(qg) == qg.QG_ERR_NO_DEVICE
    assert qt(qg) == qg.QG_ERR_NO_DEVICE
    assert s8z(qg) == qg.QG_ERR_NO_DEVICE
    assert cvz(qg) == qg.QG_ERR_NO_DEVICE
    assert dwz(qg) == qg.QG_ERR_NO_DEVICE
    assert s8z(qg, za=-128, zb=127, zo=-128, wsb=512) == qg.QG_ERR_NO_DEVICE
    assert cvz(qg, zo=7, lo=7, hi=7) == qg.QG_ERR_NO_DEVICE
    assert qt(qg, dtype=2, bits=4, ldx=72, ldq=80, scale=P + 4, clip=0.25) == qg.QG_ERR_NO_DEVICE


def test_binding_rejects_bad_tensors(qg):
    import torch
    A = torch.zeros((4, 32), dtype=torch.int16)
    with pytest.raises(TypeError):
        qg.qgemm_s8s8_requant(A, A, None, None, None)
    X = torch.zeros((1, 4, 4, 16), dtype=torch.int8)
    W = torch.zeros((16, 3, 3, 32), dtype=torch.int8)
    with pytest.raises(ValueError):
        qg.qconv2d_nhwc_s8_requant(X, W, None, torch.zeros(16, dtype=torch.int32),
                                   torch.zeros(16, dtype=torch.int32))


def test_binding_rejects_host_tensors(qg):
    """Well-formed tensors in host memory never reach the library: their
    pointers are not device addresses."""
    import torch
    A = torch.zeros((4, 32), dtype=torch.int8)
    v = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        qg.qgemm_s8s8_requant(A, A, v, v, v, C=torch.zeros((4, 4), dtype=torch.int8))
    P = torch.zeros((4, 16), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        qg.qgemm_s4s4_i32(P, P, C=torch.zeros((4, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        qg.qgemm_w4a8_requant(A, P, v, v, v, C=torch.zeros((4, 4), dtype=torch.int8))
    X = torch.zeros((1, 4, 4, 16), dtype=torch.int8)
    W = torch.zeros((16, 3, 3, 16), dtype=torch.int8)
    v16 = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        qg.qconv2d_nhwc_s8_requant(X, W, v16, v16, v16, Y=torch.zeros((1, 4, 4, 16),
                                                                     dtype=torch.int8))
    with pytest.raises(ValueError, match="GPU tensor"):
        qg.qquant_per_token(torch.zeros((4, 64), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        qg.qquant_per_token(torch.zeros((4, 64), dtype=torch.float64))

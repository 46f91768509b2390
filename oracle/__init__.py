"""CPU oracle for the quantized GEMM / conv path -- TEST INFRASTRUCTURE ONLY.

A thin ctypes layer over ``qgemm_oracle.c``: plain loops, int64 sums, the Q31
requantize written out as the MCU conv front-end page
(news.rkmt.cn/news/16638, §2.3) states it.  Only ``tests/``, the smoke check
and the benchmark's CPU-baseline leg may import this package; the GPU library
never does, and this package imports nothing from it.

Every function takes numpy arrays in the same layouts as the GPU entry points
(A ``[M][K]`` row-major, B ``[N][K]``, packed int4 as ``uint8`` with two
nibbles per byte, low nibble = even index; NHWC activations, OHWI weights)
and returns numpy arrays.  ``rows`` / ``pix`` select a subset of output rows /
output pixels, so full-size problems can be checked on samples.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qgemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at another build of the same source (for
# example one with a planted mistake, to show that the pins catch it).
_LIB_OVERRIDE = os.environ.get("QG_ORACLE_LIB")

ORC_OK = 0
ORC_E_RANGE = 1
ORC_E_DOMAIN = 2


def build(extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile the oracle with gcc (no HIP).  Returns the library path."""
    out = out or _LIB_PATH
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra"]
    cmd += list(extra_flags or [])
    cmd += [_SRC, "-o", out]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_OVERRIDE or _LIB_PATH
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    lib.orc_int4_at.argtypes = [P, I64]
    lib.orc_int4_at.restype = ctypes.c_int
    lib.orc_requant.argtypes = [I64, I32, I32, I32, P]
    lib.orc_requant.restype = ctypes.c_int
    lib.orc_requant_many.argtypes = [P, P, P, P, P, I64]
    lib.orc_requant_many.restype = ctypes.c_int
    lib.orc_gemm_acc.argtypes = [ctypes.c_int, P, I64, ctypes.c_int, P, I64, I64, I64, P, I64, P]
    lib.orc_gemm_acc.restype = ctypes.c_int
    for name in ("orc_gemm_s8s8_requant", "orc_gemm_w4a8_requant"):
        f = getattr(lib, name)
        f.argtypes = [P, I64, P, I64, P, P, P, P, I64, I64, I64, P, I64]
        f.restype = ctypes.c_int
    lib.orc_gemm_s4s4_i32.argtypes = [P, I64, P, I64, P, I64, I64, I64, P, I64]
    lib.orc_gemm_s4s4_i32.restype = ctypes.c_int
    lib.orc_conv_out_size.argtypes = [I64, I64, I64, I64]
    lib.orc_conv_out_size.restype = I64
    lib.orc_conv_macs.argtypes = [I64] * 11
    lib.orc_conv_macs.restype = I64
    lib.orc_conv2d_acc.argtypes = [P, P] + [I64] * 11 + [P, I64, P]
    lib.orc_conv2d_acc.restype = ctypes.c_int
    lib.orc_conv2d_nhwc_s8_requant.argtypes = [P, P, P, P, P, P] + [I64] * 11 + [P, I64]
    lib.orc_conv2d_nhwc_s8_requant.restype = ctypes.c_int
    lib.orc_dwconv_macs.argtypes = [I64] * 10
    lib.orc_dwconv_macs.restype = I64
    lib.orc_dwconv2d_acc.argtypes = [P, P] + [I64] * 10 + [P, I64, P]
    lib.orc_dwconv2d_acc.restype = ctypes.c_int
    lib.orc_dwconv2d_nhwc_s8_requant.argtypes = [P, P, P, P, P, P] + [I64] * 10 + [P, I64]
    lib.orc_dwconv2d_nhwc_s8_requant.restype = ctypes.c_int
    lib.orc_requant_zp.argtypes = [I64, I32, I32, I32, I32, I32, I32, P]
    lib.orc_requant_zp.restype = ctypes.c_int
    lib.orc_gemm_s8s8_acc_zp.argtypes = [P, I64, P, I64, I32, I32, I64, I64, P, I64, P]
    lib.orc_gemm_s8s8_acc_zp.restype = ctypes.c_int
    lib.orc_gemm_s8s8_requant_zp.argtypes = [P, I64, P, I64, P, P, P, I32, I32, I32, I32, I32,
                                             P, I64, I64, I64, P, I64]
    lib.orc_gemm_s8s8_requant_zp.restype = ctypes.c_int
    lib.orc_conv2d_acc_zp.argtypes = [P, P] + [I64] * 11 + [I32, I32, P, I64, P]
    lib.orc_conv2d_acc_zp.restype = ctypes.c_int
    lib.orc_conv2d_nhwc_s8_requant_zp.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P] + \
        [I64] * 11 + [P, I64]
    lib.orc_conv2d_nhwc_s8_requant_zp.restype = ctypes.c_int
    lib.orc_dwconv2d_acc_zp.argtypes = [P, P] + [I64] * 10 + [I32, I32, P, I64, P]
    lib.orc_dwconv2d_acc_zp.restype = ctypes.c_int
    lib.orc_dwconv2d_nhwc_s8_requant_zp.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P] + \
        [I64] * 10 + [P, I64]
    lib.orc_dwconv2d_nhwc_s8_requant_zp.restype = ctypes.c_int
    lib.orc_int4_at_msb.argtypes = [P, I64]
    lib.orc_int4_at_msb.restype = ctypes.c_int
    lib.orc_gemm_s4s4_i32_msb.argtypes = [P, I64, P, I64, P, I64, I64, I64, P, I64]
    lib.orc_gemm_s4s4_i32_msb.restype = ctypes.c_int
    lib.orc_gemm_w4a8_requant_msb.argtypes = [P, I64, P, I64, P, P, P, P, I64, I64, I64, P, I64]
    lib.orc_gemm_w4a8_requant_msb.restype = ctypes.c_int
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_gemm_s4s4_f16.argtypes = [P, I64, P, I64, P, P, P, I64, I64, I64, P, I64]
    lib.orc_gemm_s4s4_f16.restype = ctypes.c_int
    lib.orc_quant_per_token.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.c_float,
                                         ctypes.c_int, P, I64, P]
    lib.orc_quant_per_token.restype = ctypes.c_int
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = None
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


class OracleDomainError(ValueError):
    """An intermediate left the domain the requantize definition covers."""


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _check(status: int, what: str):
    if status != ORC_OK:
        kinds = []
        if status & ORC_E_RANGE:
            kinds.append("int32 range exceeded")
        if status & ORC_E_DOMAIN:
            kinds.append("shift/multiplier outside domain")
        raise OracleDomainError(f"{what}: " + ", ".join(kinds))


def _rows(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.size and (r.min() < 0 or r.max() >= total):
        raise IndexError("row/pixel index out of range")
    return r, int(r.size)


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


def int4_at(packed_row: np.ndarray, i: int) -> int:
    """Signed value of element i of a packed int4 row."""
    row = _c(packed_row, np.uint8)
    if not 0 <= i < 2 * row.size:
        raise IndexError(i)
    return int(_load().orc_int4_at(row.ctypes.data, int(i)))


def int4_at_msb(packed_row: np.ndarray, i: int) -> int:
    """Signed value of element i of an MSB-first packed int4 row."""
    row = _c(packed_row, np.uint8)
    if not 0 <= i < 2 * row.size:
        raise IndexError(i)
    return int(_load().orc_int4_at_msb(row.ctypes.data, int(i)))


def requant_zp(acc: int, bias: int, mult: int, shift: int, out_zero: int,
               act=(-128, 127)) -> int:
    """clamp((((acc + bias) * mult + 2^(shift-1)) >> shift) + out_zero) to
    [act[0], act[1]] (the int8 range by default; (out_zero, 127) is ReLU)."""
    out = np.zeros(1, dtype=np.int8)
    st = _load().orc_requant_zp(int(acc), int(bias), int(mult), int(shift), int(out_zero),
                                int(act[0]), int(act[1]), out.ctypes.data)
    _check(st, "requant_zp")
    return int(out[0])


def requant(acc: int, bias: int, mult: int, shift: int) -> int:
    """One Q31 requantize: clamp(((acc + bias) * mult + 2^(shift-1)) >> shift)."""
    out = np.zeros(1, dtype=np.int8)
    st = _load().orc_requant(int(acc), int(bias), int(mult), int(shift), out.ctypes.data)
    _check(st, "requant")
    return int(out[0])


def requant_many(acc, bias, mult, shift):
    """The requantize applied case by case to equal-length arrays."""
    acc = _c(acc, np.int64)
    bias = _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    out = np.zeros(acc.size, dtype=np.int8)
    st = _load().orc_requant_many(acc.ctypes.data, bias.ctypes.data, mult.ctypes.data,
                                  shift.ctypes.data, out.ctypes.data, acc.size)
    _check(st, "requant_many")
    return out


def _kind(a):
    return 4 if a.dtype == np.uint8 else 8


def gemm_acc(A, B, K=None, rows=None):
    """int64 accumulators sum_k A[m][k] * B[n][k].

    ``A``/``B`` are int8 ``[*, K]`` or packed uint8 ``[*, K/2]``.
    """
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    ka, kb = _kind(A), _kind(B)
    if (ka, kb) not in ((8, 8), (4, 4), (8, 4)):
        raise TypeError("operand kinds must be s8s8, s4s4 or s8 x s4")
    lda = A.shape[1] * (2 if ka == 4 else 1)
    ldb = B.shape[1] * (2 if kb == 4 else 1)
    if K is None:
        K = min(lda, ldb)
    N = B.shape[0]
    r, nr = _rows(rows, A.shape[0])
    out = np.zeros((nr, N), dtype=np.int64)
    _check(_load().orc_gemm_acc(ka, A.ctypes.data, lda, kb, B.ctypes.data, ldb, N, K,
                                _ptr(r), nr, out.ctypes.data), "gemm_acc")
    return out


def gemm_s8s8_requant(A, B, bias, mult, shift, rows=None):
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(rows, M)
    C = np.zeros((nr, N), dtype=np.int8)
    st = _load().orc_gemm_s8s8_requant(A.ctypes.data, K, B.ctypes.data, K, _ptr(bias_c),
                                       mult.ctypes.data, shift.ctypes.data, C.ctypes.data, N,
                                       N, K, _ptr(r), nr)
    _check(st, "gemm_s8s8_requant")
    return C


def gemm_w4a8_requant(A, Bp, bias, mult, shift, rows=None, msb_first=False):
    """int8 A [M][K] x packed int4 B [N][K/2] (low nibble first, or high
    nibble first with msb_first) -> requantized int8."""
    A = _c(A, np.int8)
    Bp = _c(Bp, np.uint8)
    M, K = A.shape
    N = Bp.shape[0]
    assert Bp.shape[1] * 2 == K
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(rows, M)
    C = np.zeros((nr, N), dtype=np.int8)
    f = _load().orc_gemm_w4a8_requant_msb if msb_first else _load().orc_gemm_w4a8_requant
    st = f(A.ctypes.data, K, Bp.ctypes.data, K, _ptr(bias_c),
                                       mult.ctypes.data, shift.ctypes.data, C.ctypes.data, N,
                                       N, K, _ptr(r), nr)
    _check(st, "gemm_w4a8_requant")
    return C


def gemm_s4s4_i32(Ap, Bp, rows=None, msb_first=False):
    """packed int4 A [M][K/2] x packed int4 B [N][K/2] -> raw int32; both
    operands low nibble first, or both high nibble first with msb_first."""
    Ap = _c(Ap, np.uint8)
    Bp = _c(Bp, np.uint8)
    M, Kh = Ap.shape
    N = Bp.shape[0]
    assert Bp.shape[1] == Kh
    K = 2 * Kh
    r, nr = _rows(rows, M)
    C = np.zeros((nr, N), dtype=np.int32)
    f = _load().orc_gemm_s4s4_i32_msb if msb_first else _load().orc_gemm_s4s4_i32
    st = f(Ap.ctypes.data, K, Bp.ctypes.data, K, C.ctypes.data, N,
                                   N, K, _ptr(r), nr)
    _check(st, "gemm_s4s4_i32")
    return C


def f32_to_f16(x) -> int:
    """binary16 bit pattern of binary32 x, rounded to nearest, ties to even."""
    return int(_load().orc_f32_to_f16(float(np.float32(x))))


def gemm_s4s4_f16(Ap, Bp, scale_a=None, scale_b=None, rows=None):
    """packed int4 A [M][K/2] x packed int4 B [N][K/2] -> binary16 C (as a
    float16 array): fp16(fp32(acc) * scale_a[m] * scale_b[n]), scales
    optional."""
    Ap = _c(Ap, np.uint8)
    Bp = _c(Bp, np.uint8)
    M, Kh = Ap.shape
    N = Bp.shape[0]
    assert Bp.shape[1] == Kh
    K = 2 * Kh
    sa = None if scale_a is None else _c(scale_a, np.float32)
    sb = None if scale_b is None else _c(scale_b, np.float32)
    r, nr = _rows(rows, M)
    C = np.zeros((nr, N), dtype=np.uint16)
    st = _load().orc_gemm_s4s4_f16(Ap.ctypes.data, K, Bp.ctypes.data, K, _ptr(sa), _ptr(sb),
                                   C.ctypes.data, N, N, K, _ptr(r), nr)
    _check(st, "gemm_s4s4_f16")
    return C.view(np.float16)


def conv_out_size(n, k, stride, pad) -> int:
    return int(_load().orc_conv_out_size(int(n), int(k), int(stride), int(pad)))


def conv_macs(batch, H, W, C_in, C_out, KH, KW, sh, sw, ph, pw) -> int:
    return int(_load().orc_conv_macs(*(int(v) for v in (batch, H, W, C_in, C_out,
                                                          KH, KW, sh, sw, ph, pw))))


def _conv_geom(X, Wt, stride, pad):
    X = _c(X, np.int8)
    Wt = _c(Wt, np.int8)
    batch, H, W, C_in = X.shape
    C_out, KH, KW, C_in2 = Wt.shape
    assert C_in2 == C_in
    sh, sw = stride
    ph, pw = pad
    Ho = conv_out_size(H, KH, sh, ph)
    Wo = conv_out_size(W, KW, sw, pw)
    return X, Wt, (batch, H, W, C_in, C_out, KH, KW, sh, sw, ph, pw), Ho, Wo


def conv2d_acc(X, Wt, stride=(1, 1), pad=(1, 1), pix=None):
    """int64 accumulators of an NHWC conv; returns [batch, Ho, Wo, C_out] or [npix, C_out]."""
    X, Wt, g, Ho, Wo = _conv_geom(X, Wt, stride, pad)
    batch, C_out = g[0], g[4]
    r, nr = _rows(pix, batch * Ho * Wo)
    out = np.zeros((nr, C_out), dtype=np.int64)
    _check(_load().orc_conv2d_acc(X.ctypes.data, Wt.ctypes.data, *g, _ptr(r), nr,
                                  out.ctypes.data), "conv2d_acc")
    if pix is None:
        return out.reshape(batch, Ho, Wo, C_out)
    return out


def conv2d_nhwc_s8_requant(X, Wt, bias, mult, shift, stride=(1, 1), pad=(1, 1), pix=None):
    """Requantized int8 NHWC conv; returns [batch, Ho, Wo, C_out] or [npix, C_out]."""
    X, Wt, g, Ho, Wo = _conv_geom(X, Wt, stride, pad)
    batch, C_out = g[0], g[4]
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(pix, batch * Ho * Wo)
    Y = np.zeros((nr, C_out), dtype=np.int8)
    st = _load().orc_conv2d_nhwc_s8_requant(X.ctypes.data, Wt.ctypes.data, _ptr(bias_c),
                                            mult.ctypes.data, shift.ctypes.data, Y.ctypes.data,
                                            *g, _ptr(r), nr)
    _check(st, "conv2d_nhwc_s8_requant")
    if pix is None:
        return Y.reshape(batch, Ho, Wo, C_out)
    return Y


# ---- depthwise conv: weights [KH][KW][C] (one input channel per output) ----

def dwconv_macs(batch, H, W, C, KH, KW, sh, sw, ph, pw) -> int:
    return int(_load().orc_dwconv_macs(*(int(v) for v in (batch, H, W, C, KH, KW,
                                                            sh, sw, ph, pw))))


def _dw_geom(X, Wt, stride, pad):
    X = _c(X, np.int8)
    Wt = _c(Wt, np.int8)
    batch, H, W, C = X.shape
    KH, KW, C2 = Wt.shape
    assert C2 == C
    sh, sw = stride
    ph, pw = pad
    Ho = conv_out_size(H, KH, sh, ph)
    Wo = conv_out_size(W, KW, sw, pw)
    return X, Wt, (batch, H, W, C, KH, KW, sh, sw, ph, pw), Ho, Wo


def dwconv2d_acc(X, Wt, stride=(1, 1), pad=(1, 1), pix=None):
    """int64 accumulators of a depthwise NHWC conv (Wt [KH, KW, C]); returns
    [batch, Ho, Wo, C] or [npix, C]."""
    X, Wt, g, Ho, Wo = _dw_geom(X, Wt, stride, pad)
    batch, C = g[0], g[3]
    r, nr = _rows(pix, batch * Ho * Wo)
    out = np.zeros((nr, C), dtype=np.int64)
    _check(_load().orc_dwconv2d_acc(X.ctypes.data, Wt.ctypes.data, *g, _ptr(r), nr,
                                    out.ctypes.data), "dwconv2d_acc")
    if pix is None:
        return out.reshape(batch, Ho, Wo, C)
    return out


def dwconv2d_nhwc_s8_requant(X, Wt, bias, mult, shift, stride=(1, 1), pad=(1, 1), pix=None):
    """Requantized int8 depthwise NHWC conv; returns [batch, Ho, Wo, C] or [npix, C]."""
    X, Wt, g, Ho, Wo = _dw_geom(X, Wt, stride, pad)
    batch, C = g[0], g[3]
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(pix, batch * Ho * Wo)
    Y = np.zeros((nr, C), dtype=np.int8)
    st = _load().orc_dwconv2d_nhwc_s8_requant(X.ctypes.data, Wt.ctypes.data, _ptr(bias_c),
                                              mult.ctypes.data, shift.ctypes.data,
                                              Y.ctypes.data, *g, _ptr(r), nr)
    _check(st, "dwconv2d_nhwc_s8_requant")
    if pix is None:
        return Y.reshape(batch, Ho, Wo, C)
    return Y


# ---- per-token activation quantizer ----

_DTYPES = {"float32": 0, "float16": 1, "bfloat16": 2}


def quant_per_token(X, bits=8, clip_ratio=1.0, dtype=None):
    """Per-token symmetric quantization of X [M][K] to int8 (bits 8) or packed
    int4 (bits 4, uint8 [M][K/2]); returns (Q, scale float32 [M]).

    X is a float32 or float16 array, or a uint16 array of bfloat16 bit
    patterns with dtype="bfloat16".  Codes are decided in binary32."""
    X = np.ascontiguousarray(X)
    if dtype is None:
        dtype = {np.dtype(np.float32): "float32", np.dtype(np.float16): "float16"}[X.dtype]
    code = _DTYPES[dtype]
    if code == 2 and X.dtype != np.uint16:
        raise TypeError("bfloat16 input is passed as uint16 bit patterns")
    M, K = X.shape
    if bits == 4:
        assert K % 2 == 0
        Q = np.zeros((M, K // 2), dtype=np.uint8)
        ldq = K
    else:
        Q = np.zeros((M, K), dtype=np.int8)
        ldq = K
    scale = np.zeros(M, dtype=np.float32)
    st = _load().orc_quant_per_token(X.ctypes.data, code, K, M, K, float(clip_ratio), bits,
                                     Q.ctypes.data, ldq, scale.ctypes.data)
    _check(st, "quant_per_token")
    return Q, scale


def f16_to_f32(h):
    return float(_load().orc_f16_to_f32(int(h)))


def bf16_to_f32(b):
    return float(_load().orc_bf16_to_f32(int(b)))


# ---- asymmetric forms: per-tensor zero points of A (or X), B (or W) and
# the output; padding holds the input zero point ----

def gemm_s8s8_acc_zp(A, B, a_zero, b_zero, rows=None):
    """int64 accumulators sum_k (A[m][k] - a_zero) * (B[n][k] - b_zero)."""
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    r, nr = _rows(rows, M)
    out = np.zeros((nr, N), dtype=np.int64)
    _check(_load().orc_gemm_s8s8_acc_zp(A.ctypes.data, K, B.ctypes.data, K, int(a_zero),
                                        int(b_zero), N, K, _ptr(r), nr, out.ctypes.data),
           "gemm_s8s8_acc_zp")
    return out


def gemm_s8s8_requant_zp(A, B, bias, mult, shift, a_zero, b_zero, out_zero, rows=None,
                         act=(-128, 127)):
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(rows, M)
    C = np.zeros((nr, N), dtype=np.int8)
    st = _load().orc_gemm_s8s8_requant_zp(A.ctypes.data, K, B.ctypes.data, K, _ptr(bias_c),
                                          mult.ctypes.data, shift.ctypes.data, int(a_zero),
                                          int(b_zero), int(out_zero), int(act[0]), int(act[1]),
                                          C.ctypes.data, N, N, K, _ptr(r), nr)
    _check(st, "gemm_s8s8_requant_zp")
    return C


def conv2d_acc_zp(X, Wt, a_zero, b_zero, stride=(1, 1), pad=(1, 1), pix=None):
    X, Wt, g, Ho, Wo = _conv_geom(X, Wt, stride, pad)
    batch, C_out = g[0], g[4]
    r, nr = _rows(pix, batch * Ho * Wo)
    out = np.zeros((nr, C_out), dtype=np.int64)
    _check(_load().orc_conv2d_acc_zp(X.ctypes.data, Wt.ctypes.data, *g, int(a_zero),
                                     int(b_zero), _ptr(r), nr, out.ctypes.data),
           "conv2d_acc_zp")
    if pix is None:
        return out.reshape(batch, Ho, Wo, C_out)
    return out


def conv2d_nhwc_s8_requant_zp(X, Wt, bias, mult, shift, a_zero, b_zero, out_zero,
                              stride=(1, 1), pad=(1, 1), pix=None, act=(-128, 127)):
    X, Wt, g, Ho, Wo = _conv_geom(X, Wt, stride, pad)
    batch, C_out = g[0], g[4]
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(pix, batch * Ho * Wo)
    Y = np.zeros((nr, C_out), dtype=np.int8)
    st = _load().orc_conv2d_nhwc_s8_requant_zp(X.ctypes.data, Wt.ctypes.data, _ptr(bias_c),
                                               mult.ctypes.data, shift.ctypes.data,
                                               int(a_zero), int(b_zero), int(out_zero),
                                               int(act[0]), int(act[1]), Y.ctypes.data, *g,
                                               _ptr(r), nr)
    _check(st, "conv2d_nhwc_s8_requant_zp")
    if pix is None:
        return Y.reshape(batch, Ho, Wo, C_out)
    return Y


def dwconv2d_acc_zp(X, Wt, a_zero, b_zero, stride=(1, 1), pad=(1, 1), pix=None):
    X, Wt, g, Ho, Wo = _dw_geom(X, Wt, stride, pad)
    batch, C = g[0], g[3]
    r, nr = _rows(pix, batch * Ho * Wo)
    out = np.zeros((nr, C), dtype=np.int64)
    _check(_load().orc_dwconv2d_acc_zp(X.ctypes.data, Wt.ctypes.data, *g, int(a_zero),
                                       int(b_zero), _ptr(r), nr, out.ctypes.data),
           "dwconv2d_acc_zp")
    if pix is None:
        return out.reshape(batch, Ho, Wo, C)
    return out


def dwconv2d_nhwc_s8_requant_zp(X, Wt, bias, mult, shift, a_zero, b_zero, out_zero,
                                stride=(1, 1), pad=(1, 1), pix=None, act=(-128, 127)):
    X, Wt, g, Ho, Wo = _dw_geom(X, Wt, stride, pad)
    batch, C = g[0], g[3]
    bias_c = None if bias is None else _c(bias, np.int32)
    mult = _c(mult, np.int32)
    shift = _c(shift, np.int32)
    r, nr = _rows(pix, batch * Ho * Wo)
    Y = np.zeros((nr, C), dtype=np.int8)
    st = _load().orc_dwconv2d_nhwc_s8_requant_zp(X.ctypes.data, Wt.ctypes.data, _ptr(bias_c),
                                                 mult.ctypes.data, shift.ctypes.data,
                                                 int(a_zero), int(b_zero), int(out_zero),
                                                 int(act[0]), int(act[1]), Y.ctypes.data, *g,
                                                 _ptr(r), nr)
    _check(st, "dwconv2d_nhwc_s8_requant_zp")
    if pix is None:
        return Y.reshape(batch, Ho, Wo, C)
    return Y

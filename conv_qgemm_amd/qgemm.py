"""Python binding of libqgemm (ctypes), with the C ABI's names.

Argument marshalling only: torch tensors on the GPU give device pointers,
leading dimensions and the current stream; every step of the computation runs
in the library's HIP kernels.  If ``libqgemm.so`` is missing or cannot be
loaded, importing this module raises -- there is no fallback path.

Layouts follow ``include/qgemm.h``: A ``[M][K]`` row-major, B ``[N][K]``
(column-major K x N), packed int4 operands as ``uint8`` ``[rows][K/2]`` with
element 2i in the low nibble of byte i, per-output-channel int32 bias /
Q31 multiplier / shift, NHWC activations and OHWI weights for the conv.
"""
from __future__ import annotations

import ctypes
import os

import torch

# QG_LIB may point the loader at another build of the same library (the
# tests load one built with host-side sanitizers this way)
_LIB_PATH = os.environ.get("QG_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libqgemm.so")

QG_OK = 0
QG_ERR_NULLPTR = 1
QG_ERR_INVALID = 2
QG_ERR_NO_DEVICE = 3
QG_ERR_LAUNCH = 4

QG_S4S4_MAX_K = 131040
QG_W4A8_MAX_K = 131040

QG_DT_F32 = 0
QG_DT_F16 = 1
QG_DT_BF16 = 2
_QUANT_DTYPES = {torch.float32: QG_DT_F32, torch.float16: QG_DT_F16,
                 torch.bfloat16: QG_DT_BF16}


class QGemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python conv_qgemm_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.qgemm_s8s8_requant.argtypes = [P, I64, P, I64, P, P, P, P, I64, I64, I64, I64, P]
    lib.qgemm_s8s8_requant.restype = S
    lib.qgemm_s4s4_i32.argtypes = [P, I64, P, I64, P, I64, I64, I64, I64, P]
    lib.qgemm_s4s4_i32.restype = S
    lib.qgemm_w4a8_requant.argtypes = [P, I64, P, I64, P, P, P, P, I64, I64, I64, I64, P]
    lib.qgemm_w4a8_requant.restype = S
    lib.qgemm_s4s4_f16.argtypes = [P, I64, P, I64, P, P, P, I64, I64, I64, I64, P]
    lib.qgemm_s4s4_f16.restype = S
    lib.qgemm_w4a8_requant_msb.argtypes = [P, I64, P, I64, P, P, P, P, I64, I64, I64, I64, P]
    lib.qgemm_w4a8_requant_msb.restype = S
    lib.qconv2d_nhwc_s8_requant.argtypes = [P, P, P, P, P, P] + [I32] * 11 + [P]
    lib.qconv2d_nhwc_s8_requant.restype = S
    lib.qdwconv2d_nhwc_s8_requant.argtypes = [P, P, P, P, P, P] + [I32] * 10 + [P]
    lib.qdwconv2d_nhwc_s8_requant.restype = S
    lib.qquant_per_token.argtypes = [P, I32, I64, P, I64, P, I64, I64, ctypes.c_float, I32, P]
    lib.qquant_per_token.restype = S
    Z = ctypes.c_size_t
    lib.qgemm_s8s8_requant_zp_workspace_size.argtypes = [I64, I64]
    lib.qgemm_s8s8_requant_zp_workspace_size.restype = Z
    lib.qgemm_s8s8_requant_zp.argtypes = [P, I64, P, I64, P, P, P, I32, I32, I32, I32, I32, P,
                                          I64, I64, I64, I64, P, Z, P]
    lib.qgemm_s8s8_requant_zp.restype = S
    lib.qgemm_s8s8_requant_zp_noalloc.argtypes = [P, I64, P, I64, P, P, P, I32, I32, I32, I32,
                                                  I32, P, I64, I64, I64, I64, P]
    lib.qgemm_s8s8_requant_zp_noalloc.restype = S
    lib.qconv2d_nhwc_s8_requant_zp_workspace_size.argtypes = [I32] * 10
    lib.qconv2d_nhwc_s8_requant_zp_workspace_size.restype = Z
    lib.qconv2d_nhwc_s8_requant_zp.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P] + \
        [I32] * 11 + [P, Z, P]
    lib.qconv2d_nhwc_s8_requant_zp.restype = S
    lib.qdwconv2d_nhwc_s8_requant_zp_workspace_size.argtypes = [I32]
    lib.qdwconv2d_nhwc_s8_requant_zp_workspace_size.restype = Z
    lib.qdwconv2d_nhwc_s8_requant_zp.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P] + \
        [I32] * 10 + [P, Z, P]
    lib.qdwconv2d_nhwc_s8_requant_zp.restype = S
    lib.qg_status_string.argtypes = [S]
    lib.qg_status_string.restype = ctypes.c_char_p
    lib.qg_version.argtypes = []
    lib.qg_version.restype = S
    return lib


lib = _load()
EXPORTS = ("qgemm_s8s8_requant", "qgemm_s4s4_i32", "qgemm_s4s4_f16", "qgemm_w4a8_requant",
           "qgemm_w4a8_requant_msb",
           "qconv2d_nhwc_s8_requant", "qdwconv2d_nhwc_s8_requant", "qquant_per_token",
           "qgemm_s8s8_requant_zp_workspace_size", "qgemm_s8s8_requant_zp",
           "qgemm_s8s8_requant_zp_noalloc",
           "qconv2d_nhwc_s8_requant_zp_workspace_size", "qconv2d_nhwc_s8_requant_zp",
           "qdwconv2d_nhwc_s8_requant_zp_workspace_size", "qdwconv2d_nhwc_s8_requant_zp",
           "qg_status_string", "qg_version")


def status_string(status: int) -> str:
    return lib.qg_status_string(int(status)).decode()


def version() -> int:
    return int(lib.qg_version())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, what: str):
    if status != QG_OK:
        raise QGemmError(status, what)


def _on_device(t, name):
    """The library launches on the current HIP device: every tensor must live
    there (a host or foreign-device pointer would reach the kernels)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _mat(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    _on_device(t, name)
    return t


def _vec(t, n, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() < n or t.stride(0) != 1:
        raise ValueError(f"{name} must be a contiguous int32 vector of length >= {n}")
    _on_device(t, name)
    return t


def qgemm_s8s8_requant(A, B, bias, mult, shift, C=None, stream=None):
    """C[m][n] = requant(sum_k A[m][k] * B[n][k]); A int8 [M, K], B int8 [N, K]."""
    _mat(A, torch.int8, "A")
    _mat(B, torch.int8, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if C is None:
        C = torch.empty((M, N), dtype=torch.int8, device=A.device)
    _mat(C, torch.int8, "C")
    st = lib.qgemm_s8s8_requant(_ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                _ptr(_vec(bias, N, "bias")), _ptr(_vec(mult, N, "mult")),
                                _ptr(_vec(shift, N, "shift")), _ptr(C), C.stride(0), M, N, K,
                                _stream(stream))
    _check(st, "qgemm_s8s8_requant")
    return C


def qgemm_s4s4_i32(A, B, C=None, K=None, stream=None):
    """C = A * B^T over packed int4 rows; A uint8 [M, K/2], B uint8 [N, K/2]."""
    _mat(A, torch.uint8, "A")
    _mat(B, torch.uint8, "B")
    M = A.shape[0]
    N = B.shape[0]
    if K is None:
        K = 2 * A.shape[1]
    if 2 * A.shape[1] < K or 2 * B.shape[1] < K:
        raise ValueError("packed rows shorter than K")
    if C is None:
        C = torch.empty((M, N), dtype=torch.int32, device=A.device)
    _mat(C, torch.int32, "C")
    st = lib.qgemm_s4s4_i32(_ptr(A), 2 * A.stride(0), _ptr(B), 2 * B.stride(0), _ptr(C),
                            C.stride(0), M, N, K, _stream(stream))
    _check(st, "qgemm_s4s4_i32")
    return C


def _fvec(t, n, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or t.dim() != 1 or t.numel() < n or t.stride(0) != 1:
        raise ValueError(f"{name} must be a contiguous float32 vector of length >= {n}")
    _on_device(t, name)
    return t


def qgemm_s4s4_f16(A, B, scale_a=None, scale_b=None, C=None, K=None, stream=None):
    """packed int4 A uint8 [M, K/2] x packed int4 B uint8 [N, K/2] -> float16
    C = fp16(fp32(acc) * scale_a[m] * scale_b[n]); the scales are optional
    float32 vectors."""
    _mat(A, torch.uint8, "A")
    _mat(B, torch.uint8, "B")
    M = A.shape[0]
    N = B.shape[0]
    if K is None:
        K = 2 * A.shape[1]
    if 2 * A.shape[1] < K or 2 * B.shape[1] < K:
        raise ValueError("packed rows shorter than K")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float16, device=A.device)
    _mat(C, torch.float16, "C")
    st = lib.qgemm_s4s4_f16(_ptr(A), 2 * A.stride(0), _ptr(B), 2 * B.stride(0),
                            _ptr(_fvec(scale_a, M, "scale_a")), _ptr(_fvec(scale_b, N, "scale_b")),
                            _ptr(C), C.stride(0), M, N, K, _stream(stream))
    _check(st, "qgemm_s4s4_f16")
    return C


def qgemm_w4a8_requant(A, B, bias, mult, shift, C=None, K=None, stream=None, msb_first=False):
    """int8 activations A [M, K] x packed int4 weights B uint8 [N, K/2] -> int8.
    msb_first: the weights hold element 2i in the high nibble of byte i
    (qgemm_w4a8_requant_msb)."""
    _mat(A, torch.int8, "A")
    _mat(B, torch.uint8, "B")
    M = A.shape[0]
    N = B.shape[0]
    if K is None:
        K = A.shape[1]
    if A.shape[1] < K or 2 * B.shape[1] < K:
        raise ValueError("rows shorter than K")
    if C is None:
        C = torch.empty((M, N), dtype=torch.int8, device=A.device)
    _mat(C, torch.int8, "C")
    f = lib.qgemm_w4a8_requant_msb if msb_first else lib.qgemm_w4a8_requant
    st = f(_ptr(A), A.stride(0), _ptr(B), 2 * B.stride(0), _ptr(_vec(bias, N, "bias")),
           _ptr(_vec(mult, N, "mult")), _ptr(_vec(shift, N, "shift")), _ptr(C), C.stride(0), M, N,
           K, _stream(stream))
    _check(st, "qgemm_w4a8_requant_msb" if msb_first else "qgemm_w4a8_requant")
    return C


def conv_out_hw(H, W, KH, KW, stride, pad):
    sh, sw = stride
    ph, pw = pad
    return (H + 2 * ph - KH) // sh + 1, (W + 2 * pw - KW) // sw + 1


def qconv2d_nhwc_s8_requant(X, W, bias, mult, shift, stride=(1, 1), pad=(1, 1), Y=None,
                            stream=None):
    """NHWC int8 conv with zero-point-0 padding and the fused requantize.

    X int8 [batch, H, W, C_in] and W int8 [C_out, KH, KW, C_in], both
    contiguous; returns Y int8 [batch, H_out, W_out, C_out].
    """
    if X.dtype != torch.int8 or W.dtype != torch.int8:
        raise TypeError("X and W must be int8")
    if X.dim() != 4 or W.dim() != 4 or not X.is_contiguous() or not W.is_contiguous():
        raise ValueError("X [B,H,W,C_in] and W [C_out,KH,KW,C_in] must be contiguous 4-D")
    _on_device(X, "X")
    _on_device(W, "W")
    batch, H, Wd, C_in = X.shape
    C_out, KH, KW, C_in2 = W.shape
    if C_in2 != C_in:
        raise ValueError("X and W disagree on C_in")
    Ho, Wo = conv_out_hw(H, Wd, KH, KW, stride, pad)
    if Y is None:
        Y = torch.empty((batch, max(Ho, 0), max(Wo, 0), C_out), dtype=torch.int8,
                        device=X.device)
    if not Y.is_contiguous() or Y.dtype != torch.int8 or tuple(Y.shape) != (batch, Ho, Wo, C_out):
        raise ValueError("Y must be a contiguous int8 [batch, H_out, W_out, C_out] tensor")
    _on_device(Y, "Y")
    st = lib.qconv2d_nhwc_s8_requant(_ptr(X), _ptr(W), _ptr(_vec(bias, C_out, "bias")),
                                     _ptr(_vec(mult, C_out, "mult")),
                                     _ptr(_vec(shift, C_out, "shift")), _ptr(Y),
                                     batch, H, Wd, C_in, C_out, KH, KW, stride[0], stride[1],
                                     pad[0], pad[1], _stream(stream))
    _check(st, "qconv2d_nhwc_s8_requant")
    return Y


def qdwconv2d_nhwc_s8_requant(X, W, bias, mult, shift, stride=(1, 1), pad=(1, 1), Y=None,
                              stream=None):
    """Depthwise NHWC int8 conv (output channel c sees only input channel c)
    with zero-point-0 padding and the fused requantize.

    X int8 [batch, H, W, C] and W int8 [KH, KW, C], both contiguous; returns
    Y int8 [batch, H_out, W_out, C].
    """
    if X.dtype != torch.int8 or W.dtype != torch.int8:
        raise TypeError("X and W must be int8")
    if X.dim() != 4 or W.dim() != 3 or not X.is_contiguous() or not W.is_contiguous():
        raise ValueError("X [B,H,W,C] and W [KH,KW,C] must be contiguous")
    _on_device(X, "X")
    _on_device(W, "W")
    batch, H, Wd, C = X.shape
    KH, KW, C2 = W.shape
    if C2 != C:
        raise ValueError("X and W disagree on C")
    Ho, Wo = conv_out_hw(H, Wd, KH, KW, stride, pad)
    if Y is None:
        Y = torch.empty((batch, max(Ho, 0), max(Wo, 0), C), dtype=torch.int8, device=X.device)
    if not Y.is_contiguous() or Y.dtype != torch.int8 or tuple(Y.shape) != (batch, Ho, Wo, C):
        raise ValueError("Y must be a contiguous int8 [batch, H_out, W_out, C] tensor")
    _on_device(Y, "Y")
    st = lib.qdwconv2d_nhwc_s8_requant(_ptr(X), _ptr(W), _ptr(_vec(bias, C, "bias")),
                                       _ptr(_vec(mult, C, "mult")), _ptr(_vec(shift, C, "shift")),
                                       _ptr(Y), batch, H, Wd, C, KH, KW, stride[0], stride[1],
                                       pad[0], pad[1], _stream(stream))
    _check(st, "qdwconv2d_nhwc_s8_requant")
    return Y


def qquant_per_token(X, bits=8, clip_ratio=1.0, Q=None, scale=None, stream=None):
    """Symmetric per-token quantization of X [M, K] (float32, float16 or
    bfloat16, unit column stride): scale[m] = max|X[m]| / (qmax / clip_ratio),
    codes X / scale rounded half away from zero, clamped to +-qmax (127 for
    bits 8, 7 for bits 4).  Returns (Q, scale): Q int8 [M, K], or for bits 4
    uint8 [M, K/2] with element 2i in the low nibble of byte i; scale float32
    [M]."""
    if X.dtype not in _QUANT_DTYPES:
        raise TypeError(f"X must be float32, float16 or bfloat16, got {X.dtype}")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D tensor with unit column stride")
    _on_device(X, "X")
    M, K = X.shape
    if bits == 8:
        qdtype, qcols = torch.int8, K
    elif bits == 4:
        qdtype, qcols = torch.uint8, K // 2
    else:
        raise ValueError("bits must be 8 or 4")
    if Q is None:
        Q = torch.empty((M, qcols), dtype=qdtype, device=X.device)
    _mat(Q, qdtype, "Q")
    if Q.shape[0] != M or Q.shape[1] < qcols:
        raise ValueError(f"Q must have {M} rows of at least {qcols} columns")
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if scale.dtype != torch.float32 or scale.dim() != 1 or scale.numel() < M or \
            scale.stride(0) != 1:
        raise ValueError(f"scale must be a contiguous float32 vector of length >= {M}")
    _on_device(scale, "scale")
    ldq = Q.stride(0) * (2 if bits == 4 else 1)
    st = lib.qquant_per_token(_ptr(X), _QUANT_DTYPES[X.dtype], X.stride(0), _ptr(Q), ldq,
                              _ptr(scale), M, K, float(clip_ratio), bits, _stream(stream))
    _check(st, "qquant_per_token")
    return Q, scale


# ---- asymmetric (zero-point) forms ----

def _workspace(ws, need, device):
    """The caller's workspace (a uint8 GPU tensor of at least `need` bytes),
    or a new one."""
    if need == 0:
        raise ValueError("the library rejects this shape")
    if ws is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.numel() < need:
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {need} bytes")
    _on_device(ws, "workspace")
    return ws


def qgemm_s8s8_requant_zp(A, B, bias, mult, shift, a_zero, b_zero, out_zero, C=None,
                          workspace=None, stream=None, act=(-128, 127)):
    """Asymmetric int8 GEMM: C = requant(sum_k (A - a_zero)(B - b_zero)) +
    out_zero, saturated to [act[0], act[1]] (the int8 range by default;
    (out_zero, 127) is a fused ReLU).  A int8 [M, K], B int8 [N, K]."""
    _mat(A, torch.int8, "A")
    _mat(B, torch.int8, "B")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    if C is None:
        C = torch.empty((M, N), dtype=torch.int8, device=A.device)
    _mat(C, torch.int8, "C")
    ws = _workspace(workspace, int(lib.qgemm_s8s8_requant_zp_workspace_size(M, N)), A.device)
    st = lib.qgemm_s8s8_requant_zp(_ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                   _ptr(_vec(bias, N, "bias")), _ptr(_vec(mult, N, "mult")),
                                   _ptr(_vec(shift, N, "shift")), int(a_zero), int(b_zero),
                                   int(out_zero), int(act[0]), int(act[1]), _ptr(C), C.stride(0),
                                   M, N, K, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "qgemm_s8s8_requant_zp")
    return C


def qgemm_s8s8_requant_zp_noalloc(A, B, bias, mult, shift, a_zero, b_zero, out_zero, C=None,
                                  stream=None, act=(-128, 127)):
    """qgemm_s8s8_requant_zp through the library's allocation-free entry
    point: no workspace, the compensation sums stay in the library's own
    per-GPU array (M + N up to about 262,000; calls that overlap on one GPU
    race on it).  With C given, nothing is allocated on this path."""
    _mat(A, torch.int8, "A")
    _mat(B, torch.int8, "B")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    if C is None:
        C = torch.empty((M, N), dtype=torch.int8, device=A.device)
    _mat(C, torch.int8, "C")
    st = lib.qgemm_s8s8_requant_zp_noalloc(_ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                           _ptr(_vec(bias, N, "bias")),
                                           _ptr(_vec(mult, N, "mult")),
                                           _ptr(_vec(shift, N, "shift")), int(a_zero),
                                           int(b_zero), int(out_zero), int(act[0]), int(act[1]),
                                           _ptr(C), C.stride(0), M, N, K, _stream(stream))
    _check(st, "qgemm_s8s8_requant_zp_noalloc")
    return C


def qconv2d_nhwc_s8_requant_zp(X, W, bias, mult, shift, a_zero, b_zero, out_zero, stride=(1, 1),
                               pad=(1, 1), Y=None, workspace=None, stream=None, act=(-128, 127)):
    """Asymmetric NHWC int8 conv: padding holds a_zero, products are
    (X - a_zero)(W - b_zero), the output gets out_zero before the
    saturation to [act[0], act[1]].  X [batch, H, W, C_in],
    W [C_out, KH, KW, C_in]."""
    if X.dtype != torch.int8 or W.dtype != torch.int8:
        raise TypeError("X and W must be int8")
    if X.dim() != 4 or W.dim() != 4 or not X.is_contiguous() or not W.is_contiguous():
        raise ValueError("X [B,H,W,C_in] and W [C_out,KH,KW,C_in] must be contiguous 4-D")
    _on_device(X, "X")
    _on_device(W, "W")
    batch, H, Wd, C_in = X.shape
    C_out, KH, KW, C_in2 = W.shape
    if C_in2 != C_in:
        raise ValueError("X and W disagree on C_in")
    Ho, Wo = conv_out_hw(H, Wd, KH, KW, stride, pad)
    if Y is None:
        Y = torch.empty((batch, max(Ho, 0), max(Wo, 0), C_out), dtype=torch.int8,
                        device=X.device)
    if not Y.is_contiguous() or Y.dtype != torch.int8 or tuple(Y.shape) != (batch, Ho, Wo, C_out):
        raise ValueError("Y must be a contiguous int8 [batch, H_out, W_out, C_out] tensor")
    _on_device(Y, "Y")
    need = int(lib.qconv2d_nhwc_s8_requant_zp_workspace_size(batch, H, Wd, C_out, KH, KW,
                                                             stride[0], stride[1], pad[0],
                                                             pad[1]))
    ws = _workspace(workspace, need, X.device)
    st = lib.qconv2d_nhwc_s8_requant_zp(_ptr(X), _ptr(W), _ptr(_vec(bias, C_out, "bias")),
                                        _ptr(_vec(mult, C_out, "mult")),
                                        _ptr(_vec(shift, C_out, "shift")), int(a_zero),
                                        int(b_zero), int(out_zero), int(act[0]), int(act[1]),
                                        _ptr(Y), batch, H, Wd, C_in,
                                        C_out, KH, KW, stride[0], stride[1], pad[0], pad[1],
                                        _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "qconv2d_nhwc_s8_requant_zp")
    return Y


def qdwconv2d_nhwc_s8_requant_zp(X, W, bias, mult, shift, a_zero, b_zero, out_zero,
                                 stride=(1, 1), pad=(1, 1), Y=None, workspace=None, stream=None,
                                 act=(-128, 127)):
    """Asymmetric depthwise NHWC int8 conv (W [KH, KW, C]); zero points as
    for qconv2d_nhwc_s8_requant_zp."""
    if X.dtype != torch.int8 or W.dtype != torch.int8:
        raise TypeError("X and W must be int8")
    if X.dim() != 4 or W.dim() != 3 or not X.is_contiguous() or not W.is_contiguous():
        raise ValueError("X [B,H,W,C] and W [KH,KW,C] must be contiguous")
    _on_device(X, "X")
    _on_device(W, "W")
    batch, H, Wd, C = X.shape
    KH, KW, C2 = W.shape
    if C2 != C:
        raise ValueError("X and W disagree on C")
    Ho, Wo = conv_out_hw(H, Wd, KH, KW, stride, pad)
    if Y is None:
        Y = torch.empty((batch, max(Ho, 0), max(Wo, 0), C), dtype=torch.int8, device=X.device)
    if not Y.is_contiguous() or Y.dtype != torch.int8 or tuple(Y.shape) != (batch, Ho, Wo, C):
        raise ValueError("Y must be a contiguous int8 [batch, H_out, W_out, C] tensor")
    _on_device(Y, "Y")
    ws = _workspace(workspace, int(lib.qdwconv2d_nhwc_s8_requant_zp_workspace_size(C)), X.device)
    st = lib.qdwconv2d_nhwc_s8_requant_zp(_ptr(X), _ptr(W), _ptr(_vec(bias, C, "bias")),
                                          _ptr(_vec(mult, C, "mult")),
                                          _ptr(_vec(shift, C, "shift")), int(a_zero),
                                          int(b_zero), int(out_zero), int(act[0]), int(act[1]),
                                          _ptr(Y), batch, H, Wd, C,
                                          KH, KW, stride[0], stride[1], pad[0], pad[1],
                                          _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "qdwconv2d_nhwc_s8_requant_zp")
    return Y

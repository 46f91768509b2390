"""Seeded synthetic inputs for the quantized GEMM / conv workloads.

This module only draws random numbers; it holds none of the method's
arithmetic.  It serves the CPU oracle, the GPU tests and the benchmark alike.

Every draw uses ``numpy.random.default_rng(seed)`` (PCG64) with inclusive
integer ranges for "[a, b]" / "a..b" and an exclusive upper end for "[a, b)".
Packed signed int4 operands are drawn as uniform random bytes: each byte holds
two independent nibbles, each uniform over the 16 codes, i.e. uniform over
the values [-8, 7] once read as 4-bit two's complement.  Arrays are drawn in
the order A, B, bias, multiplier, shift.

Workloads (sizes from the problem statement; distributions not stated for
some configs take the pointwise config's: int8 weights in [-127, 127], int32
bias in [-2^15, 2^15], Q31 multiplier in [2^30, 2^31), shift in 31..40):

  pointwise   1x1 conv as GEMM, M=320 (20x16 NHWC pixels), K=64, N=64
  s4s4        INT4 x INT4 -> INT32, M=N=K=4096, both operands packed
  conv3x3     NHWC 3x3 s1 p1, batch 32, 56x56, 64 -> 64 channels
  w4a8        skinny M=16, K=8192, N=28672, packed int4 weights
  s8s8        M=N=K=8192 int8, shift 35..44
  dw3x3       depthwise NHWC 3x3 s1 p1, batch 32, 56x56, 64 channels,
              weights [3][3][64] (the MCU front-end page's depthwise layout)
  quant_a8    per-token quantization of bfloat16 activations [8192][8192]
              to int8 codes and float32 scales: the A operand of s8s8
  w4a8_prefill  W4A8 with M=2048 tokens (a prefill chunk), N=28672, K=8192
  w4a8_m64    the skinny W4A8 with 64 tokens (four 16-token blocks)
  s8s8_zp     s8s8 with zero points a=-11, b=6, out=20 (same arrays)
  conv3x3_zp  conv3x3 with zero points a=-5, b=3, out=11 (same arrays)

Float activations (``activations``) are standard normal, each token (row)
scaled by a magnitude drawn log-uniformly from [1/16, 16], and a fixed set of
outlier channels (columns, 1 in 128) scaled by 32 -- the shape of a
transformer layer's input, whose per-token spread and few large channels are
what per-token scales and clipping are for.
"""
from __future__ import annotations

import hashlib

import numpy as np

I8_LO, I8_HI = -127, 127
BIAS_LO, BIAS_HI = -(2 ** 15), 2 ** 15
MULT_LO, MULT_HI = 2 ** 30, 2 ** 31  # upper end exclusive
SHIFT_DEFAULT = (31, 40)

# name -> (kind, shape parameters, shift window, seed)
WORKLOADS = {
    "pointwise": dict(kind="s8s8", M=320, N=64, K=64, shift=(31, 40), seed=1),
    "s4s4": dict(kind="s4s4", M=4096, N=4096, K=4096, seed=2),
    "conv3x3": dict(kind="conv", batch=32, H=56, W=56, C_in=64, C_out=64, KH=3, KW=3,
                    stride=(1, 1), pad=(1, 1), shift=(31, 40), seed=3),
    "w4a8": dict(kind="w4a8", M=16, N=28672, K=8192, shift=(31, 40), seed=4),
    "s8s8": dict(kind="s8s8", M=8192, N=8192, K=8192, shift=(35, 44), seed=5),
    "dw3x3": dict(kind="dwconv", batch=32, H=56, W=56, C=64, KH=3, KW=3,
                  stride=(1, 1), pad=(1, 1), shift=(31, 40), seed=6),
    "quant_a8": dict(kind="quant", M=8192, K=8192, dtype="bfloat16", bits=8, seed=7),
    "w4a8_prefill": dict(kind="w4a8", M=2048, N=28672, K=8192, shift=(31, 40), seed=8),
    "w4a8_m64": dict(kind="w4a8", M=64, N=28672, K=8192, shift=(31, 40), seed=9),
    "s8s8_zp": dict(kind="s8s8", M=8192, N=8192, K=8192, shift=(35, 44), seed=5,
                    zp=(-11, 6, 20)),
    "conv3x3_zp": dict(kind="conv", batch=32, H=56, W=56, C_in=64, C_out=64, KH=3, KW=3,
                       stride=(1, 1), pad=(1, 1), shift=(31, 40), seed=3, zp=(-5, 3, 11)),
}

# Variants whose shift windows keep most outputs inside [-128, 127], so that
# parity is also exercised away from saturation.
UNSATURATED_SHIFT = {"pointwise": (38, 44), "conv3x3": (39, 45), "w4a8": (37, 43),
                     "w4a8_prefill": (37, 43), "w4a8_m64": (37, 43),
                     "s8s8": (41, 47), "dw3x3": (39, 45)}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def int8_uniform(g: np.random.Generator, shape, lo=I8_LO, hi=I8_HI) -> np.ndarray:
    return g.integers(lo, hi, size=shape, endpoint=True, dtype=np.int8)


def int4_packed_uniform(g: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """Packed signed int4 operand [rows][k/2]: uniform random bytes."""
    assert k % 2 == 0
    return g.integers(0, 255, size=(rows, k // 2), endpoint=True, dtype=np.uint8)


def channel_params(g: np.random.Generator, n: int, shift=SHIFT_DEFAULT):
    """Per-output-channel int32 bias, Q31 multiplier and shift."""
    bias = g.integers(BIAS_LO, BIAS_HI, size=n, endpoint=True, dtype=np.int32)
    mult = g.integers(MULT_LO, MULT_HI, size=n, endpoint=False, dtype=np.int64).astype(np.int32)
    sh = g.integers(shift[0], shift[1], size=n, endpoint=True, dtype=np.int32)
    return bias, mult, sh


def gemm_s8s8(M, N, K, seed, shift=SHIFT_DEFAULT):
    g = rng(seed)
    A = int8_uniform(g, (M, K))
    B = int8_uniform(g, (N, K))
    bias, mult, sh = channel_params(g, N, shift)
    return dict(A=A, B=B, bias=bias, mult=mult, shift=sh)


def gemm_s4s4(M, N, K, seed):
    g = rng(seed)
    A = int4_packed_uniform(g, M, K)
    B = int4_packed_uniform(g, N, K)
    return dict(A=A, B=B)


def gemm_w4a8(M, N, K, seed, shift=SHIFT_DEFAULT):
    g = rng(seed)
    A = int8_uniform(g, (M, K))
    B = int4_packed_uniform(g, N, K)
    bias, mult, sh = channel_params(g, N, shift)
    return dict(A=A, B=B, bias=bias, mult=mult, shift=sh)


def conv_nhwc(batch, H, W, C_in, C_out, KH, KW, seed, shift=SHIFT_DEFAULT):
    g = rng(seed)
    X = int8_uniform(g, (batch, H, W, C_in))
    Wt = int8_uniform(g, (C_out, KH, KW, C_in))
    bias, mult, sh = channel_params(g, C_out, shift)
    return dict(X=X, W=Wt, bias=bias, mult=mult, shift=sh)


def dwconv_nhwc(batch, H, W, C, KH, KW, seed, shift=SHIFT_DEFAULT):
    """Depthwise conv operands: X [batch][H][W][C], weights [KH][KW][C]."""
    g = rng(seed)
    X = int8_uniform(g, (batch, H, W, C))
    Wt = int8_uniform(g, (KH, KW, C))
    bias, mult, sh = channel_params(g, C, shift)
    return dict(X=X, W=Wt, bias=bias, mult=mult, shift=sh)


def activations(M, K, seed, outlier_every=128, outlier_gain=32.0):
    """Float32 activations [M][K]: standard normal, times a per-token
    magnitude 2^u with u uniform in [-4, 4), with every outlier_every-th
    channel (from a random offset) times outlier_gain.  Draw order: values,
    token exponents, outlier offset."""
    g = rng(seed)
    X = g.standard_normal((M, K), dtype=np.float32)
    u = g.uniform(-4.0, 4.0, size=(M, 1)).astype(np.float32)
    X *= np.exp2(u)
    off = int(g.integers(0, outlier_every))
    X[:, off::outlier_every] *= np.float32(outlier_gain)
    return X


def workload(name: str, unsaturated: bool = False, seed: int | None = None):
    """Arrays of a named workload (seeded); ``unsaturated`` picks the
    parity variant's shift window and seeds 101..105."""
    w = dict(WORKLOADS[name])
    s = w["seed"] + (100 if unsaturated else 0) if seed is None else seed
    shift = UNSATURATED_SHIFT.get(name, w.get("shift")) if unsaturated else w.get("shift")
    k = w["kind"]
    if k == "s8s8":
        return gemm_s8s8(w["M"], w["N"], w["K"], s, shift)
    if k == "s4s4":
        return gemm_s4s4(w["M"], w["N"], w["K"], s)
    if k == "w4a8":
        return gemm_w4a8(w["M"], w["N"], w["K"], s, shift)
    if k == "conv":
        return conv_nhwc(w["batch"], w["H"], w["W"], w["C_in"], w["C_out"], w["KH"], w["KW"],
                         s, shift)
    if k == "dwconv":
        return dwconv_nhwc(w["batch"], w["H"], w["W"], w["C"], w["KH"], w["KW"], s, shift)
    if k == "quant":
        return dict(X=activations(w["M"], w["K"], s))
    raise KeyError(name)


def sha256(arrays: dict) -> dict:
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
            for k, v in arrays.items()}

"""Pins of the oracle's INT4 x INT4 GEMM with a binary16 output (INT4 GEMM
article, www.cf-1.com/news/6060138, §6: C in FP16, converted from the int32
accumulator) and of its binary32 -> binary16 rounding.

The conversion is checked against numpy's IEEE conversion (round to nearest,
ties to even) over every exponent, tie and overflow boundary; the GEMM
against the pinned int32 oracle plus that conversion, closed forms with
power-of-two scales, and the overflow point of binary16.
"""
import numpy as np
import pytest

from conv_qgemm_amd import datagen


def _np_f16_bits(x32):
    with np.errstate(over="ignore"):
        return np.asarray(x32, np.float32).astype(np.float16).view(np.uint16)


def test_conversion_matches_ieee_rne(orc):
    g = np.random.default_rng(1)
    vals = []
    # every binary16-relevant exponent, random significands, both signs
    for e in range(-30, 18):
        m = g.integers(0, 1 << 23, size=40, dtype=np.uint32)
        bits = ((e + 127) << 23) | m
        vals.append(bits.astype(np.uint32).view(np.float32))
    # exact ties and their neighbours at several exponents (normal: 13 low
    # bits dropped; subnormal: more)
    for e in (-24, -20, -15, -14, -13, 0, 5, 15):
        for low in (0x1000, 0x0FFF, 0x1001, 0x3000, 0x2000):
            for hi in (0, 1, 0x155, 0x3FF):
                bits = np.uint32(((e + 127) << 23) | (hi << 13) | low)
                vals.append(np.array([bits], np.uint32).view(np.float32))
    x = np.concatenate(vals)
    x = np.concatenate([x, -x, np.float32([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e9,
                                           2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25,
                                           2.0 ** -26, np.inf, -np.inf])])
    want = _np_f16_bits(x)
    got = np.array([orc.f32_to_f16(v) for v in x], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]
    # a NaN stays a NaN of the same sign (the quiet NaN as numpy gives it)
    qnan = np.float32(np.nan)
    assert orc.f32_to_f16(qnan) == int(_np_f16_bits(qnan))
    assert orc.f32_to_f16(-qnan) == int(_np_f16_bits(-qnan))
    for bits in (0x7F800001, 0x7FBFFFFF, 0xFFC00000, 0xFF800010):
        h = orc.f32_to_f16(np.array([bits], np.uint32).view(np.float32)[0])
        assert (h & 0x7C00) == 0x7C00 and (h & 0x3FF) != 0 and (h >> 15) == (bits >> 31)


@pytest.mark.parametrize("M,N,K", [(1, 1, 2), (7, 9, 64), (33, 20, 256), (5, 3, 4096)])
def test_gemm_f16_plain_is_the_converted_accumulator(orc, M, N, K):
    d = datagen.gemm_s4s4(M, N, K, seed=M + N + K)
    acc = orc.gemm_s4s4_i32(d["A"], d["B"])
    got = orc.gemm_s4s4_f16(d["A"], d["B"])
    assert np.array_equal(got.view(np.uint16), _np_f16_bits(acc.astype(np.float32)))


def test_gemm_f16_scales(orc):
    d = datagen.gemm_s4s4(40, 24, 512, seed=3)
    g = np.random.default_rng(4)
    sa = g.uniform(1e-3, 2.0, 40).astype(np.float32)
    sb = g.uniform(1e-3, 2.0, 24).astype(np.float32)
    acc = orc.gemm_s4s4_i32(d["A"], d["B"]).astype(np.float32)
    got = orc.gemm_s4s4_f16(d["A"], d["B"], sa, sb)
    # (acc * sa) * sb, each product rounded to binary32, then to binary16
    want = _np_f16_bits((acc * sa[:, None]).astype(np.float32) * sb[None, :])
    assert np.array_equal(got.view(np.uint16), want)
    # either scale alone, and power-of-two scales that only move the exponent
    assert np.array_equal(orc.gemm_s4s4_f16(d["A"], d["B"], sa, None).view(np.uint16),
                          _np_f16_bits(acc * sa[:, None]))
    # a subset of rows takes each selected row's own scale
    rows = np.array([39, 0, 17, 17], np.int64)
    sub = orc.gemm_s4s4_f16(d["A"], d["B"], sa, sb, rows=rows)
    assert np.array_equal(sub.view(np.uint16), got.view(np.uint16)[rows])
    p2a = np.full(40, 2.0 ** -4, np.float32)
    p2b = np.full(24, 2.0 ** -3, np.float32)
    assert np.array_equal(orc.gemm_s4s4_f16(d["A"], d["B"], p2a, p2b).view(np.uint16),
                          _np_f16_bits(acc / 128.0))


def test_gemm_f16_overflow_point(orc):
    """All -8 x -8: acc = 64 K.  K = 1022 gives 65408, a binary16 value;
    K = 1024 gives 65536, which rounds to infinity."""
    for K, want in ((1022, 65408.0), (1024, np.inf)):
        A = np.full((1, K // 2), 0x88, np.uint8)
        out = orc.gemm_s4s4_f16(A, A)
        assert out[0, 0] == want
    A = np.full((1, 512), 0x88, np.uint8)
    assert orc.gemm_s4s4_f16(A, A, np.float32([-1.0]), None)[0, 0] == -np.inf

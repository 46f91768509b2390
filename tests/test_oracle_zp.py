"""Pins of the oracle's asymmetric forms and of MSB-first INT4 packing.

Definitions: a code Q stands for (Q - zero_point) * scale (Voyager
quantization article, www.dpshk.com/news/2695434, §1.1), so the GEMM's
integer accumulator is sum_k (A - za) * (B - zb), both operands carrying a
zero point (INT4 GEMM article, www.cf-1.com/news/6060138, §4.1); the padding
of an asymmetric input is its zero point, and the requantize adds the output
zero point (MCU conv front-end article, news.rkmt.cn/news/16638, §2.3, §3.3).
MSB-first packing puts element 2i in the high nibble (INT4 GEMM article
§3.2's alternative order, the packing of its §4.1 script).

Each pin reaches the result by another route: the symmetric oracle (already
pinned) plus the row/column-sum expansion of the product, invariance under
shifting codes and zero point together, closed forms, hand-worked values, an
explicit im2col with the zero point as padding, and the nibble swap that
turns one packing order into the other.
"""
import numpy as np
import pytest

from conv_qgemm_amd import datagen


def _i8(g, shape, lo=-128, hi=127):
    return g.integers(lo, hi, size=shape, endpoint=True, dtype=np.int8)


# ---------------------------------------------------------------- requantize

# acc, bias, mult, shift, out_zero, expected; mult 2^30 with shift 31 halves
HAND = [
    (200, 0, 2 ** 30, 31, 0, 100),
    (200, 0, 2 ** 30, 31, 10, 110),
    (200, 0, 2 ** 30, 31, 27, 127),      # 100 + 27 just fits
    (200, 0, 2 ** 30, 31, 28, 127),      # 128 saturates
    (200, 0, 2 ** 30, 31, -128, -28),
    (-300, 0, 2 ** 30, 31, -128, -128),  # -150 - 128 saturates low
    (-300, 0, 2 ** 30, 31, 127, -23),
    (3, 0, 2 ** 30, 31, -2, 0),          # 1.5 rounds up to 2, then -2
    (-3, 0, 2 ** 30, 31, 5, 4),          # -1.5 rounds up to -1, then +5
    (100, 56, 2 ** 30, 31, 1, 79),       # bias first: (100 + 56) / 2 + 1
    (2 ** 31 - 1, 0, 2 ** 31 - 1, 1, -128, 127),  # far past int8 before the zero point
    (-2 ** 31, 0, 2 ** 31 - 1, 1, 127, -128),
]


@pytest.mark.parametrize("acc,bias,mult,shift,zo,want", HAND)
def test_requant_zp_hand(orc, acc, bias, mult, shift, zo, want):
    assert orc.requant_zp(acc, bias, mult, shift, zo) == want


def test_requant_zp_reduces_and_shifts(orc):
    g = np.random.default_rng(1)
    for _ in range(3000):
        acc = int(g.integers(-2 ** 20, 2 ** 20))
        bias = int(g.integers(-2 ** 15, 2 ** 15))
        mult = int(g.integers(2 ** 30, 2 ** 31))
        shift = int(g.integers(20, 40))
        zo = int(g.integers(-128, 128))
        base = orc.requant(acc, bias, mult, shift)
        assert orc.requant_zp(acc, bias, mult, shift, 0) == base
        # away from saturation the zero point is a plain offset
        if -100 < base < 100 and -128 <= base + zo <= 127:
            assert orc.requant_zp(acc, bias, mult, shift, zo) == base + zo
    with pytest.raises(orc.OracleDomainError):
        orc.requant_zp(1, 0, 2 ** 30, 31, 128)


# acc, bias, mult, shift, out_zero, (act_min, act_max), expected
HAND_ACT = [
    (200, 0, 2 ** 30, 31, 10, (-128, 100), 100),   # 110 capped by the upper bound
    (-300, 0, 2 ** 30, 31, 0, (0, 127), 0),         # ReLU of -150
    (-300, 0, 2 ** 30, 31, -20, (-20, 127), -20),   # ReLU at a nonzero zero point
    (3, 0, 2 ** 30, 31, -2, (-2, 127), 0),          # above the ReLU bound: unchanged
    (200, 0, 2 ** 30, 31, -128, (-50, 50), -28),    # inside the bounds: unchanged
    (2 ** 31 - 1, 0, 2 ** 31 - 1, 1, 5, (5, 17), 17),
]


@pytest.mark.parametrize("acc,bias,mult,shift,zo,act,want", HAND_ACT)
def test_requant_act_hand(orc, acc, bias, mult, shift, zo, act, want):
    assert orc.requant_zp(acc, bias, mult, shift, zo, act=act) == want


def test_requant_act_is_a_clamp_of_the_plain_result(orc):
    g = np.random.default_rng(11)
    for _ in range(2000):
        acc = int(g.integers(-2 ** 22, 2 ** 22))
        mult = int(g.integers(2 ** 30, 2 ** 31))
        shift = int(g.integers(25, 40))
        zo = int(g.integers(-128, 128))
        lo = int(g.integers(-128, 128))
        hi = int(g.integers(lo, 128))
        y = orc.requant_zp(acc, 0, mult, shift, zo)
        assert orc.requant_zp(acc, 0, mult, shift, zo, act=(lo, hi)) == min(max(y, lo), hi)
        assert orc.requant_zp(acc, 0, mult, shift, zo, act=(zo, 127)) == max(y, zo)  # ReLU
    for bad in ((5, 4), (-129, 0), (0, 128)):
        with pytest.raises(orc.OracleDomainError):
            orc.requant_zp(1, 0, 2 ** 30, 31, 0, act=bad)


# ---------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 16), (33, 9, 100), (17, 40, 257)])
@pytest.mark.parametrize("za,zb", [(0, 0), (-128, 0), (0, 127), (17, -5), (-128, -128)])
def test_gemm_zp_row_column_expansion(orc, M, N, K, za, zb):
    """sum (a - za)(b - zb) = sum ab - zb sum a - za sum b + K za zb, with
    sum ab from the symmetric oracle and the sums from numpy."""
    g = np.random.default_rng(M * 100 + N + K)
    A, B = _i8(g, (M, K)), _i8(g, (N, K))
    raw = orc.gemm_acc(A, B)
    ra = A.astype(np.int64).sum(axis=1)
    cb = B.astype(np.int64).sum(axis=1)
    want = raw - zb * ra[:, None] - za * cb[None, :] + K * za * zb
    assert np.array_equal(orc.gemm_s8s8_acc_zp(A, B, za, zb), want)


def test_gemm_zp_shift_invariance(orc):
    """Shifting every code of an operand and its zero point together leaves
    the real values, hence the accumulator, unchanged."""
    g = np.random.default_rng(2)
    A = _i8(g, (12, 48), -100, 100)
    B = _i8(g, (10, 48), -100, 100)
    base = orc.gemm_s8s8_acc_zp(A, B, 3, -4)
    assert np.array_equal(orc.gemm_s8s8_acc_zp((A + 20).astype(np.int8), B, 23, -4), base)
    assert np.array_equal(orc.gemm_s8s8_acc_zp(A, (B - 27).astype(np.int8), 3, -31), base)
    # a zero point that does not move with the codes does change the result
    assert not np.array_equal(orc.gemm_s8s8_acc_zp((A + 20).astype(np.int8), B, 3, -4), base)


def test_gemm_zp_closed_forms(orc):
    K = 64
    A = np.full((3, K), 9, np.int8)
    B = np.full((4, K), -7, np.int8)
    assert np.all(orc.gemm_s8s8_acc_zp(A, B, 2, 5) == K * (9 - 2) * (-7 - 5))
    # codes equal to their zero point are real zeros
    assert np.all(orc.gemm_s8s8_acc_zp(A, B, 9, 100 - 128) == 0)
    # extremes: (127 - (-128)) * (-128 - 127) per term
    A = np.full((1, K), 127, np.int8)
    B = np.full((1, K), -128, np.int8)
    assert orc.gemm_s8s8_acc_zp(A, B, -128, 127)[0, 0] == K * 255 * -255


def test_gemm_zp_requant_composition(orc):
    d = datagen.gemm_s8s8(21, 30, 96, seed=3, shift=(36, 42))
    za, zb, zo = -37, 11, 23
    acc = orc.gemm_s8s8_acc_zp(d["A"], d["B"], za, zb)
    C = orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"], za, zb, zo)
    want = np.array([[orc.requant_zp(int(acc[m, n]), int(d["bias"][n]), int(d["mult"][n]),
                                     int(d["shift"][n]), zo) for n in range(30)]
                     for m in range(21)], dtype=np.int8)
    assert np.array_equal(C, want)
    sym = orc.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"],
                                                   d["shift"], 0, 0, 0), sym)
    rows = np.array([0, 7, 20])
    assert np.array_equal(orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"],
                                                   d["shift"], za, zb, zo, rows=rows), C[rows])
    relu = orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"], za, zb, zo,
                                    act=(zo, 127))
    assert np.array_equal(relu, np.maximum(C, zo))
    assert (C < zo).any()  # the ReLU case is not vacuous


def test_gemm_zp_domain(orc):
    A = np.zeros((2, 16), np.int8)
    with pytest.raises(orc.OracleDomainError):
        orc.gemm_s8s8_acc_zp(A, A, 128, 0)
    with pytest.raises(orc.OracleDomainError):
        orc.gemm_s8s8_acc_zp(A, A, 0, -129)


# ---------------------------------------------------------------- conv

def _im2col_zp(X, KH, KW, stride, pad, za):
    """Explicit im2col rows (tap-major, channels innermost) with the input
    zero point written into the padding."""
    b, H, W, C = X.shape
    sh, sw = stride
    ph, pw = pad
    Ho = (H + 2 * ph - KH) // sh + 1
    Wo = (W + 2 * pw - KW) // sw + 1
    Xp = np.full((b, H + 2 * ph, W + 2 * pw, C), za, np.int8)
    Xp[:, ph:ph + H, pw:pw + W, :] = X
    rows = np.zeros((b, Ho, Wo, KH, KW, C), np.int8)
    for kh in range(KH):
        for kw in range(KW):
            rows[:, :, :, kh, kw, :] = Xp[:, kh:kh + sh * Ho:sh, kw:kw + sw * Wo:sw, :]
    return rows.reshape(b * Ho * Wo, KH * KW * C), (b, Ho, Wo)


@pytest.mark.parametrize("geom", [
    (1, 6, 7, 8, 5, 3, 3, (1, 1), (1, 1)),
    (2, 9, 8, 16, 4, 3, 3, (2, 2), (1, 1)),
    (1, 5, 5, 3, 2, 5, 5, (1, 1), (2, 2)),
    (1, 7, 6, 4, 3, 1, 3, (2, 1), (0, 1)),
])
@pytest.mark.parametrize("za,zb", [(0, 0), (-128, 0), (45, -9), (127, 127)])
def test_conv_zp_equals_im2col_gemm(orc, geom, za, zb):
    b, H, W, C_in, C_out, KH, KW, stride, pad = geom
    g = np.random.default_rng(H * W + C_in)
    X = _i8(g, (b, H, W, C_in))
    Wt = _i8(g, (C_out, KH, KW, C_in))
    cols, (bb, Ho, Wo) = _im2col_zp(X, KH, KW, stride, pad, za)
    want = orc.gemm_s8s8_acc_zp(cols, Wt.reshape(C_out, -1), za, zb)
    got = orc.conv2d_acc_zp(X, Wt, za, zb, stride=stride, pad=pad)
    assert np.array_equal(got.reshape(-1, C_out), want)


def test_conv_zp_padding_is_the_zero_point(orc):
    """Every input at za + 1 with weights zb + w: each tap inside the image
    adds C * w, a padded tap adds nothing -- 9 / 6 / 4 taps at interior /
    edge / corner for 3x3 s1 p1.  Padding with 0 instead would add
    (0 - za) * w per padded input."""
    za, zb, w, C = -20, 3, 2, 5
    X = np.full((1, 5, 6, C), za + 1, np.int8)
    Wt = np.full((4, 3, 3, C), zb + w, np.int8)
    acc = orc.conv2d_acc_zp(X, Wt, za, zb)
    taps = np.full((5, 6), 9)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    assert np.array_equal(acc[0, :, :, 0], taps * C * w)
    # an input that sits at its zero point everywhere is all real zeros
    Xz = np.full((1, 5, 6, C), za, np.int8)
    assert np.all(orc.conv2d_acc_zp(Xz, Wt, za, zb) == 0)


def test_conv_zp_reduces_and_composes(orc):
    d = datagen.conv_nhwc(2, 7, 6, 16, 8, 3, 3, seed=4, shift=(34, 40))
    assert np.array_equal(orc.conv2d_acc_zp(d["X"], d["W"], 0, 0), orc.conv2d_acc(d["X"], d["W"]))
    za, zb, zo = 9, -2, -50
    acc = orc.conv2d_acc_zp(d["X"], d["W"], za, zb).reshape(-1, 8)
    Y = orc.conv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                      za, zb, zo).reshape(-1, 8)
    for p in (0, 13, 41, acc.shape[0] - 1):
        for n in range(8):
            assert Y[p, n] == orc.requant_zp(int(acc[p, n]), int(d["bias"][n]),
                                             int(d["mult"][n]), int(d["shift"][n]), zo)
    pix = np.array([3, 50, 83])
    assert np.array_equal(orc.conv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"],
                                                        d["shift"], za, zb, zo, pix=pix), Y[pix])
    act = orc.conv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"], za, zb,
                                        zo, act=(-40, 60)).reshape(-1, 8)
    assert np.array_equal(act, np.clip(Y, -40, 60))


def test_conv_zp_shift_invariance(orc):
    g = np.random.default_rng(5)
    X = _i8(g, (1, 6, 5, 4), -100, 100)
    Wt = _i8(g, (3, 3, 3, 4), -100, 100)
    base = orc.conv2d_acc_zp(X, Wt, 7, -3)
    assert np.array_equal(orc.conv2d_acc_zp((X + 20).astype(np.int8), Wt, 27, -3), base)
    assert np.array_equal(orc.conv2d_acc_zp(X, (Wt - 9).astype(np.int8), 7, -12), base)


# ---------------------------------------------------------------- depthwise

def _block_diagonal(Wt):
    KH, KW, C = Wt.shape
    full = np.zeros((C, KH, KW, C), dtype=np.int8)
    for c in range(C):
        full[c, :, :, c] = Wt[:, :, c]
    return full


@pytest.mark.parametrize("za", [0, -128, 33, 127])
def test_dwconv_zp_equals_full_conv_block_diagonal(orc, za):
    """With symmetric weights (zb 0) the zero weights off the diagonal stay
    real zeros, so the full asymmetric conv with block-diagonal weights is the
    depthwise conv."""
    g = np.random.default_rng(200 + za)
    X = _i8(g, (2, 7, 6, 8))
    Wt = _i8(g, (3, 3, 8))
    for stride, pad in (((1, 1), (1, 1)), ((2, 2), (1, 1)), ((1, 2), (2, 0))):
        dw = orc.dwconv2d_acc_zp(X, Wt, za, 0, stride=stride, pad=pad)
        full = orc.conv2d_acc_zp(X, _block_diagonal(Wt), za, 0, stride=stride, pad=pad)
        assert np.array_equal(dw, full)


def test_dwconv_zp_closed_form_and_shift(orc):
    za, zb, w = 40, -6, -3
    X = np.full((1, 4, 5, 16), za + 1, np.int8)
    Wt = np.full((3, 3, 16), zb + w, np.int8)
    acc = orc.dwconv2d_acc_zp(X, Wt, za, zb)
    taps = np.full((4, 5), 9)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    assert np.array_equal(acc[0, :, :, 5], taps * w)
    g = np.random.default_rng(7)
    X = _i8(g, (1, 6, 6, 16), -100, 100)
    Wt = _i8(g, (3, 3, 16), -100, 100)
    base = orc.dwconv2d_acc_zp(X, Wt, 5, 8)
    assert np.array_equal(orc.dwconv2d_acc_zp(X, (Wt + 19).astype(np.int8), 5, 27), base)
    assert np.array_equal(orc.dwconv2d_acc_zp((X - 15).astype(np.int8), Wt, -10, 8), base)
    assert np.array_equal(orc.dwconv2d_acc_zp(X, Wt, 0, 0), orc.dwconv2d_acc(X, Wt))


def test_dwconv_zp_requant_composition(orc):
    d = datagen.dwconv_nhwc(1, 6, 7, 16, 3, 3, seed=8, shift=(30, 36))
    za, zb, zo = -7, 4, 12
    acc = orc.dwconv2d_acc_zp(d["X"], d["W"], za, zb).reshape(-1, 16)
    Y = orc.dwconv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                        za, zb, zo).reshape(-1, 16)
    for p in (0, 20, acc.shape[0] - 1):
        for c in range(16):
            assert Y[p, c] == orc.requant_zp(int(acc[p, c]), int(d["bias"][c]),
                                             int(d["mult"][c]), int(d["shift"][c]), zo)
    relu = orc.dwconv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                           za, zb, zo, act=(zo, 127)).reshape(-1, 16)
    assert np.array_equal(relu, np.maximum(Y, zo))


# ---------------------------------------------------------------- MSB-first INT4

def test_msb_first_page_packing_rule(orc):
    """The INT4 GEMM article's §4.1 conversion packs a pair as
    (first << 4) | second, each as a 4-bit two's complement nibble."""
    vals = [3, -2, 7, -8, 0, -1, -7, 5]
    packed = np.array([((vals[i] & 0xF) << 4) | (vals[i + 1] & 0xF)
                       for i in range(0, len(vals), 2)], np.uint8)
    assert packed.tolist() == [0x3E, 0x78, 0x0F, 0x95]
    assert [orc.int4_at_msb(packed, i) for i in range(len(vals))] == vals
    # the same bytes read low nibble first give each pair swapped
    assert [orc.int4_at(packed, i) for i in range(len(vals))] == [-2, 3, -8, 7, -1, 0, 5, -7]


def _swap_nibbles(p):
    return ((p << 4) | (p >> 4)).astype(np.uint8)


def test_msb_first_is_the_nibble_swap(orc):
    every = np.arange(256, dtype=np.uint8)
    sw = _swap_nibbles(every)
    for i in range(2):
        assert [orc.int4_at_msb(every[j:j + 1], i) for j in range(256)] == \
            [orc.int4_at(sw[j:j + 1], i) for j in range(256)]
    g = np.random.default_rng(9)
    A = datagen.int4_packed_uniform(g, 13, 96)
    B = datagen.int4_packed_uniform(g, 11, 96)
    assert np.array_equal(orc.gemm_s4s4_i32(_swap_nibbles(A), _swap_nibbles(B), msb_first=True),
                          orc.gemm_s4s4_i32(A, B))
    w = datagen.gemm_w4a8(9, 11, 96, seed=10, shift=(39, 43))  # mostly unsaturated
    assert np.array_equal(
        orc.gemm_w4a8_requant(w["A"], _swap_nibbles(w["B"]), w["bias"], w["mult"], w["shift"],
                              msb_first=True),
        orc.gemm_w4a8_requant(w["A"], w["B"], w["bias"], w["mult"], w["shift"]))
    # with both operands in the same order, reading every byte the other way
    # swaps the two products of each pair alike, so the int4 x int4 sum does
    # not change; against unpermuted int8 activations the order matters
    assert np.array_equal(orc.gemm_s4s4_i32(A, B, msb_first=True), orc.gemm_s4s4_i32(A, B))
    assert not np.array_equal(
        orc.gemm_w4a8_requant(w["A"], w["B"], w["bias"], w["mult"], w["shift"],
                              msb_first=True),
        orc.gemm_w4a8_requant(w["A"], w["B"], w["bias"], w["mult"], w["shift"]))

"""Pins of the oracle's NHWC conv: the MCU conv front-end page's
(news.rkmt.cn/news/16638) closed-form geometry and MAC counts (§2.1), the
all-ones padding closed form (zero-point padding, §2.3), and three
formulations that must agree: direct conv, explicit im2col followed by a
GEMM (§3.2), and a sum of shifted 1x1 convs (Groq TSP ResNet50 page,
www.pwwt.cn/news/1982903, §2.1)."""
import numpy as np
import pytest

from conv_qgemm_amd import datagen


def test_first_layer_geometry_and_macs(orc):
    # 40x32x1 input, 3x3 kernel, stride 2, padding 1 -> 20x16, 16 channels
    assert orc.conv_out_size(40, 3, 2, 1) == 20
    assert orc.conv_out_size(32, 3, 2, 1) == 16
    assert orc.conv_macs(1, 40, 32, 1, 16, 3, 3, 2, 2, 1, 1) == 46080


def test_pointwise_macs(orc):
    # 20x16x64 -> 64 pointwise conv: 20*16*64*64 = 1,310,720 (the page rounds to 1.3M)
    assert orc.conv_macs(1, 20, 16, 64, 64, 1, 1, 1, 1, 0, 0) == 1310720


def test_resnet_style_layer_macs(orc):
    # batch 32, 56x56, 64 -> 64, 3x3 s1 p1
    assert orc.conv_out_size(56, 3, 1, 1) == 56
    assert orc.conv_macs(32, 56, 56, 64, 64, 3, 3, 1, 1, 1, 1) == 3699376128


def test_all_ones_padding_closed_form(orc):
    C = 16
    X = np.ones((1, 6, 5, C), np.int8)
    W = np.ones((2, 3, 3, C), np.int8)
    acc = orc.conv2d_acc(X, W, stride=(1, 1), pad=(1, 1))[0, :, :, 0]
    H, Wd = 6, 5
    for h in range(H):
        for w in range(Wd):
            rows = 3 - (h == 0) - (h == H - 1)
            cols = 3 - (w == 0) - (w == Wd - 1)
            assert acc[h, w] == rows * cols * C
    assert acc[2, 2] == 9 * C and acc[0, 2] == 6 * C and acc[0, 0] == 4 * C


def _im2col_gemm(X, W, stride, pad):
    """Explicit im2col + numpy matmul: A[pixel][(kh*KW + kw)*C_in + ci]."""
    B, H, Wd, C = X.shape
    O, KH, KW, _ = W.shape
    sh, sw = stride
    ph, pw = pad
    Xp = np.pad(X.astype(np.int64), ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    Ho = (H + 2 * ph - KH) // sh + 1
    Wo = (Wd + 2 * pw - KW) // sw + 1
    cols = np.empty((B, Ho, Wo, KH, KW, C), np.int64)
    for kh in range(KH):
        for kw in range(KW):
            cols[:, :, :, kh, kw, :] = Xp[:, kh:kh + sh * (Ho - 1) + 1:sh,
                                          kw:kw + sw * (Wo - 1) + 1:sw, :]
    A = cols.reshape(B * Ho * Wo, KH * KW * C)
    Wm = W.astype(np.int64).reshape(O, KH * KW * C)
    return (A @ Wm.T).reshape(B, Ho, Wo, O)


def _shifted_1x1_sum(X, W, stride, pad):
    """Sum over taps of 1x1 convs of the shifted (zero-padded) input."""
    B, H, Wd, C = X.shape
    O, KH, KW, _ = W.shape
    sh, sw = stride
    ph, pw = pad
    Ho = (H + 2 * ph - KH) // sh + 1
    Wo = (Wd + 2 * pw - KW) // sw + 1
    out = np.zeros((B, Ho, Wo, O), np.int64)
    Xl = X.astype(np.int64)
    for kh in range(KH):
        for kw in range(KW):
            shifted = np.zeros((B, Ho, Wo, C), np.int64)
            for oh in range(Ho):
                ih = oh * sh - ph + kh
                if not 0 <= ih < H:
                    continue
                for ow in range(Wo):
                    iw = ow * sw - pw + kw
                    if 0 <= iw < Wd:
                        shifted[:, oh, ow, :] = Xl[:, ih, iw, :]
            out += shifted @ W[:, kh, kw, :].astype(np.int64).T
    return out


GEOMS = [
    # batch, H, W, C_in, C_out, KH, KW, stride, pad
    (1, 7, 6, 16, 16, 3, 3, (1, 1), (1, 1)),
    (2, 9, 8, 16, 32, 3, 3, (2, 2), (1, 1)),
    (1, 10, 7, 32, 16, 3, 3, (1, 1), (0, 0)),
    (1, 8, 8, 16, 16, 5, 5, (1, 1), (2, 2)),
    (2, 6, 11, 16, 16, 1, 3, (1, 2), (0, 1)),
    (1, 5, 5, 16, 16, 3, 3, (2, 1), (2, 0)),
]


@pytest.mark.parametrize("geom", GEOMS)
def test_three_formulations_agree(orc, geom):
    b, H, Wd, Ci, Co, KH, KW, stride, pad = geom
    g = np.random.default_rng(H * 31 + Wd)
    X = g.integers(-128, 128, size=(b, H, Wd, Ci), dtype=np.int8)
    W = g.integers(-128, 128, size=(Co, KH, KW, Ci), dtype=np.int8)
    direct = orc.conv2d_acc(X, W, stride=stride, pad=pad)
    assert np.array_equal(direct, _im2col_gemm(X, W, stride, pad))
    assert np.array_equal(direct, _shifted_1x1_sum(X, W, stride, pad))


def test_pointwise_conv_is_gemm(orc):
    d = datagen.workload("pointwise")
    A, B = d["A"], d["B"]  # A: 320 pixels x 64 channels, B: 64 out x 64 in
    X = A.reshape(1, 20, 16, 64)
    W = B.reshape(64, 1, 1, 64)
    y_conv = orc.conv2d_nhwc_s8_requant(X, W, d["bias"], d["mult"], d["shift"],
                                        stride=(1, 1), pad=(0, 0))
    y_gemm = orc.gemm_s8s8_requant(A, B, d["bias"], d["mult"], d["shift"])
    assert np.array_equal(y_conv.reshape(320, 64), y_gemm)


def test_conv_requant_composition_and_pixels(orc):
    d = datagen.conv_nhwc(2, 6, 7, 16, 16, 3, 3, seed=11, shift=(36, 42))
    acc = orc.conv2d_acc(d["X"], d["W"]).reshape(-1, 16)
    want = np.empty(acc.shape, np.int8)
    for p in range(acc.shape[0]):
        for c in range(16):
            want[p, c] = orc.requant(int(acc[p, c]), int(d["bias"][c]), int(d["mult"][c]),
                                     int(d["shift"][c]))
    got = orc.conv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(got.reshape(-1, 16), want)
    pix = [83, 0, 41, 41]
    part = orc.conv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"], pix=pix)
    assert np.array_equal(part, want[pix])

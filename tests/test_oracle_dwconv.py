"""Pins of the oracle's depthwise NHWC conv (MCU conv front-end article,
news.rkmt.cn/news/16638, §3.3: one input channel per output channel, weights
[kh][kw][c]; zero-point padding §2.3; MAC count §2.1).

Each pin reaches the result by a route other than the oracle's own loop: a
closed form, the full-conv oracle with block-diagonal weights, or an
invariant the definition implies.
"""
import numpy as np
import pytest

from conv_qgemm_amd import datagen

GEOMS = [
    # batch, H, W, C, KH, KW, stride, pad
    (1, 5, 6, 3, 3, 3, (1, 1), (1, 1)),
    (2, 9, 8, 16, 3, 3, (2, 2), (1, 1)),
    (1, 10, 7, 5, 3, 3, (1, 1), (0, 0)),
    (1, 8, 8, 4, 5, 5, (1, 1), (2, 2)),
    (2, 6, 11, 6, 1, 3, (1, 2), (0, 1)),
    (1, 5, 5, 2, 3, 3, (2, 1), (2, 0)),
    (1, 20, 16, 16, 3, 3, (1, 1), (1, 1)),  # the MCU front-end's 20x16x16 map
]


def _data(g, b, H, W, C, KH, KW):
    X = g.integers(-128, 128, size=(b, H, W, C), dtype=np.int8)
    Wt = g.integers(-128, 128, size=(KH, KW, C), dtype=np.int8)
    return X, Wt


def _block_diagonal(Wt):
    """OHWI weights of a full conv that does what the depthwise conv does:
    output channel c sees only input channel c."""
    KH, KW, C = Wt.shape
    full = np.zeros((C, KH, KW, C), dtype=np.int8)
    for c in range(C):
        full[c, :, :, c] = Wt[:, :, c]
    return full


def test_all_ones_closed_form(orc):
    """3x3 s1 p1 on all-a input with all-w weights: a*w times the number of
    taps inside the image -- 9 inside, 6 on an edge, 4 in a corner."""
    a, w = 3, -5
    X = np.full((2, 6, 7, 8), a, np.int8)
    Wt = np.full((3, 3, 8), w, np.int8)
    acc = orc.dwconv2d_acc(X, Wt, stride=(1, 1), pad=(1, 1))
    taps = np.full((6, 7), 9)
    taps[0, :] = taps[-1, :] = 6
    taps[:, 0] = taps[:, -1] = 6
    taps[0, 0] = taps[0, -1] = taps[-1, 0] = taps[-1, -1] = 4
    want = a * w * taps
    assert np.array_equal(acc, np.broadcast_to(want[None, :, :, None], acc.shape))


def test_pointwise_closed_form(orc):
    """A 1x1 depthwise conv scales each channel by its weight."""
    g = np.random.default_rng(1)
    X, Wt = _data(g, 2, 4, 5, 7, 1, 1)
    acc = orc.dwconv2d_acc(X, Wt, stride=(1, 1), pad=(0, 0))
    assert np.array_equal(acc, X.astype(np.int64) * Wt[0, 0].astype(np.int64))


@pytest.mark.parametrize("geom", GEOMS)
def test_equals_full_conv_with_block_diagonal_weights(orc, geom):
    b, H, W, C, KH, KW, stride, pad = geom
    g = np.random.default_rng(H * W + C)
    X, Wt = _data(g, b, H, W, C, KH, KW)
    dw = orc.dwconv2d_acc(X, Wt, stride=stride, pad=pad)
    full = orc.conv2d_acc(X, _block_diagonal(Wt), stride=stride, pad=pad)
    assert np.array_equal(dw, full)


def test_requant_composition_matches_full_conv(orc):
    b, H, W, C = 2, 9, 10, 16
    d = datagen.conv_nhwc(b, H, W, C, C, 3, 3, seed=5, shift=(36, 42))
    g = np.random.default_rng(6)
    Wt = g.integers(-128, 128, size=(3, 3, C), dtype=np.int8)
    Y = orc.dwconv2d_nhwc_s8_requant(d["X"], Wt, d["bias"], d["mult"], d["shift"],
                                     stride=(1, 1), pad=(1, 1))
    want = orc.conv2d_nhwc_s8_requant(d["X"], _block_diagonal(Wt), d["bias"], d["mult"],
                                      d["shift"], stride=(1, 1), pad=(1, 1))
    assert np.array_equal(Y, want)
    pix = np.array([0, 5, 77, b * H * W - 1])
    assert np.array_equal(orc.dwconv2d_nhwc_s8_requant(d["X"], Wt, d["bias"], d["mult"],
                                                       d["shift"], pix=pix),
                          Y.reshape(-1, C)[pix])


def test_channels_are_independent(orc):
    """Changing channel c of the input or the weights changes only output
    channel c; permuting channels permutes the outputs."""
    g = np.random.default_rng(2)
    X, Wt = _data(g, 1, 7, 6, 9, 3, 3)
    base = orc.dwconv2d_acc(X, Wt, stride=(2, 1), pad=(1, 1))
    X2, W2 = X.copy(), Wt.copy()
    X2[..., 4] = g.integers(-128, 128, size=X2[..., 4].shape, dtype=np.int8)
    W2[..., 4] = -W2[..., 4] // 2
    moved = orc.dwconv2d_acc(X2, W2, stride=(2, 1), pad=(1, 1))
    others = [c for c in range(9) if c != 4]
    assert np.array_equal(moved[..., others], base[..., others])
    assert not np.array_equal(moved[..., 4], base[..., 4])
    perm = g.permutation(9)
    permuted = orc.dwconv2d_acc(X[..., perm], Wt[..., perm], stride=(2, 1), pad=(1, 1))
    assert np.array_equal(permuted, base[..., perm])


def test_macs(orc):
    # one input channel per output channel in the page's MAC formula
    assert orc.dwconv_macs(1, 20, 16, 16, 3, 3, 1, 1, 1, 1) == 20 * 16 * 16 * 3 * 3
    assert orc.dwconv_macs(32, 56, 56, 64, 3, 3, 1, 1, 1, 1) == 32 * 56 * 56 * 64 * 9
    # stride 2 halves both output sides
    assert orc.dwconv_macs(1, 112, 112, 32, 3, 3, 2, 2, 1, 1) == 56 * 56 * 32 * 9
    # equals the full conv's count divided by C_in for the block-diagonal form
    assert orc.dwconv_macs(2, 9, 8, 16, 3, 3, 2, 2, 1, 1) * 16 == \
        orc.conv_macs(2, 9, 8, 16, 16, 3, 3, 2, 2, 1, 1)

"""Exact half-LSB ties through every requantize route of every kernel.

The requantize (MCU conv front-end article, news.rkmt.cn/news/16638, §2.3)
adds half an LSB, 2^(shift-1), before the arithmetic shift, so a product
x * M that sits exactly halfway between two output steps rounds up (toward
+infinity).  Random operands almost never land there: at shift s a tie has
probability about 2^-s per element.  These tests build inputs whose every
accumulator is a chosen value, put most of them on a tie or one step beside
it, and compare the GPU result with the oracle (and, for the hand-worked
table in tests/golden/requant_hand_table.txt, with the page-derived values
directly).

How a tie is placed.  With M = 2^p * q (q odd) and d = s - p >= 1,
x * M / 2^s = x * q / 2^d, which is an exact half exactly when
x = 2^(d-1) * (2j + 1).  Each output column n gets such a multiplier and a
bias T_n on one of its ties; one-hot operands make the accumulator of row
(or pixel) m equal a_m * w_n, with a_m in {0, +-1, +-2, ...}, so the rows
see x = T_n, T_n +- 1, ... .

Every kernel picks one of three exact requantize routes per tile or wave
from the shifts of its columns (a general 64-bit route, one for shifts >= 31
and one for shifts >= 33).  Each test therefore runs three times: with
shifts in [31, 32], with shifts in [33, 63], and with every column free in
[1, 63] but at least one shift below 31 in every 8 columns (which forces the
general route onto the high shifts too).
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TIERS = ["general", "s31", "s33"]


@pytest.fixture(scope="module")
def qg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conv_qgemm_amd import qgemm
    return qgemm


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- tie design

def _shifts(n, tier, g):
    if tier == "s31":
        return g.integers(31, 32, size=n, endpoint=True)
    if tier == "s33":
        return g.integers(33, 63, size=n, endpoint=True)
    s = g.integers(1, 63, size=n, endpoint=True)
    s[::8] = g.integers(1, 30, size=len(s[::8]), endpoint=True)
    return s


def tie_columns(n, tier, seed, wmax=3):
    """Per-column (bias, mult, shift, w): bias on a tie of (mult, shift) for
    every column whose shift allows one inside int32 (shift <= 61), a large
    bias toward either saturation end for the others; w is the column's
    weight (the per-row offset a_m is multiplied by it)."""
    g = np.random.default_rng(seed)
    sh = _shifts(n, tier, g)
    bias = np.zeros(n, np.int64)
    mult = np.zeros(n, np.int64)
    w = g.choice([1, -1, 1, -1, 2, -2, wmax], size=n).astype(np.int64)
    margin = 1 << 15  # room for the row offsets a_m * w_n
    for i, s in enumerate(sh):
        s = int(s)
        # p = s - d with 1 <= d <= 31 and 0 <= p <= 30
        plo, phi = max(0, s - 31), min(30, s - 1)
        if plo > phi:  # no tie reachable inside int32: saturation / extremes
            mult[i] = int(g.integers(1 << 30, 1 << 31))
            bias[i] = int(g.choice([(1 << 31) - 1 - margin, -(1 << 31) + margin, 0]))
            continue
        p = int(g.integers(plo, phi, endpoint=True))
        d = s - p
        qmax = min((1 << (31 - p)) - 1, 255)
        if i % 2:  # half the columns keep q / 2^d < 1, so a_m = +-1 stays near the tie
            qmax = min(qmax, max(1, (1 << d) - 1))
        q = int(g.integers(0, (qmax - 1) // 2, endpoint=True)) * 2 + 1
        mult[i] = (1 << p) * q
        # odd factors o = 2j + 1 with x = 2^(d-1) * o inside int32 (with the
        # margin) and |o * q| <= 260: outputs around, and just past, the
        # int8 range (ties at +-127.5 and +-128.5 included)
        omax = min(((1 << 31) - 1 - margin) >> (d - 1), max(1, 260 // q))
        if omax < 1:
            mult[i] = int(g.integers(1 << 30, 1 << 31))
            bias[i] = 0
            continue
        o = int(g.integers(-omax, omax, endpoint=True))
        if o % 2 == 0:
            o += 1 if o < omax else -1
        bias[i] = (1 << (d - 1)) * o
    assert np.all(np.abs(bias) < (1 << 31))
    return bias.astype(np.int32), mult.astype(np.int32), sh.astype(np.int32), w


def row_offsets(m, seed, amax=127):
    """a_m: 0, 1, -1, 2, -2 repeated on most rows (the tie and its two
    neighbours), random int8 values on every fourth row."""
    g = np.random.default_rng(seed + 1)
    a = np.resize(np.array([0, 1, -1, 0, 2, -2, 0, 1, -1]), m).astype(np.int64)
    r = g.integers(-amax, amax, size=m, endpoint=True)
    a[3::4] = r[3::4]
    return a


def count_ties(x, mult, shift):
    """Elements whose x * M is exactly halfway between two output steps."""
    x = x.astype(np.int64)
    t = x * mult.astype(np.int64)[None, :]
    s = shift.astype(np.int64)[None, :]
    ok = s <= 62
    mod = np.where(ok, np.int64(1) << np.minimum(s, 62), 1)
    half = np.where(ok, np.int64(1) << np.minimum(s - 1, 61), 0)
    return int(np.sum(ok & (np.mod(t, mod) == half)))


def _check_cover(x, mult, shift, y):
    ties = count_ties(x, mult, shift)
    assert ties >= x.shape[1], f"only {ties} ties placed"
    inside = np.sum((y > -128) & (y < 127))
    assert inside >= x.size // 8, "too few outputs inside the int8 range"
    return ties


# ---------------------------------------------------------------- GEMMs

def one_hot_s8(M, K, a):
    A = np.zeros((M, K), np.int8)
    A[np.arange(M), np.arange(M) % K] = a
    return A


def s8_weights(N, K, w):
    return np.repeat(w.astype(np.int8)[:, None], K, axis=1)


def s4_weights(N, K, w):
    nib = (w.astype(np.int64) & 0xF).astype(np.uint8)
    byte = nib | (nib << 4)
    return np.repeat(byte[:, None], K // 2, axis=1)


GEMM_S8 = {"ring": (2048, 4096, 256), "tile": (300, 260, 64)}


@pytest.mark.parametrize("tier", TIERS)
@pytest.mark.parametrize("kernel", list(GEMM_S8))
def test_ties_s8s8(qg, kernel, tier):
    M, N, K = GEMM_S8[kernel]
    _say("ties s8s8", kernel, tier, M, N, K)
    bias, mult, shift, w = tie_columns(N, tier, seed=N + len(tier))
    a = row_offsets(M, seed=M)
    A, B = one_hot_s8(M, K, a), s8_weights(N, K, w)
    C = host(qg.qgemm_s8s8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift)))
    want = oracle.gemm_s8s8_requant(A, B, bias, mult, shift)
    x = oracle.gemm_acc(A, B) + bias.astype(np.int64)[None, :]
    _check_cover(x, mult, shift, want)
    assert np.array_equal(C, want)


GEMM_W4 = {"ring": (2048, 4096, 384), "tile": (100, 260, 64), "skinny": (16, 1024, 1024),
           "skinny_blocks": (40, 520, 4096)}


@pytest.mark.parametrize("tier", TIERS)
@pytest.mark.parametrize("kernel", list(GEMM_W4))
def test_ties_w4a8(qg, kernel, tier):
    M, N, K = GEMM_W4[kernel]
    _say("ties w4a8", kernel, tier, M, N, K)
    bias, mult, shift, w = tie_columns(N, tier, seed=3 * N + len(tier), wmax=7)
    a = row_offsets(M, seed=M + 1)
    A, B = one_hot_s8(M, K, a), s4_weights(N, K, w)
    C = host(qg.qgemm_w4a8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift)))
    want = oracle.gemm_w4a8_requant(A, B, bias, mult, shift)
    x = oracle.gemm_acc(A, B) + bias.astype(np.int64)[None, :]
    _check_cover(x, mult, shift, want)
    assert np.array_equal(C, want)


@pytest.mark.parametrize("tier", TIERS)
@pytest.mark.parametrize("kernel", list(GEMM_S8))
@pytest.mark.parametrize("zo,act", [(7, (-128, 127)), (-20, (-20, 100))])
def test_ties_s8s8_zp(qg, kernel, tier, zo, act):
    """The asymmetric epilogue: the output zero point is added after the
    rounding, then the (activation) clamp.  Zero input and weight points
    keep the accumulator at a_m * w_n."""
    M, N, K = GEMM_S8[kernel]
    _say("ties s8s8 zp", kernel, tier, zo, act)
    bias, mult, shift, w = tie_columns(N, tier, seed=5 * N + len(tier))
    a = row_offsets(M, seed=M + 2)
    A, B = one_hot_s8(M, K, a), s8_weights(N, K, w)
    C = host(qg.qgemm_s8s8_requant_zp(dev(A), dev(B), dev(bias), dev(mult), dev(shift), 0, 0, zo,
                                      act=act))
    want = oracle.gemm_s8s8_requant_zp(A, B, bias, mult, shift, 0, 0, zo, act=act)
    x = oracle.gemm_acc(A, B) + bias.astype(np.int64)[None, :]
    assert count_ties(x, mult, shift) >= N
    assert np.array_equal(C, want)


# ---------------------------------------------------------------- convs

CONVS = {
    # batch, H, W, C_in, C_out, stride: the LDS-staged band kernel (stride 1,
    # 64 input channels) and the implicit-im2col tile kernel (32 channels)
    "halo": (2, 14, 15, 64, 192, 1),
    "tile": (2, 13, 11, 32, 64, 1),
    "tile_s2": (1, 21, 19, 64, 128, 2),
}


def conv_operands(b, H, Wd, Ci, Co, w, seed):
    """X holds a_p in channel 0 of each pixel (zeros elsewhere); W has only
    the centre tap of channel 0, w_oc: the accumulator of output pixel p is
    a_p' * w_oc, where p' is the input pixel under the centre tap."""
    a = row_offsets(b * H * Wd, seed)
    X = np.zeros((b, H, Wd, Ci), np.int8)
    X[..., 0] = a.reshape(b, H, Wd)
    Wt = np.zeros((Co, 3, 3, Ci), np.int8)
    Wt[:, 1, 1, 0] = w
    return X, Wt


@pytest.mark.parametrize("tier", TIERS)
@pytest.mark.parametrize("kernel", list(CONVS))
def test_ties_conv(qg, kernel, tier):
    b, H, Wd, Ci, Co, st = CONVS[kernel]
    _say("ties conv", kernel, tier)
    bias, mult, shift, w = tie_columns(Co, tier, seed=7 * Co + len(tier) + st)
    X, Wt = conv_operands(b, H, Wd, Ci, Co, w, seed=H * Wd)
    Y = host(qg.qconv2d_nhwc_s8_requant(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift),
                                        stride=(st, st), pad=(1, 1)))
    want = oracle.conv2d_nhwc_s8_requant(X, Wt, bias, mult, shift, stride=(st, st), pad=(1, 1))
    acc = oracle.conv2d_acc(X, Wt, stride=(st, st), pad=(1, 1)).reshape(-1, Co)
    _check_cover(acc + bias.astype(np.int64)[None, :], mult, shift, want.reshape(-1, Co))
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("tier", TIERS)
@pytest.mark.parametrize("kernel", ["halo", "tile"])
def test_ties_conv_zp(qg, kernel, tier):
    b, H, Wd, Ci, Co, st = CONVS[kernel]
    _say("ties conv zp", kernel, tier)
    bias, mult, shift, w = tie_columns(Co, tier, seed=11 * Co + len(tier))
    X, Wt = conv_operands(b, H, Wd, Ci, Co, w, seed=H * Wd + 3)
    Y = host(qg.qconv2d_nhwc_s8_requant_zp(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift),
                                           0, 0, -9, stride=(st, st), pad=(1, 1),
                                           act=(-9, 127)))
    want = oracle.conv2d_nhwc_s8_requant_zp(X, Wt, bias, mult, shift, 0, 0, -9, stride=(st, st),
                                            pad=(1, 1), act=(-9, 127))
    acc = oracle.conv2d_acc(X, Wt, stride=(st, st), pad=(1, 1)).reshape(-1, Co)
    assert count_ties(acc + bias.astype(np.int64)[None, :], mult, shift) >= Co
    assert np.array_equal(Y, want)


DWCONVS = {
    # batch, H, W, C, KH (3: the matrix-core kernel, 5: the direct kernel)
    "mfma": (2, 14, 15, 128, 3),
    "direct": (1, 9, 10, 64, 5),
}


@pytest.mark.parametrize("tier", TIERS)
@pytest.mark.parametrize("kernel", list(DWCONVS))
@pytest.mark.parametrize("zp", [False, True])
def test_ties_dwconv(qg, kernel, tier, zp):
    b, H, Wd, C, KH = DWCONVS[kernel]
    _say("ties dwconv", kernel, tier, zp)
    bias, mult, shift, w = tie_columns(C, tier, seed=13 * C + len(tier) + KH)
    a = row_offsets(b * H * Wd, seed=H * Wd + 5)
    X = np.repeat(a.astype(np.int8).reshape(b, H, Wd, 1), C, axis=3)
    Wt = np.zeros((KH, KH, C), np.int8)
    Wt[KH // 2, KH // 2, :] = w
    pad = (KH // 2, KH // 2)
    if zp:
        Y = qg.qdwconv2d_nhwc_s8_requant_zp(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift),
                                            0, 0, 13, pad=pad)
        want = oracle.dwconv2d_nhwc_s8_requant_zp(X, Wt, bias, mult, shift, 0, 0, 13, pad=pad)
    else:
        Y = qg.qdwconv2d_nhwc_s8_requant(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift),
                                         pad=pad)
        want = oracle.dwconv2d_nhwc_s8_requant(X, Wt, bias, mult, shift, pad=pad)
    acc = oracle.dwconv2d_acc(X, Wt, pad=pad).reshape(-1, C)
    x = acc + bias.astype(np.int64)[None, :]
    if not zp:
        _check_cover(x, mult, shift, want.reshape(-1, C))
    assert count_ties(x, mult, shift) >= C
    assert np.array_equal(host(Y), want)


# ---------------------------------------------------------------- the hand table

def _golden_by_tier():
    rows = [tuple(int(v) for v in r) for r in read_golden("requant_hand_table.txt")]
    groups = {"general": [], "s31": [], "s33": []}
    for acc, b, m, s, y in rows:
        groups["general"].append((acc + b, m, s, y))
        if s in (31, 32):
            groups["s31"].append((acc + b, m, s, y))
        elif s >= 33:
            groups["s33"].append((acc + b, m, s, y))
    return groups


def _golden_columns(entries, N):
    """Entry i of the table in columns i, i + len, i + 2 len, ... (its x as
    the column's bias, the accumulator 0); spare columns repeat entry 0."""
    x = np.array([e[0] for e in entries], np.int64)
    m = np.array([e[1] for e in entries], np.int64)
    s = np.array([e[2] for e in entries], np.int64)
    y = np.array([e[3] for e in entries], np.int64)
    idx = np.arange(N) % len(entries)
    return (x[idx].astype(np.int32), m[idx].astype(np.int32), s[idx].astype(np.int32),
            y[idx].astype(np.int8))


@pytest.mark.parametrize("tier", TIERS)
def test_hand_table_every_kernel(qg, tier):
    """Each worked value of tests/golden/requant_hand_table.txt (ties,
    saturation at both ends, halving, identity, extremes) as a whole output
    column of every kernel, grouped so that each requantize route sees the
    entries it takes: zero operands make the accumulator 0, the bias holds
    acc + bias of the table, and every row of the column must equal the
    table's value."""
    entries = _golden_by_tier()[tier]
    _say("hand table", tier, len(entries))

    def expect(got, y):
        assert np.array_equal(got, np.broadcast_to(y[None, :], got.shape))

    for kernel, (M, N, K) in GEMM_S8.items():
        bias, mult, shift, y = _golden_columns(entries, N)
        A, B = np.zeros((M, K), np.int8), np.ones((N, K), np.int8)
        expect(host(qg.qgemm_s8s8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift))), y)
        expect(host(qg.qgemm_s8s8_requant_zp(dev(A), dev(B), dev(bias), dev(mult), dev(shift),
                                             0, 0, 0)), y)
    for kernel, (M, N, K) in GEMM_W4.items():
        bias, mult, shift, y = _golden_columns(entries, N)
        A, B = np.zeros((M, K), np.int8), np.full((N, K // 2), 0x11, np.uint8)
        expect(host(qg.qgemm_w4a8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift))), y)
    for kernel, (b, H, Wd, Ci, Co, st) in CONVS.items():
        bias, mult, shift, y = _golden_columns(entries, Co)
        X, Wt = np.zeros((b, H, Wd, Ci), np.int8), np.ones((Co, 3, 3, Ci), np.int8)
        Y = host(qg.qconv2d_nhwc_s8_requant(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift),
                                            stride=(st, st), pad=(1, 1)))
        expect(Y.reshape(-1, Co), y)
    for kernel, (b, H, Wd, C, KH) in DWCONVS.items():
        bias, mult, shift, y = _golden_columns(entries, C)
        X, Wt = np.zeros((b, H, Wd, C), np.int8), np.ones((KH, KH, C), np.int8)
        Y = host(qg.qdwconv2d_nhwc_s8_requant(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift),
                                              pad=(KH // 2, KH // 2)))
        expect(Y.reshape(-1, C), y)

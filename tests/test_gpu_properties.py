"""Property-based shape tests: hypothesis draws GEMM sizes (M, N not
multiples of any tile, K at its minimum and with tails, odd sizes, row
strides wider than the rows, output strides that do and do not allow the
wide stores) and conv / depthwise geometries (kernel sizes, strides,
paddings, channel counts, images smaller than a kernel tile), and every
result is compared with the oracle bit for bit.  The same draws run the
asymmetric forms (every input, weight and output zero point, fused
activation bounds, the allocation-free GEMM on the same inputs), the
binary16-output INT4 GEMM (scales absent, on one side or both, of either
sign) and the per-token quantizer (every input type, both code widths,
clip ratios, all-zero tokens).  Derandomized: the same examples run every
time, so a failure names a reproducible case.

Definitions: C = A x B with INT32 sums (INT4 GEMM article,
www.cf-1.com/news/6060138, §3.2), its binary16 output (same article, §6)
and the per-token quantizer (same article, §4); the requantize, zero points
and the conv geometry of the MCU conv front-end article
(news.rkmt.cn/news/16638, §2.1, §2.3, §3.1, §3.3)."""
import numpy as np
import pytest

import oracle
from conv_qgemm_amd import datagen

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SETTINGS = settings(max_examples=100, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))


@pytest.fixture(scope="module")
def qg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conv_qgemm_amd import qgemm
    return qgemm


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def strided(a, extra_cols, fill):
    """a [rows][cols] placed in a wider device buffer; returns the view."""
    rows, cols = a.shape
    w = np.full((rows, cols + extra_cols), fill, dtype=a.dtype)
    w[:, :cols] = a
    return dev(w)[:, :cols]


def out_buffer(M, N, extra, dtype, fill):
    return torch.full((M, N + extra), fill, dtype=dtype, device="cuda")


gemm_dims = st.tuples(st.integers(1, 700), st.integers(1, 700))
shift_windows = st.sampled_from([(1, 20), (29, 40), (36, 44), (44, 60)])


@SETTINGS
@given(mn=gemm_dims, kq=st.integers(1, 24), lda_x=st.sampled_from([0, 16, 48]),
       ldb_x=st.sampled_from([0, 32]), ldc_x=st.sampled_from([0, 1, 3, 16]), win=shift_windows,
       bias=st.booleans(), seed=st.integers(0, 2 ** 16))
def test_prop_s8s8(qg, mn, kq, lda_x, ldb_x, ldc_x, win, bias, seed):
    (M, N), K = mn, 16 * kq
    d = datagen.gemm_s8s8(M, N, K, seed=seed, shift=win)
    b = d["bias"] if bias else None
    C = out_buffer(M, N, ldc_x, torch.int8, 55)
    qg.qgemm_s8s8_requant(strided(d["A"], lda_x, 0), strided(d["B"], ldb_x, 0),
                          None if b is None else dev(b), dev(d["mult"]), dev(d["shift"]),
                          C=C[:, :N])
    got = C.cpu().numpy()
    assert np.array_equal(got[:, :N], oracle.gemm_s8s8_requant(d["A"], d["B"], b, d["mult"],
                                                               d["shift"]))
    assert np.all(got[:, N:] == 55)


@SETTINGS
@given(mn=gemm_dims, kq=st.integers(1, 20), lda_x=st.sampled_from([0, 32]),
       ldc_x=st.sampled_from([0, 1, 4]), seed=st.integers(0, 2 ** 16))
def test_prop_s4s4(qg, mn, kq, lda_x, ldc_x, seed):
    (M, N), K = mn, 32 * kq
    d = datagen.gemm_s4s4(M, N, K, seed=seed)
    C = out_buffer(M, N, ldc_x, torch.int32, -3)
    qg.qgemm_s4s4_i32(strided(d["A"], lda_x // 2, 0), dev(d["B"]), C=C[:, :N], K=K)
    got = C.cpu().numpy()
    assert np.array_equal(got[:, :N], oracle.gemm_s4s4_i32(d["A"], d["B"]))
    assert np.all(got[:, N:] == -3)


@SETTINGS
@given(m=st.one_of(st.integers(1, 64), st.integers(65, 300)), n=st.integers(1, 700),
       kq=st.integers(1, 40), lda_x=st.sampled_from([0, 16]), ldc_x=st.sampled_from([0, 2, 4]),
       win=shift_windows, msb=st.booleans(), seed=st.integers(0, 2 ** 16))
def test_prop_w4a8(qg, m, n, kq, lda_x, ldc_x, win, msb, seed):
    M, N, K = m, n, 32 * kq
    d = datagen.gemm_w4a8(M, N, K, seed=seed, shift=win)
    C = out_buffer(M, N, ldc_x, torch.int8, 9)
    qg.qgemm_w4a8_requant(strided(d["A"], lda_x, 0), dev(d["B"]), dev(d["bias"]),
                          dev(d["mult"]), dev(d["shift"]), C=C[:, :N], msb_first=msb)
    got = C.cpu().numpy()
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"],
                                    msb_first=msb)
    assert np.array_equal(got[:, :N], want)
    assert np.all(got[:, N:] == 9)


@st.composite
def conv_geoms(draw):
    KH, KW = draw(st.sampled_from([(1, 1), (3, 3), (5, 5), (1, 3), (3, 1), (7, 7)]))
    sh, sw = draw(st.sampled_from([(1, 1), (2, 2), (1, 2), (3, 3)]))
    ph, pw = draw(st.integers(0, KH // 2 + 1)), draw(st.integers(0, KW // 2 + 1))
    H = draw(st.integers(max(1, KH - 2 * ph), 24))
    W = draw(st.integers(max(1, KW - 2 * pw), 60))
    batch = draw(st.integers(1, 3))
    return batch, H, W, KH, KW, (sh, sw), (ph, pw)


@SETTINGS
@given(g=conv_geoms(), ci=st.sampled_from([16, 32, 48, 64, 80]),
       co=st.sampled_from([16, 32, 64, 96, 128]), win=shift_windows, seed=st.integers(0, 2 ** 16))
def test_prop_conv(qg, g, ci, co, win, seed):
    batch, H, W, KH, KW, stride, pad = g
    d = datagen.conv_nhwc(batch, H, W, ci, co, KH, KW, seed=seed, shift=win)
    Y = qg.qconv2d_nhwc_s8_requant(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"]), stride=stride, pad=pad)
    want = oracle.conv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                         stride=stride, pad=pad)
    assert np.array_equal(Y.cpu().numpy(), want)


@SETTINGS
@given(g=conv_geoms(), c=st.sampled_from([16, 32, 64, 96, 192]), win=shift_windows,
       seed=st.integers(0, 2 ** 16))
def test_prop_dwconv(qg, g, c, win, seed):
    batch, H, W, KH, KW, stride, pad = g
    d = datagen.dwconv_nhwc(batch, H, W, c, KH, KW, seed=seed, shift=win)
    Y = qg.qdwconv2d_nhwc_s8_requant(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                     dev(d["shift"]), stride=stride, pad=pad)
    want = oracle.dwconv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                           stride=stride, pad=pad)
    assert np.array_equal(Y.cpu().numpy(), want)


# ---- asymmetric forms ----

zero_points = st.tuples(st.integers(-128, 127), st.integers(-128, 127), st.integers(-128, 127))
act_bounds = st.one_of(st.just((-128, 127)),
                       st.tuples(st.integers(-128, 127), st.integers(-128, 127)).map(
                           lambda t: (min(t), max(t))))


def full_range(seed, shape):
    return np.random.default_rng(seed).integers(-128, 127, size=shape, endpoint=True,
                                                dtype=np.int8)


@SETTINGS
@given(mn=gemm_dims, kq=st.integers(1, 24), zp=zero_points, act=act_bounds, win=shift_windows,
       bias=st.booleans(), ldc_x=st.sampled_from([0, 1, 16]), seed=st.integers(0, 2 ** 16))
def test_prop_s8s8_zp(qg, mn, kq, zp, act, win, bias, ldc_x, seed):
    (M, N), K = mn, 16 * kq
    d = datagen.gemm_s8s8(M, N, K, seed=seed, shift=win)
    A = full_range(seed + 1, (M, K))
    b = d["bias"] if bias else None
    za, zb, zo = zp
    want = oracle.gemm_s8s8_requant_zp(A, d["B"], b, d["mult"], d["shift"], za, zb, zo, act=act)
    args = (dev(A), dev(d["B"]), None if b is None else dev(b), dev(d["mult"]), dev(d["shift"]),
            za, zb, zo)
    C = out_buffer(M, N, ldc_x, torch.int8, 55)
    qg.qgemm_s8s8_requant_zp(*args, C=C[:, :N], act=act)
    got = C.cpu().numpy()
    assert np.array_equal(got[:, :N], want)
    assert np.all(got[:, N:] == 55)
    C.fill_(55)
    qg.qgemm_s8s8_requant_zp_noalloc(*args, C=C[:, :N], act=act)
    got = C.cpu().numpy()
    assert np.array_equal(got[:, :N], want)
    assert np.all(got[:, N:] == 55)


@SETTINGS
@given(g=conv_geoms(), ci=st.sampled_from([16, 32, 64, 80]), co=st.sampled_from([16, 64, 128]),
       zp=zero_points, act=act_bounds, win=shift_windows, seed=st.integers(0, 2 ** 16))
def test_prop_conv_zp(qg, g, ci, co, zp, act, win, seed):
    batch, H, W, KH, KW, stride, pad = g
    d = datagen.conv_nhwc(batch, H, W, ci, co, KH, KW, seed=seed, shift=win)
    X = full_range(seed + 1, d["X"].shape)
    za, zb, zo = zp
    Y = qg.qconv2d_nhwc_s8_requant_zp(dev(X), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                      dev(d["shift"]), za, zb, zo, stride=stride, pad=pad,
                                      act=act)
    want = oracle.conv2d_nhwc_s8_requant_zp(X, d["W"], d["bias"], d["mult"], d["shift"], za, zb,
                                            zo, stride=stride, pad=pad, act=act)
    assert np.array_equal(Y.cpu().numpy(), want)


@SETTINGS
@given(g=conv_geoms(), c=st.sampled_from([16, 32, 64, 192]), zp=zero_points,
       zb0=st.booleans(), act=act_bounds, win=shift_windows, seed=st.integers(0, 2 ** 16))
def test_prop_dwconv_zp(qg, g, c, zp, zb0, act, win, seed):
    batch, H, W, KH, KW, stride, pad = g
    d = datagen.dwconv_nhwc(batch, H, W, c, KH, KW, seed=seed, shift=win)
    X = full_range(seed + 1, d["X"].shape)
    za, zb, zo = zp
    zb = 0 if zb0 else zb  # zb == 0 keeps the 3x3 matrix-core path
    Y = qg.qdwconv2d_nhwc_s8_requant_zp(dev(X), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                        dev(d["shift"]), za, zb, zo, stride=stride, pad=pad,
                                        act=act)
    want = oracle.dwconv2d_nhwc_s8_requant_zp(X, d["W"], d["bias"], d["mult"], d["shift"], za,
                                              zb, zo, stride=stride, pad=pad, act=act)
    assert np.array_equal(Y.cpu().numpy(), want)


# ---- binary16 output ----

@SETTINGS
@given(mn=gemm_dims, kq=st.integers(1, 20), scaled=st.sampled_from(["none", "a", "b", "both"]),
       signed=st.booleans(), ldc_x=st.sampled_from([0, 1, 4]), seed=st.integers(0, 2 ** 16))
def test_prop_s4s4_f16(qg, mn, kq, scaled, signed, ldc_x, seed):
    (M, N), K = mn, 32 * kq
    d = datagen.gemm_s4s4(M, N, K, seed=seed)
    g = np.random.default_rng(seed + 1)
    lo = -4e-3 if signed else 1e-4

    def scales(n, on):
        return g.uniform(lo, 4e-3, n).astype(np.float32) if on else None

    sa = scales(M, scaled in ("a", "both"))
    sb = scales(N, scaled in ("b", "both"))
    C = torch.full((M, N + ldc_x), 1.5, dtype=torch.float16, device="cuda")
    qg.qgemm_s4s4_f16(dev(d["A"]), dev(d["B"]), None if sa is None else dev(sa),
                      None if sb is None else dev(sb), C=C[:, :N])
    want = oracle.gemm_s4s4_f16(d["A"], d["B"], sa, sb)
    got = C.cpu().numpy()
    assert np.array_equal(got[:, :N].view(np.uint16), want.view(np.uint16))
    assert np.all(got[:, N:] == np.float16(1.5))


# ---- per-token quantizer ----

@SETTINGS
@given(m=st.integers(1, 300), kq=st.integers(1, 150),
       dtype=st.sampled_from(["float32", "float16", "bfloat16"]), bits=st.sampled_from([8, 4]),
       clip=st.sampled_from([1.0, 0.9, 0.5]), zero_row=st.booleans(),
       seed=st.integers(0, 2 ** 16))
def test_prop_quant(qg, m, kq, dtype, bits, clip, zero_row, seed):
    K = 16 * kq  # the entry point's rule: K >= 16, K % 16 == 0
    X = datagen.activations(m, K, seed=seed)
    if zero_row:
        X[m // 2] = 0.0
    tdt = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(X)).to(tdt)
    h = t.view(torch.int16).numpy().view(np.uint16) if dtype == "bfloat16" else t.numpy()
    Q, scale = qg.qquant_per_token(t.cuda(), bits=bits, clip_ratio=clip)
    Qw, sw = oracle.quant_per_token(h, bits=bits, clip_ratio=clip, dtype=dtype)
    assert np.array_equal(Q.cpu().numpy().view(np.uint8), Qw.view(np.uint8))
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), sw.view(np.uint32))

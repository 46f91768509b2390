"""Parity of the asymmetric (zero-point) entry points with the oracle, byte
for byte.

The GEMM runs on both of its kernels (the tile kernel for small shapes, the
direct-to-LDS ring kernel for large ones); the conv on the LDS-staged kernel
(stride 1, 64 input channels) and the implicit-im2col one; the depthwise
conv on the 3x3 matrix-core kernel (weight zero point 0) and the direct one.
Zero points cover 0, both ends of the int8 range and values in between, for
each operand separately and together, with shift windows that keep most
outputs away from the clamp as well as saturating ones.
"""
import numpy as np
import pytest

from conv_qgemm_amd import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conv_qgemm_amd import qgemm
    return qgemm


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _say(*a):
    print(*a, flush=True)


def _full_range(g, shape):
    return g.integers(-128, 127, size=shape, endpoint=True, dtype=np.int8)


ZPS = [(0, 0, 0), (-128, 0, 5), (0, 127, -7), (17, -5, 100), (-128, -128, -128),
       (127, 127, 127), (3, 0, 0), (0, 0, -1)]


# ---------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (33, 17, 48), (129, 65, 144), (300, 260, 512),
                                   (4096, 2048, 256)])
@pytest.mark.parametrize("za,zb,zo", ZPS)
def test_gemm_zp(qg, orc, M, N, K, za, zb, zo):
    _say("gemm zp", M, N, K, za, zb, zo)
    d = datagen.gemm_s8s8(M, N, K, seed=M + N + K, shift=(40, 47))
    g = np.random.default_rng(M * 3 + K)
    A = _full_range(g, (M, K))
    C = qg.qgemm_s8s8_requant_zp(dev(A), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                 dev(d["shift"]), za, zb, zo)
    rows = None if M <= 512 else np.unique(np.r_[0, M - 1, g.choice(M, 24, replace=False)])
    want = orc.gemm_s8s8_requant_zp(A, d["B"], d["bias"], d["mult"], d["shift"], za, zb, zo,
                                    rows=rows)
    got = C.cpu().numpy()
    assert np.array_equal(got if rows is None else got[rows], want)


@pytest.mark.parametrize("M,N,K", [(70, 90, 160), (4096, 2048, 256)])
@pytest.mark.parametrize("act", [(5, 127), (-40, 60), (-128, -100), (9, 9)])
def test_gemm_zp_fused_activation(qg, orc, M, N, K, act):
    """ReLU at the output zero point (5, 127), a bounded clamp, a range at
    the low end, and a single value; on the tile and the ring kernel."""
    _say("gemm zp act", M, N, K, act)
    d = datagen.gemm_s8s8(M, N, K, seed=M + K, shift=(38, 44))
    C = qg.qgemm_s8s8_requant_zp(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                 dev(d["shift"]), -9, 4, 5, act=act)
    rows = None if M <= 512 else np.array([0, 77, 2048, 4095])
    want = orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"], -9, 4, 5,
                                    rows=rows, act=act)
    got = C.cpu().numpy()
    assert np.array_equal(got if rows is None else got[rows], want)


def test_gemm_zp_saturating_and_no_bias(qg, orc):
    d = datagen.gemm_s8s8(70, 90, 160, seed=5, shift=(31, 40))
    C = qg.qgemm_s8s8_requant_zp(dev(d["A"]), dev(d["B"]), None, dev(d["mult"]), dev(d["shift"]),
                                 -20, 9, -60)
    want = orc.gemm_s8s8_requant_zp(d["A"], d["B"], None, d["mult"], d["shift"], -20, 9, -60)
    assert np.array_equal(C.cpu().numpy(), want)


def test_gemm_zp_extremes(qg, orc):
    """(127 - (-128)) * (-128 - 127) in every term, at the largest K whose
    accumulator still fits in int32."""
    M, N, K = 64, 64, 33024 // 16 * 16
    A = np.full((M, K), 127, np.int8)
    B = np.full((N, K), -128, np.int8)
    mult = np.full(N, 2 ** 30, np.int32)
    shift = np.full(N, 63, np.int32)
    bias = np.zeros(N, np.int32)
    C = qg.qgemm_s8s8_requant_zp(dev(A), dev(B), dev(bias), dev(mult), dev(shift), -128, 127, 3)
    want = orc.gemm_s8s8_requant_zp(A, B, bias, mult, shift, -128, 127, 3)
    assert np.array_equal(C.cpu().numpy(), want)


def test_gemm_zp_full_size(qg, orc):
    """8192^3 with zero points on both operands and the output, on the ring
    kernel: every output against the oracle (about 15 s of oracle time on 16
    cores)."""
    _say("gemm zp 8192^3 full")
    d = datagen.workload("s8s8", unsaturated=True)
    za, zb, zo = -11, 6, 20
    C = qg.qgemm_s8s8_requant_zp(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                 dev(d["shift"]), za, zb, zo)
    got = C.cpu().numpy()
    want = orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"], za, zb, zo)
    _say("  mismatches:", int(np.sum(got != want)))
    assert np.array_equal(got, want)


def test_gemm_zp_workspace_reuse_and_strides(qg, orc):
    """Two calls in a row share one workspace; strided A and C."""
    ws = torch.empty(qg.lib.qgemm_s8s8_requant_zp_workspace_size(96, 80), dtype=torch.uint8,
                     device="cuda")
    d1 = datagen.gemm_s8s8(96, 80, 128, seed=8, shift=(38, 44))
    d2 = datagen.gemm_s8s8(40, 48, 64, seed=9, shift=(36, 42))
    Aw = torch.zeros((96, 160), dtype=torch.int8, device="cuda")
    Aw[:, :128] = dev(d1["A"])
    Cw = torch.full((96, 96), 7, dtype=torch.int8, device="cuda")
    qg.qgemm_s8s8_requant_zp(Aw[:, :128], dev(d1["B"]), dev(d1["bias"]), dev(d1["mult"]),
                             dev(d1["shift"]), 12, -3, 4, C=Cw[:, :80], workspace=ws)
    C2 = qg.qgemm_s8s8_requant_zp(dev(d2["A"]), dev(d2["B"]), dev(d2["bias"]), dev(d2["mult"]),
                                  dev(d2["shift"]), -7, 0, -2, workspace=ws)
    w1 = orc.gemm_s8s8_requant_zp(d1["A"], d1["B"], d1["bias"], d1["mult"], d1["shift"], 12, -3, 4)
    w2 = orc.gemm_s8s8_requant_zp(d2["A"], d2["B"], d2["bias"], d2["mult"], d2["shift"], -7, 0, -2)
    got = Cw.cpu().numpy()
    assert np.array_equal(got[:, :80], w1)
    assert np.all(got[:, 80:] == 7)
    assert np.array_equal(C2.cpu().numpy(), w2)


# ---------------------------------------------------------------- conv

CONV_GEOMS = [
    # batch, H, W, C_in, C_out, KH, KW, stride, pad  (first three: LDS-staged kernel)
    (2, 9, 11, 64, 64, 3, 3, (1, 1), (1, 1)),
    (1, 14, 14, 64, 128, 3, 3, (1, 1), (1, 1)),
    (1, 7, 9, 64, 64, 1, 1, (1, 1), (0, 0)),
    (1, 40, 32, 16, 16, 3, 3, (2, 2), (1, 1)),
    (2, 8, 7, 32, 48, 3, 3, (1, 1), (1, 1)),
    (1, 9, 9, 16, 32, 5, 5, (2, 1), (2, 2)),
]


@pytest.mark.parametrize("geom", CONV_GEOMS)
@pytest.mark.parametrize("za,zb,zo", [(0, 0, 0), (-128, 0, 9), (45, -9, -30), (127, 127, 127),
                                      (0, 64, 0)])
def test_conv_zp(qg, orc, geom, za, zb, zo):
    b, H, W, C_in, C_out, KH, KW, stride, pad = geom
    _say("conv zp", geom, za, zb, zo)
    d = datagen.conv_nhwc(b, H, W, C_in, C_out, KH, KW, seed=H + W + C_in, shift=(38, 45))
    g = np.random.default_rng(H * W)
    X = _full_range(g, (b, H, W, C_in))
    Y = qg.qconv2d_nhwc_s8_requant_zp(dev(X), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                      dev(d["shift"]), za, zb, zo, stride=stride, pad=pad)
    want = orc.conv2d_nhwc_s8_requant_zp(X, d["W"], d["bias"], d["mult"], d["shift"], za, zb, zo,
                                         stride=stride, pad=pad)
    assert np.array_equal(Y.cpu().numpy(), want)


@pytest.mark.parametrize("geom", [CONV_GEOMS[0], CONV_GEOMS[3]])
@pytest.mark.parametrize("act", [(-30, 127), (-60, 20)])
def test_conv_zp_fused_activation(qg, orc, geom, act):
    b, H, W, C_in, C_out, KH, KW, stride, pad = geom
    _say("conv zp act", geom, act)
    d = datagen.conv_nhwc(b, H, W, C_in, C_out, KH, KW, seed=H + W, shift=(38, 45))
    Y = qg.qconv2d_nhwc_s8_requant_zp(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                      dev(d["shift"]), 11, -3, -30, stride=stride, pad=pad,
                                      act=act)
    want = orc.conv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"], 11, -3,
                                         -30, stride=stride, pad=pad, act=act)
    assert np.array_equal(Y.cpu().numpy(), want)


def test_conv_zp_workload_full(qg, orc):
    """The 32x56x56x64 -> 64 3x3 layer with zero points on input, weights and
    output, every output compared."""
    _say("conv zp workload")
    d = datagen.workload("conv3x3", unsaturated=True)
    za, zb, zo = -5, 3, 11
    Y = qg.qconv2d_nhwc_s8_requant_zp(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                      dev(d["shift"]), za, zb, zo)
    want = orc.conv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"], za, zb,
                                         zo)
    assert np.array_equal(Y.cpu().numpy(), want)


# ---------------------------------------------------------------- depthwise

DW_GEOMS = [
    # batch, H, W, C, KH, KW, stride, pad
    (2, 9, 11, 64, 3, 3, (1, 1), (1, 1)),
    (1, 12, 10, 32, 3, 3, (2, 2), (1, 1)),
    (1, 7, 7, 80, 3, 3, (1, 1), (1, 1)),
    (1, 9, 8, 16, 5, 5, (1, 1), (2, 2)),
    (2, 6, 9, 48, 3, 3, (1, 2), (1, 1)),
    (2, 30, 24, 64, 3, 3, (1, 1), (1, 1)),  # Wo 24: paired taps, zero-point padding
]


@pytest.mark.parametrize("geom", DW_GEOMS)
@pytest.mark.parametrize("za,zb,zo", [(0, 0, 0), (-128, 0, 9), (45, 0, -30), (45, -9, -30),
                                      (127, 127, 127)])
def test_dwconv_zp(qg, orc, geom, za, zb, zo):
    b, H, W, C, KH, KW, stride, pad = geom
    _say("dwconv zp", geom, za, zb, zo)
    d = datagen.dwconv_nhwc(b, H, W, C, KH, KW, seed=H * W + C, shift=(30, 37))
    g = np.random.default_rng(C + H)
    X = _full_range(g, (b, H, W, C))
    Wt = _full_range(g, (KH, KW, C))
    Y = qg.qdwconv2d_nhwc_s8_requant_zp(dev(X), dev(Wt), dev(d["bias"]), dev(d["mult"]),
                                        dev(d["shift"]), za, zb, zo, stride=stride, pad=pad)
    want = orc.dwconv2d_nhwc_s8_requant_zp(X, Wt, d["bias"], d["mult"], d["shift"], za, zb, zo,
                                           stride=stride, pad=pad)
    assert np.array_equal(Y.cpu().numpy(), want)


@pytest.mark.parametrize("geom", [DW_GEOMS[0], DW_GEOMS[3]])
def test_dwconv_zp_relu(qg, orc, geom):
    """ReLU at the output zero point on the matrix-core and the direct path."""
    b, H, W, C, KH, KW, stride, pad = geom
    d = datagen.dwconv_nhwc(b, H, W, C, KH, KW, seed=C, shift=(30, 37))
    Y = qg.qdwconv2d_nhwc_s8_requant_zp(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                        dev(d["shift"]), 6, 0, -12, stride=stride, pad=pad,
                                        act=(-12, 127))
    want = orc.dwconv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"], 6, 0,
                                           -12, stride=stride, pad=pad, act=(-12, 127))
    assert np.array_equal(Y.cpu().numpy(), want)


def test_dwconv_zp_workload_full(qg, orc):
    _say("dwconv zp workload")
    d = datagen.workload("dw3x3", unsaturated=True)
    for za, zb, zo in ((-7, 0, 15), (9, 4, -3)):
        Y = qg.qdwconv2d_nhwc_s8_requant_zp(dev(d["X"]), dev(d["W"]), dev(d["bias"]),
                                            dev(d["mult"]), dev(d["shift"]), za, zb, zo)
        want = orc.dwconv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                               za, zb, zo)
        assert np.array_equal(Y.cpu().numpy(), want), (za, zb, zo)


# ---------------------------------------------------------------- MSB-first INT4

@pytest.mark.parametrize("M,N,K", [(16, 512, 1024), (5, 100, 8224), (64, 96, 16416),
                                   (100, 160, 512), (300, 260, 1024)])
def test_w4a8_msb_first(qg, orc, M, N, K):
    """Skinny kernel for M <= 64 (including K tails), tile kernel above."""
    _say("w4a8 msb", M, N, K)
    d = datagen.gemm_w4a8(M, N, K, seed=M + N, shift=(37, 43))
    C = qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]), msb_first=True)
    want = orc.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"],
                                 msb_first=True)
    assert np.array_equal(C.cpu().numpy(), want)
    # the same bytes read low nibble first give a different result
    lsb = orc.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert not np.array_equal(want, lsb)


def test_w4a8_msb_workload_full(qg, orc):
    _say("w4a8 msb workload")
    d = datagen.workload("w4a8", unsaturated=True)
    C = qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]), msb_first=True)
    want = orc.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"],
                                 msb_first=True)
    assert np.array_equal(C.cpu().numpy(), want)


def test_s4s4_msb_first_operands(qg, orc):
    """Both operands high nibble first: qgemm_s4s4_i32 gives the MSB-first
    product as it stands."""
    d = datagen.gemm_s4s4(130, 70, 512, seed=12)
    C = qg.qgemm_s4s4_i32(dev(d["A"]), dev(d["B"]))
    assert np.array_equal(C.cpu().numpy(), orc.gemm_s4s4_i32(d["A"], d["B"], msb_first=True))

"""Parity of the HIP path with the CPU oracle, byte for byte.

Every case draws seeded inputs, runs the library through its C ABI (via the
ctypes binding) on the GPU and compares with the oracle on the same inputs.
Integer results are unique, so the bar is exact equality.  Small cases span
several tiles with ragged tails in M, N and K.  The full-size workloads of
the step (pointwise, s4s4 4096^3, conv3x3, skinny W4A8, s8s8 8192^3,
depthwise 3x3) are compared on every output; only the 2048-token W4A8
prefill, outside that set, is checked on sampled rows.
"""
import numpy as np
import pytest

import oracle
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


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _say(*a):
    print(*a, flush=True)


def _sample_rows(M, n, seed):
    g = np.random.default_rng(seed)
    rows = set(g.choice(M, size=min(n, M), replace=False).tolist())
    rows |= {0, M - 1, max(M - 2, 0)}
    return np.array(sorted(rows), dtype=np.int64)


# ---------------------------------------------------------------- s8s8

S8_SHAPES = [
    (1, 1, 16), (7, 5, 16), (33, 17, 48), (64, 64, 64), (129, 65, 144), (320, 64, 64),
    (300, 260, 512), (517, 389, 272), (1500, 1500, 96),
]


@pytest.mark.parametrize("M,N,K", S8_SHAPES)
@pytest.mark.parametrize("unsat", [False, True])
def test_s8s8_small(qg, M, N, K, unsat):
    _say("s8s8", M, N, K, unsat)
    d = datagen.gemm_s8s8(M, N, K, seed=M + N + K, shift=(38, 44) if unsat else (31, 40))
    C = qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]))
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(host(C), want)


def test_s8s8_large_tile_sampled(qg):
    # enough 256x256 tiles to select the largest tile, ragged in M and N
    M, N, K = 4100, 4130, 160
    _say("s8s8 large tile", M, N, K)
    d = datagen.gemm_s8s8(M, N, K, seed=77, shift=(36, 42))
    C = host(qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    rows = _sample_rows(M, 200, 1)
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
    assert np.array_equal(C[rows], want)


def test_s8s8_no_bias_and_strided(qg):
    M, N, K = 96, 80, 128
    d = datagen.gemm_s8s8(M, N, K, seed=3, shift=(36, 40))
    Aw = np.zeros((M, K + 48), np.int8)
    Aw[:, :K] = d["A"]
    Bw = np.zeros((N, K + 16), np.int8)
    Bw[:, :K] = d["B"]
    At, Bt = dev(Aw), dev(Bw)
    Cw = torch.full((M, N + 32), 99, dtype=torch.int8, device="cuda")
    qg.qgemm_s8s8_requant(At[:, :K], Bt[:, :K], None, dev(d["mult"]), dev(d["shift"]),
                          C=Cw[:, :N])
    got = host(Cw)
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], None, d["mult"], d["shift"])
    assert np.array_equal(got[:, :N], want)
    assert np.all(got[:, N:] == 99)  # nothing written past N


@pytest.mark.parametrize("ldc_extra", [1, 3])
def test_unaligned_output_stride(qg, ldc_extra):
    # an output row stride that is not a multiple of 4 takes the scalar stores
    M, N, K = 70, 36, 64
    d = datagen.gemm_s8s8(M, N, K, seed=31, shift=(36, 40))
    Cw = torch.zeros((M, N + ldc_extra), dtype=torch.int8, device="cuda")
    qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                          dev(d["shift"]), C=Cw[:, :N])
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    got = host(Cw)
    assert np.array_equal(got[:, :N], want) and np.all(got[:, N:] == 0)
    s = datagen.gemm_s4s4(M, N, K, seed=32)
    Ci = torch.zeros((M, N + ldc_extra), dtype=torch.int32, device="cuda")
    qg.qgemm_s4s4_i32(dev(s["A"]), dev(s["B"]), C=Ci[:, :N])
    goti = host(Ci)
    assert np.array_equal(goti[:, :N], oracle.gemm_s4s4_i32(s["A"], s["B"]))
    assert np.all(goti[:, N:] == 0)
    w = datagen.gemm_w4a8(9, N, 128, seed=33, shift=(37, 43))
    Cs = torch.zeros((9, N + ldc_extra), dtype=torch.int8, device="cuda")
    qg.qgemm_w4a8_requant(dev(w["A"]), dev(w["B"]), dev(w["bias"]), dev(w["mult"]),
                          dev(w["shift"]), C=Cs[:, :N])
    gots = host(Cs)
    assert np.array_equal(gots[:, :N], oracle.gemm_w4a8_requant(w["A"], w["B"], w["bias"],
                                                                w["mult"], w["shift"]))


def test_s8s8_extremes(qg):
    # -128 operands, large K, shifts at both ends of the domain
    M, N, K = 64, 48, 1024
    A = np.full((M, K), -128, np.int8)
    B = np.full((N, K), -128, np.int8)
    B[1::2] = 127
    bias = np.zeros(N, np.int32)
    mult = np.full(N, 2 ** 31 - 1, np.int32)
    shift = np.array([1, 63, 31, 44] * (N // 4), np.int32)
    C = qg.qgemm_s8s8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift))
    assert np.array_equal(host(C), oracle.gemm_s8s8_requant(A, B, bias, mult, shift))


# ---------------------------------------------------------------- s4s4

S4_SHAPES = [(1, 1, 32), (16, 64, 32), (37, 29, 96), (130, 70, 288), (300, 200, 544),
             (1500, 1500, 64)]


@pytest.mark.parametrize("M,N,K", S4_SHAPES)
def test_s4s4_small(qg, M, N, K):
    _say("s4s4", M, N, K)
    d = datagen.gemm_s4s4(M, N, K, seed=M * 3 + K)
    C = qg.qgemm_s4s4_i32(dev(d["A"]), dev(d["B"]))
    assert np.array_equal(host(C), oracle.gemm_s4s4_i32(d["A"], d["B"]))


def test_s4s4_hello_world(qg):
    # the INT4 GEMM article's example: A all 0x11, B all 0x22, K = 32 -> 64
    A = np.full((16, 16), 0x11, np.uint8)
    B = np.full((64, 16), 0x22, np.uint8)
    C = host(qg.qgemm_s4s4_i32(dev(A), dev(B)))
    assert np.all(C == 64)


def test_s4s4_extremes(qg):
    M, N, K = 64, 64, 4096
    A = np.full((M, K // 2), 0x88, np.uint8)  # all -8
    B = np.full((N, K // 2), 0x88, np.uint8)
    B[::3] = 0x77                              # all 7
    C = host(qg.qgemm_s4s4_i32(dev(A), dev(B)))
    assert np.array_equal(C, oracle.gemm_s4s4_i32(A, B))
    assert C[0, 1] == 64 * K and C[0, 0] == -56 * K


def test_s4s4_max_k(qg):
    """K at the API bound (131040): +-8 x +-8 products summed over K, scaled
    by 256 inside the kernel, sit right at the int32 edge."""
    M, N, K = 64, 64, 131040
    A = np.full((M, K // 2), 0x88, np.uint8)  # all -8
    B = np.full((N, K // 2), 0x88, np.uint8)
    B[1::2] = 0x77                             # all 7
    g = np.random.default_rng(11)
    A[5:] = g.integers(0, 256, size=(M - 5, K // 2), dtype=np.uint8)
    C = host(qg.qgemm_s4s4_i32(dev(A), dev(B)))
    assert C[0, 0] == 64 * K and C[0, 1] == -56 * K
    assert np.array_equal(C, oracle.gemm_s4s4_i32(A, B))


def test_s4s4_max_k_ring_kernel(qg):
    """The largest K (a multiple of 128) that the direct-to-LDS ring kernel
    takes, on enough tiles to select it; constant operands give closed forms."""
    M, N, K = 2048, 4096, 130944
    A = torch.full((M, K // 2), 0x88, dtype=torch.uint8, device="cuda")
    B = torch.full((N, K // 2), 0x88, dtype=torch.uint8, device="cuda")
    B[1::2] = 0x77
    C = host(qg.qgemm_s4s4_i32(A, B))
    assert np.all(C[:, 0::2] == 64 * K) and np.all(C[:, 1::2] == -56 * K)


# ---------------------------------------------------------------- w4a8

W4_SHAPES = [
    (1, 16, 32), (5, 100, 544), (16, 64, 8192), (16, 1000, 8224), (16, 48, 16416),
    (33, 77, 256), (64, 32, 512), (65, 130, 160), (300, 260, 640),
]


@pytest.mark.parametrize("M", [16, 100])
def test_w4a8_max_k(qg, M):
    """K at the API bound (131040) with -128 activations against -8 / 7
    weights: the x16-scaled accumulator sits right at the int32 edge (M = 16
    is the weight-streaming kernel, M = 100 the tile kernel)."""
    N, K = 64, 131040
    g = np.random.default_rng(12)
    A = np.full((M, K), -128, np.int8)
    A[3:] = g.integers(-128, 128, size=(M - 3, K), dtype=np.int8)
    B = np.full((N, K // 2), 0x88, np.uint8)
    B[1::2] = 0x77
    bias = g.integers(-2 ** 15, 2 ** 15, size=N, dtype=np.int32)
    mult = g.integers(2 ** 30, 2 ** 31, size=N, dtype=np.int64).astype(np.int32)
    shift = g.integers(44, 53, size=N, dtype=np.int32)
    C = qg.qgemm_w4a8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift))
    assert np.array_equal(host(C), oracle.gemm_w4a8_requant(A, B, bias, mult, shift))


@pytest.mark.parametrize("M,N,K", W4_SHAPES)
def test_w4a8_small(qg, M, N, K):
    _say("w4a8", M, N, K)
    d = datagen.gemm_w4a8(M, N, K, seed=M + 7 * N + K, shift=(37, 43))
    C = qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]))
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(host(C), want)


@pytest.mark.parametrize("M,N,K", [(40, 1000, 8192), (17, 4100, 8128), (64, 96, 8192),
                                   (16, 1, 8192), (64, 8, 32), (63, 17, 4096)])
@pytest.mark.parametrize("msb", [False, True])
def test_w4a8_skinny_staged_activations(qg, M, N, K, msb):
    """K <= 8192 on the weight-streaming kernel: six of its eight waves bring
    their activation slices through LDS (token-swizzled direct-to-LDS copies
    read back in the MFMA layout), two load them directly.  Several 16-token
    row blocks (M > 16), a ragged last block, a K tail short of the 8192-value
    chunk and a ragged N, in both nibble orders; one column (a single group,
    whose parameters arrive at the end of its only unit) and K = 32."""
    _say("w4a8 staged", M, N, K, msb)
    d = datagen.gemm_w4a8(M, N, K, seed=M + N + K, shift=(37, 43))
    C = qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]), msb_first=msb)
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"],
                                    msb_first=msb)
    assert np.array_equal(host(C), want)


# ---------------------------------------------------------------- conv

CONV_GEOMS = [
    # batch, H, W, C_in, C_out, KH, KW, stride, pad
    (1, 7, 6, 16, 16, 3, 3, (1, 1), (1, 1)),
    (2, 9, 8, 16, 32, 3, 3, (2, 2), (1, 1)),
    (1, 10, 7, 32, 16, 3, 3, (1, 1), (0, 0)),
    (1, 8, 8, 16, 48, 5, 5, (1, 1), (2, 2)),
    (2, 6, 11, 16, 16, 1, 3, (1, 2), (0, 1)),
    (1, 5, 5, 16, 16, 3, 3, (2, 1), (2, 0)),
    (3, 20, 16, 64, 64, 1, 1, (1, 1), (0, 0)),
    (2, 14, 14, 64, 64, 3, 3, (1, 1), (1, 1)),
    (1, 12, 13, 32, 128, 3, 3, (1, 1), (1, 1)),
    (1, 11, 9, 48, 80, 3, 3, (2, 2), (1, 1)),
    (1, 40, 32, 16, 16, 3, 3, (2, 2), (1, 1)),  # first layer of the MCU front-end, C_in padded to 16
    # stride 1, 64 input channels: the kernel that stages input rows in LDS
    (1, 12, 13, 64, 128, 3, 3, (1, 1), (1, 1)),   # two output-channel tiles
    (2, 10, 9, 64, 64, 3, 3, (1, 1), (0, 0)),     # no padding
    (1, 9, 30, 64, 192, 3, 3, (1, 1), (2, 0)),    # unequal padding, three channel tiles
    (2, 40, 3, 64, 64, 3, 3, (1, 1), (1, 1)),     # 3 pixels wide: one tile spans the image
    (1, 4, 100, 64, 64, 3, 3, (1, 1), (1, 1)),    # wide rows: a 392-pixel band and an 8-pixel one
    (2, 30, 30, 64, 64, 3, 3, (1, 1), (1, 1)),    # bands of 392 pixels starting mid-row
    (1, 200, 3, 64, 64, 3, 3, (1, 1), (1, 1)),    # a band spanning 131 rows
    (1, 5, 6, 64, 64, 1, 1, (1, 1), (1, 1)),      # 1x1 with padding: border pixels see zeros
    (3, 17, 19, 64, 64, 3, 3, (1, 1), (1, 1)),    # several images, partial last tile
]


@pytest.mark.parametrize("geom", CONV_GEOMS)
def test_conv_small(qg, geom):
    b, H, Wd, Ci, Co, KH, KW, stride, pad = geom
    _say("conv", geom)
    d = datagen.conv_nhwc(b, H, Wd, Ci, Co, KH, KW, seed=H * Wd + Ci, shift=(35, 41))
    Y = qg.qconv2d_nhwc_s8_requant(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"]), stride=stride, pad=pad)
    want = oracle.conv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                         stride=stride, pad=pad)
    assert np.array_equal(host(Y), want)


def test_conv_pointwise_equals_gemm(qg):
    d = datagen.workload("pointwise", unsaturated=True)
    X = dev(d["A"].reshape(1, 20, 16, 64))
    W = dev(d["B"].reshape(64, 1, 1, 64))
    Y = qg.qconv2d_nhwc_s8_requant(X, W, dev(d["bias"]), dev(d["mult"]), dev(d["shift"]),
                                   stride=(1, 1), pad=(0, 0))
    C = qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]))
    assert np.array_equal(host(Y).reshape(320, 64), host(C))


# ---------------------------------------------------------------- depthwise conv

DW_GEOMS = [
    # batch, H, W, C, KH, KW, stride, pad
    (1, 7, 6, 16, 3, 3, (1, 1), (1, 1)),
    (2, 9, 8, 32, 3, 3, (2, 2), (1, 1)),
    (1, 10, 7, 96, 3, 3, (1, 1), (0, 0)),     # a full and a 32-channel slice
    (1, 20, 16, 16, 3, 3, (1, 1), (1, 1)),    # the MCU front-end's 20x16x16 map
    (2, 40, 3, 64, 3, 3, (1, 1), (1, 1)),     # 3 pixels wide: one tile spans the image
    (2, 30, 30, 64, 3, 3, (1, 1), (1, 1)),    # bands of 392 pixels starting mid-row
    (1, 200, 3, 64, 3, 3, (1, 1), (1, 1)),    # a band spanning 131 rows
    (1, 61, 60, 64, 3, 3, (2, 2), (1, 1)),    # stride 2, bands starting mid-row
    (1, 13, 30, 128, 3, 3, (2, 2), (1, 1)),   # stride 2, two slices
    (3, 17, 19, 64, 3, 3, (1, 1), (2, 0)),    # unequal padding, several images
    (1, 8, 8, 16, 5, 5, (1, 1), (2, 2)),      # direct kernel: 5x5
    (2, 6, 11, 32, 1, 3, (1, 2), (0, 1)),     # direct kernel: 1x3, unequal strides
    (1, 9, 9, 48, 3, 3, (2, 1), (1, 1)),      # direct kernel: unequal strides
    (1, 3, 200, 16, 3, 3, (2, 2), (1, 1)),    # wide rows at stride 2
    # stride 1, Wo a multiple of 8: LDS rows padded to Wo mod 16, paired taps
    (1, 12, 8, 32, 3, 3, (1, 1), (1, 1)),     # Wo 8
    (2, 30, 24, 64, 3, 3, (1, 1), (1, 1)),    # Wo 24, bands starting mid-row
    (1, 12, 112, 64, 3, 3, (1, 1), (1, 1)),   # Wo 112: a band is 3.5 rows
    (1, 14, 18, 32, 3, 3, (1, 1), (1, 0)),    # Wo 16 with no column padding
]


@pytest.mark.parametrize("geom", DW_GEOMS)
def test_dwconv_small(qg, geom):
    b, H, Wd, C, KH, KW, stride, pad = geom
    _say("dwconv", geom)
    d = datagen.dwconv_nhwc(b, H, Wd, C, KH, KW, seed=H * Wd + C, shift=(36, 42))
    Y = qg.qdwconv2d_nhwc_s8_requant(dev(d["X"]), dev(d["W"]), dev(d["bias"]), dev(d["mult"]),
                                     dev(d["shift"]), stride=stride, pad=pad)
    want = oracle.dwconv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                           stride=stride, pad=pad)
    assert np.array_equal(host(Y), want)


def test_dwconv_extremes(qg):
    """-128 inputs against -128 / 127 weights, shifts at both ends."""
    b, H, Wd, C = 1, 9, 10, 32
    X = np.full((b, H, Wd, C), -128, np.int8)
    Wt = np.full((3, 3, C), -128, np.int8)
    Wt[..., 1::2] = 127
    bias = np.zeros(C, np.int32)
    mult = np.full(C, 2 ** 31 - 1, np.int32)
    shift = np.array([1, 63, 31, 44] * (C // 4), np.int32)
    Y = qg.qdwconv2d_nhwc_s8_requant(dev(X), dev(Wt), dev(bias), dev(mult), dev(shift))
    assert np.array_equal(host(Y), oracle.dwconv2d_nhwc_s8_requant(X, Wt, bias, mult, shift))


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("unsat", [False, True])
def test_workload_pointwise(qg, unsat):
    d = datagen.workload("pointwise", unsaturated=unsat)
    C = qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                              dev(d["shift"]))
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(host(C), want)


def test_workload_s4s4_full(qg):
    """INT4 x INT4 4096^3: every one of the 16.8 M int32 outputs against the
    oracle (about 10 s of oracle time on 16 cores)."""
    _say("workload s4s4 4096^3 full")
    d = datagen.workload("s4s4")
    C = host(qg.qgemm_s4s4_i32(dev(d["A"]), dev(d["B"])))
    want = oracle.gemm_s4s4_i32(d["A"], d["B"])
    _say("  mismatches:", int(np.sum(C != want)))
    assert np.array_equal(C, want)


@pytest.mark.parametrize("unsat", [False, True])
def test_workload_conv3x3_full(qg, unsat):
    _say("workload conv3x3 full", unsat)
    d = datagen.workload("conv3x3", unsaturated=unsat)
    Y = host(qg.qconv2d_nhwc_s8_requant(dev(d["X"]), dev(d["W"]), dev(d["bias"]),
                                        dev(d["mult"]), dev(d["shift"]), stride=(1, 1),
                                        pad=(1, 1)))
    want = oracle.conv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                         stride=(1, 1), pad=(1, 1))
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("unsat", [False, True])
def test_workload_dw3x3_full(qg, unsat):
    _say("workload dw3x3 full", unsat)
    d = datagen.workload("dw3x3", unsaturated=unsat)
    Y = host(qg.qdwconv2d_nhwc_s8_requant(dev(d["X"]), dev(d["W"]), dev(d["bias"]),
                                          dev(d["mult"]), dev(d["shift"]), stride=(1, 1),
                                          pad=(1, 1)))
    want = oracle.dwconv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                           stride=(1, 1), pad=(1, 1))
    assert np.array_equal(Y, want)


@pytest.mark.parametrize("unsat", [False, True])
def test_workload_w4a8_full(qg, unsat):
    _say("workload w4a8 full", unsat)
    d = datagen.workload("w4a8", unsaturated=unsat)
    C = host(qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(C, want)


@pytest.mark.parametrize("M", [17, 33, 64])
def test_skinny_token_blocks_full(qg, M):
    """17, 33 and 64 tokens against the full 28672 x 8192 int4 weights: two to
    four 16-token blocks share the weight-streaming kernel's pass over the
    weights (the last block ragged at 17 and 33); every output compared."""
    _say("w4a8 skinny token blocks", M)
    d = datagen.gemm_w4a8(M, 28672, 8192, seed=200 + M, shift=(37, 43))
    C = host(qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(C, want)


W4A8_RING = [(2048, 4096, 256), (2048, 4096, 1152), (2000, 4100, 640), (1025, 8200, 384)]


@pytest.mark.parametrize("M,N,K", W4A8_RING)
@pytest.mark.parametrize("msb", [False, True])
def test_w4a8_ring_kernel(qg, M, N, K, msb):
    """Shapes with enough 256 x 256 tiles and K % 128 == 0 take the
    direct-to-LDS ring kernel (int8 A rows of 128 bytes per stage); ragged M
    and N included."""
    _say("w4a8 ring", M, N, K, msb)
    d = datagen.gemm_w4a8(M, N, K, seed=M + K, shift=(37, 43))
    C = host(qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"]), msb_first=msb))
    rows = _sample_rows(M, 10, seed=K)
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows,
                                    msb_first=msb)
    assert np.array_equal(C[rows], want)


RING_STAGES = [(2048, 4096, 4), (2048, 4096, 5), (2000, 4100, 6), (1025, 8200, 7)]


@pytest.mark.parametrize("M,N,stages", RING_STAGES)
def test_ring_kernel_stage_parity(qg, M, N, stages):
    """The ring kernel multiplies int8 and packed int4 operands in pairs of
    64-byte K stages when the stage count is even (one slot of 128-byte rows
    per pair) and stage by stage otherwise: 4 to 7 stages, ragged M and N,
    every output of s8s8 (requantize) and s4s4 (raw int32) compared."""
    _say("ring stages", M, N, stages)
    K = 64 * stages
    d = datagen.gemm_s8s8(M, N, K, seed=stages, shift=(37, 43))
    C = host(qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(C, want)
    K4 = 128 * stages  # 64 packed bytes per stage
    d4 = datagen.gemm_s4s4(M, N, K4, seed=stages + 10)
    C4 = host(qg.qgemm_s4s4_i32(dev(d4["A"]), dev(d4["B"])))
    rows = _sample_rows(M, 64, seed=stages)
    assert np.array_equal(C4[rows], oracle.gemm_s4s4_i32(d4["A"], d4["B"], rows=rows))



RING_SHORT_K_TILES = [(4096, 8192, 4), (4096, 8192, 5), (4000, 8200, 6)]


@pytest.mark.parametrize("M,N,stages", RING_SHORT_K_TILES)
def test_ring_kernel_short_k_several_tiles(qg, M, N, stages):
    """512 and more 256x256 tiles, so that a workgroup walks two or three
    of them: with 4 and 6 stages (2 and 3 pairs) the last pairs of a tile
    load the next tile's first two, into slots that tile then multiplies
    from; every output of s8s8 and of s4s4 compared."""
    _say("ring short K, several tiles", M, N, stages)
    K = 64 * stages
    d = datagen.gemm_s8s8(M, N, K, seed=20 + stages, shift=(37, 43))
    C = host(qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    assert np.array_equal(C, oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"],
                                                      d["shift"]))
    d4 = datagen.gemm_s4s4(M, N, 128 * stages, seed=30 + stages)
    C4 = host(qg.qgemm_s4s4_i32(dev(d4["A"]), dev(d4["B"])))
    assert np.array_equal(C4, oracle.gemm_s4s4_i32(d4["A"], d4["B"]))

def test_w4a8_ring_kernel_max_k(qg):
    """The largest K of whole 128-value stages under the int4 bound, with
    operands at the ends of their ranges, so that the x16 widened sums sit at
    the int32 edge."""
    M, N, K = 2048, 4096, 130944
    A = np.full((M, K), -128, np.int8)
    A[1::2] = 127
    B = np.full((N, K // 2), 0x88, np.uint8)  # every weight -8
    B[1::3] = 0x77                            # every weight 7
    mult = np.full(N, 2 ** 30, np.int32)
    shift = np.full(N, 44, np.int32)
    bias = np.zeros(N, np.int32)
    C = host(qg.qgemm_w4a8_requant(dev(A), dev(B), dev(bias), dev(mult), dev(shift)))
    rows = np.array([0, 1, 2046, 2047])
    want = oracle.gemm_w4a8_requant(A, B, bias, mult, shift, rows=rows)
    assert np.array_equal(C[rows], want)
    assert len(np.unique(want)) > 1


@pytest.mark.parametrize("unsat", [False, True])
def test_workload_w4a8_prefill_sampled(qg, unsat):
    """2048 tokens x 28672 x 8192 (the prefill shape), sampled rows."""
    _say("workload w4a8 prefill", unsat)
    d = datagen.workload("w4a8_prefill", unsaturated=unsat)
    C = host(qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    rows = _sample_rows(2048, 64, seed=31)
    want = oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
    assert np.array_equal(C[rows], want)


@pytest.mark.parametrize("unsat", [False, True])
def test_workload_s8s8_full(qg, unsat):
    """s8s8 8192^3 in both shift windows: every one of the 67 M int8 outputs
    against the oracle (about 12 s of oracle time per window on 16 cores)."""
    _say("workload s8s8 8192^3 full", unsat)
    d = datagen.workload("s8s8", unsaturated=unsat)
    C = host(qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    want = oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    _say("  mismatches:", int(np.sum(C != want)),
         " saturated:", round(float(np.mean((want == 127) | (want == -128))), 3))
    assert np.array_equal(C, want)


# ---------------------------------------------------------------- runtime behaviour

def test_deterministic_and_side_stream(qg):
    d = datagen.gemm_s8s8(700, 300, 256, seed=12, shift=(36, 42))
    args = [dev(d[k]) for k in ("A", "B", "bias", "mult", "shift")]
    ref = host(qg.qgemm_s8s8_requant(*args))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = [qg.qgemm_s8s8_requant(*args, stream=s) for _ in range(3)]
    s.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy(), ref)


def test_invalid_call_on_gpu_raises(qg):
    A = torch.zeros((32, 40), dtype=torch.int8, device="cuda")  # K = 40 breaks K % 16
    B = torch.zeros((16, 40), dtype=torch.int8, device="cuda")
    p = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_s8s8_requant(A, B, p, p, p)
    assert e.value.status == qg.QG_ERR_INVALID

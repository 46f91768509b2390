"""Pins of the oracle's GEMMs: numpy int64 matmul and big-int brute force on
small shapes, constant-operand closed forms, and the requantized GEMMs
against the separately pinned requantize."""
import numpy as np
import pytest

from conv_qgemm_amd import datagen


def _decode(packed):
    """numpy-only int4 decode (int8 sign extension), low nibble = even index."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p << 4).astype(np.uint8).view(np.int8) >> 4
    hi = p.view(np.int8) >> 4
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _bigint_gemm(A, B):
    M, K = len(A), len(A[0])
    N = len(B)
    return [[sum(int(A[m][k]) * int(B[n][k]) for k in range(K)) for n in range(N)]
            for m in range(M)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 9, 16), (7, 1, 33)])
def test_s8s8_bruteforce_tiny(orc, M, N, K):
    g = np.random.default_rng(M * 100 + N * 10 + K)
    A = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    B = g.integers(-128, 128, size=(N, K), dtype=np.int8)
    assert orc.gemm_acc(A, B).tolist() == _bigint_gemm(A.tolist(), B.tolist())


@pytest.mark.parametrize("M,N,K", [(64, 48, 96), (100, 37, 160), (33, 65, 512)])
def test_s8s8_vs_numpy(orc, M, N, K):
    g = np.random.default_rng(M + N + K)
    A = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    B = g.integers(-128, 128, size=(N, K), dtype=np.int8)
    want = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(orc.gemm_acc(A, B), want)


@pytest.mark.parametrize("M,N,K", [(4, 4, 2), (5, 3, 8), (16, 64, 32), (37, 29, 96)])
def test_s4s4_vs_numpy(orc, M, N, K):
    g = np.random.default_rng(K * 7 + M)
    Ap = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    Bp = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    want = _decode(Ap) @ _decode(Bp).T
    assert np.array_equal(orc.gemm_acc(Ap, Bp), want)
    assert np.array_equal(orc.gemm_s4s4_i32(Ap, Bp), want.astype(np.int32))
    if M * N * K <= 20000:
        assert orc.gemm_acc(Ap, Bp).tolist() == _bigint_gemm(_decode(Ap).tolist(),
                                                             _decode(Bp).tolist())


@pytest.mark.parametrize("M,N,K", [(3, 4, 6), (16, 48, 64), (9, 31, 130)])
def test_s8s4_vs_numpy(orc, M, N, K):
    g = np.random.default_rng(K * 11 + N)
    A = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    Bp = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    want = A.astype(np.int64) @ _decode(Bp).T
    assert np.array_equal(orc.gemm_acc(A, Bp), want)


def test_closed_forms(orc):
    K = 96
    # all -8 x all -8 (code 0x88) -> 64 K
    a = np.full((3, K // 2), 0x88, np.uint8)
    assert np.all(orc.gemm_s4s4_i32(a, a) == 64 * K)
    # all 7 x all -8 -> -56 K
    b = np.full((5, K // 2), 0x77, np.uint8)
    assert np.all(orc.gemm_s4s4_i32(b, a) == -56 * K)
    # int8 127 x 127 and -127 x 127
    p = np.full((2, K), 127, np.int8)
    n = np.full((4, K), -127, np.int8)
    assert np.all(orc.gemm_acc(p, p) == 16129 * K)
    assert np.all(orc.gemm_acc(n, p) == -16129 * K)
    # -128 x -128 is the largest int8 product
    q = np.full((1, K), -128, np.int8)
    assert np.all(orc.gemm_acc(q, q) == 16384 * K)


def test_identity_operand(orc):
    g = np.random.default_rng(1)
    A = g.integers(-128, 128, size=(12, 32), dtype=np.int8)
    I = np.eye(32, dtype=np.int8)
    assert np.array_equal(orc.gemm_acc(A, I), A.astype(np.int64))
    # an int4 identity: element k of row n is 1 iff k == n
    Ip = np.zeros((32, 16), np.uint8)
    for n in range(32):
        Ip[n, n // 2] = 0x01 if n % 2 == 0 else 0x10
    assert np.array_equal(orc.gemm_acc(A, Ip), A.astype(np.int64))


def test_row_selection(orc):
    d = datagen.gemm_s8s8(50, 20, 48, seed=9)
    full = orc.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    rows = [49, 0, 17, 17]
    part = orc.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
    assert np.array_equal(part, full[rows])


def _requant_table(orc, acc, bias, mult, shift):
    M, N = acc.shape
    out = np.empty((M, N), np.int8)
    for m in range(M):
        for n in range(N):
            b = 0 if bias is None else int(bias[n])
            out[m, n] = orc.requant(int(acc[m, n]), b, int(mult[n]), int(shift[n]))
    return out


@pytest.mark.parametrize("unsat", [False, True])
def test_s8s8_requant_composition(orc, unsat):
    shift = (38, 44) if unsat else (31, 40)
    d = datagen.gemm_s8s8(40, 24, 64, seed=5, shift=shift)
    acc = d["A"].astype(np.int64) @ d["B"].astype(np.int64).T
    want = _requant_table(orc, acc, d["bias"], d["mult"], d["shift"])
    got = orc.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(got, want)
    if unsat:
        assert np.mean(np.abs(got.astype(int)) < 127) > 0.5
    # bias None means zero bias
    got0 = orc.gemm_s8s8_requant(d["A"], d["B"], None, d["mult"], d["shift"])
    assert np.array_equal(got0, _requant_table(orc, acc, None, d["mult"], d["shift"]))


def test_w4a8_requant_composition(orc):
    d = datagen.gemm_w4a8(16, 40, 128, seed=4, shift=(37, 43))
    acc = d["A"].astype(np.int64) @ _decode(d["B"]).T
    want = _requant_table(orc, acc, d["bias"], d["mult"], d["shift"])
    assert np.array_equal(orc.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"],
                                                d["shift"]), want)


def test_requant_reports_an_accumulator_past_int32(orc):
    """The accumulator is an int32: one past its range is an error even when
    the bias would bring the sum back inside (all -128 x -128 rows give
    16384 K; all -128 x -8 give 1024 K)."""
    mult = np.array([1 << 30], np.int32)
    shift = np.array([31], np.int32)
    bias = np.array([-(1 << 30)], np.int32)
    for K, bad in ((130000, False), (140000, True)):      # 2.13e9 fits, 2.29e9 does not
        a = np.full((1, K), -128, np.int8)
        if bad:
            with pytest.raises(orc.OracleDomainError):
                orc.gemm_s8s8_requant(a, a, bias, mult, shift)
        else:
            y = orc.gemm_s8s8_requant(a, a, bias, mult, shift)
            assert y[0, 0] == 127          # (2129920000 - 2^30) / 2 saturates
    for K, bad in ((2096000, False), (2098000, True)):     # 2^31 / 1024 = 2097152
        a = np.full((1, K), -128, np.int8)
        b = np.full((1, K // 2), 0x88, np.uint8)            # -8 in either nibble order
        for msb in (False, True):
            if bad:
                with pytest.raises(orc.OracleDomainError):
                    orc.gemm_w4a8_requant(a, b, bias, mult, shift, msb_first=msb)
            else:
                assert orc.gemm_w4a8_requant(a, b, bias, mult, shift, msb_first=msb)[0, 0] == 127


def test_s4s4_range_error(orc):
    # an int32 overflow of the raw output is reported, not wrapped
    K = 2 ** 26  # 64 * 2^26 = 2^32 > int32
    a = np.full((1, K // 2), 0x88, np.uint8)
    with pytest.raises(orc.OracleDomainError):
        orc.gemm_s4s4_i32(a, a)

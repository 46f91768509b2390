"""Parity of qgemm_s4s4_f16 (packed int4 x packed int4, binary16 output)
with the oracle, bit for bit.

Both sides take the same steps in IEEE binary32 (the accumulator converted
exactly, times the row scale, times the column scale) and round to binary16
to nearest even, so the results are unique.  Shapes cover the tile kernel
(small and ragged, unaligned output stride) and the direct-to-LDS ring
kernel (4096^3, sampled rows), with and without scales, and the binary16
overflow point.
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


def _scales(g, n):
    return g.uniform(1e-4, 4e-3, n).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (7, 5, 64), (33, 17, 96), (129, 65, 288),
                                   (300, 260, 512), (2048, 4096, 640), (4096, 4096, 4096)])
@pytest.mark.parametrize("scaled", [False, True])
def test_s4s4_f16(qg, orc, M, N, K, scaled):
    print("s4s4 f16", M, N, K, scaled, flush=True)
    d = datagen.gemm_s4s4(M, N, K, seed=M + N + K)
    g = np.random.default_rng(M + 1)
    sa = _scales(g, M) if scaled else None
    sb = _scales(g, N) if scaled else None
    C = qg.qgemm_s4s4_f16(dev(d["A"]), dev(d["B"]), None if sa is None else dev(sa),
                          None if sb is None else dev(sb))
    # large shapes take the ring kernel (K = 640: five 64-byte stages, one at
    # a time; K = 4096: paired stages): 64 rows, every offset inside a 16-row
    # block and both row halves of a 256-row tile, the last row included
    rows = None if M <= 512 else np.unique(np.concatenate([
        np.arange(16) * 17 % 256 + 256 * np.arange(16) % M,
        np.random.default_rng(K).integers(0, M, 47), [M - 1]]))
    want = orc.gemm_s4s4_f16(d["A"], d["B"], sa, sb, rows=rows)
    got = C.cpu().numpy()
    got = got if rows is None else got[rows]
    bad = np.argwhere(got.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, f"{len(bad)} values differ, first at {bad[0].tolist()}"


def test_s4s4_f16_one_scale_and_strided_output(qg, orc):
    d = datagen.gemm_s4s4(70, 45, 160, seed=5)
    sa = _scales(np.random.default_rng(6), 70)
    Cw = torch.full((70, 51), 7.0, dtype=torch.float16, device="cuda")
    qg.qgemm_s4s4_f16(dev(d["A"]), dev(d["B"]), dev(sa), None, C=Cw[:, :45])
    want = orc.gemm_s4s4_f16(d["A"], d["B"], sa, None)
    got = Cw.cpu().numpy()
    assert np.array_equal(got[:, :45].view(np.uint16), want.view(np.uint16))
    assert np.all(got[:, 45:] == 7.0)


def test_s4s4_f16_overflow_and_sign(qg, orc):
    """All -8 x -8: 64 K per output; K = 1024 overflows binary16 to +inf, a
    negative scale to -inf; K = 992 stays finite."""
    for K in (992, 1024):
        A = np.full((64, K // 2), 0x88, np.uint8)
        sa = np.where(np.arange(64) % 2 == 0, 1.0, -1.0).astype(np.float32)
        C = qg.qgemm_s4s4_f16(dev(A), dev(A), dev(sa), None)
        want = orc.gemm_s4s4_f16(A, A, sa, None)
        assert np.array_equal(C.cpu().numpy().view(np.uint16), want.view(np.uint16))

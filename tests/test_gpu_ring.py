"""Parity of the persistent direct-to-LDS ring kernel's tile walk.

One workgroup per compute unit walks its tiles, and the operand ring runs
from one tile's last K stages straight into the next tile's first ones.  The
cases here stress what that walk adds, for every epilogue the ring kernel
has (int8 requantize at both shift tiers, asymmetric requantize, raw int32,
binary16, W4A8 with either nibble order):
  * more tiles than compute units, with a ragged last round (some workgroups
    take one tile more than others);
  * M and N that are not multiples of 256, so the bottom and right edge
    tiles are moved inward and overlap their neighbours;
  * K at the ring's minimum (one ring of stages per tile) and just above it;
  * strided operands, no bias, and output row strides with and without the
    16-byte alignment the vector stores need.
Every row of the bottom edge tile and of its neighbour is compared, with a
random sample of the rest, all bit for bit with the oracle.
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


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _say(*a):
    print(*a, flush=True)


def _rows(M, seed, n=24):
    """The last 2 x 256 rows (the inward edge tile and the tile it
    overlaps), rows on both sides of each 256-row boundary in a sample, and
    random rows."""
    g = np.random.default_rng(seed)
    rows = set(range(max(M - 512, 0), M))
    for b in g.choice(np.arange(256, M, 256), size=min(6, (M - 1) // 256), replace=False):
        rows |= {int(b) - 1, int(b)}
    rows |= set(g.choice(M, size=min(n, M), replace=False).tolist())
    rows |= {0, 1}
    return np.array(sorted(rows), dtype=np.int64)


# (M, N, K): > 256 tiles with a ragged last round and both edges ragged;
# K at the int8 ring's minimum (4 stages of 64) and one stage above it; a
# shape whose M is a multiple of 256 with a ragged N only
S8_RING = [(4100, 4400, 256), (4352, 4130, 320), (2304, 7990, 1024)]


@pytest.mark.parametrize("M,N,K", S8_RING)
@pytest.mark.parametrize("unsat", [False, True])
def test_s8s8_ring_walk(qg, orc, M, N, K, unsat):
    _say("s8s8 ring walk", M, N, K, unsat)
    d = datagen.gemm_s8s8(M, N, K, seed=M + K, shift=(36, 42) if unsat else (29, 40))
    C = host(qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"])))
    rows = _rows(M, K)
    want = orc.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
    assert np.array_equal(C[rows], want)


@pytest.mark.parametrize("M,N,K", [(4100, 4400, 256), (2304, 7990, 1024)])
def test_s8s8_zp_ring_walk(qg, orc, M, N, K):
    _say("s8s8 zp ring walk", M, N, K)
    d = datagen.gemm_s8s8(M, N, K, seed=M + K + 1, shift=(37, 43))
    za, zb, zo = -9, 5, 13
    C = host(qg.qgemm_s8s8_requant_zp(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                      dev(d["shift"]), za, zb, zo, act=(-100, 120)))
    rows = _rows(M, K + 1)
    want = orc.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"], za, zb,
                                    zo, rows=rows, act=(-100, 120))
    assert np.array_equal(C[rows], want)


# int4 x int4: K at the ring's minimum (4 stages of 128 values) and above
S4_RING = [(4100, 4400, 512), (2304, 4130, 1152)]


@pytest.mark.parametrize("M,N,K", S4_RING)
def test_s4s4_i32_ring_walk(qg, orc, M, N, K):
    _say("s4s4 i32 ring walk", M, N, K)
    d = datagen.gemm_s4s4(M, N, K, seed=M + K)
    C = host(qg.qgemm_s4s4_i32(dev(d["A"]), dev(d["B"])))
    rows = _rows(M, K)
    want = orc.gemm_s4s4_i32(d["A"], d["B"], rows=rows)
    assert np.array_equal(C[rows], want)


@pytest.mark.parametrize("M,N,K", S4_RING)
@pytest.mark.parametrize("scaled", [False, True])
def test_s4s4_f16_ring_walk(qg, orc, M, N, K, scaled):
    _say("s4s4 f16 ring walk", M, N, K, scaled)
    d = datagen.gemm_s4s4(M, N, K, seed=M + K + 2)
    g = np.random.default_rng(K)
    sa = g.uniform(1e-4, 4e-3, M).astype(np.float32) if scaled else None
    sb = g.uniform(1e-4, 4e-3, N).astype(np.float32) if scaled else None
    C = host(qg.qgemm_s4s4_f16(dev(d["A"]), dev(d["B"]), None if sa is None else dev(sa),
                               None if sb is None else dev(sb)))
    rows = _rows(M, K + 2)
    want = orc.gemm_s4s4_f16(d["A"], d["B"], sa, sb, rows=rows)
    assert np.array_equal(C[rows].view(np.uint16), want.view(np.uint16))


# int8 x int4: K at the ring's minimum (3 stages of 128 values) and above
@pytest.mark.parametrize("M,N,K", [(4100, 4400, 384), (2304, 4130, 896)])
@pytest.mark.parametrize("msb", [False, True])
def test_w4a8_ring_walk(qg, orc, M, N, K, msb):
    _say("w4a8 ring walk", M, N, K, msb)
    d = datagen.gemm_w4a8(M, N, K, seed=M + K + 3, shift=(37, 43))
    C = host(qg.qgemm_w4a8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                                   dev(d["shift"]), msb_first=msb))
    rows = _rows(M, K + 3)
    want = orc.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows,
                                 msb_first=msb)
    assert np.array_equal(C[rows], want)


# strided operands, no bias, and output row strides that do (ldc % 16 == 0)
# and do not allow the 16-byte stores
@pytest.mark.parametrize("ldc_extra", [16, 3])
def test_s8s8_ring_walk_strided(qg, orc, ldc_extra):
    M, N, K = 4100, 4400, 320
    _say("s8s8 ring walk strided", M, N, K, ldc_extra)
    d = datagen.gemm_s8s8(M, N, K, seed=9 + ldc_extra, shift=(36, 42))
    Aw = np.zeros((M, K + 64), np.int8)
    Aw[:, :K] = d["A"]
    Bw = np.zeros((N, K + 32), np.int8)
    Bw[:, :K] = d["B"]
    At, Bt = dev(Aw), dev(Bw)
    Cw = torch.full((M, N + ldc_extra), 99, dtype=torch.int8, device="cuda")
    qg.qgemm_s8s8_requant(At[:, :K], Bt[:, :K], None, dev(d["mult"]), dev(d["shift"]),
                          C=Cw[:, :N])
    got = host(Cw)
    rows = _rows(M, ldc_extra)
    want = orc.gemm_s8s8_requant(d["A"], d["B"], None, d["mult"], d["shift"], rows=rows)
    assert np.array_equal(got[rows, :N], want)
    assert np.all(got[:, N:] == 99)  # nothing written past N


@pytest.mark.parametrize("ldc_extra", [4, 1])
def test_s4s4_ring_walk_output_stride(qg, orc, ldc_extra):
    M, N, K = 2304, 4130, 512
    _say("s4s4 ring walk output stride", M, N, K, ldc_extra)
    d = datagen.gemm_s4s4(M, N, K, seed=21 + ldc_extra)
    Ci = torch.full((M, N + ldc_extra), -7, dtype=torch.int32, device="cuda")
    qg.qgemm_s4s4_i32(dev(d["A"]), dev(d["B"]), C=Ci[:, :N])
    Ch = torch.full((M, N + ldc_extra), -1.0, dtype=torch.float16, device="cuda")
    qg.qgemm_s4s4_f16(dev(d["A"]), dev(d["B"]), None, None, C=Ch[:, :N])
    gi, gh = host(Ci), host(Ch)
    rows = _rows(M, ldc_extra + 1)
    assert np.array_equal(gi[rows, :N], orc.gemm_s4s4_i32(d["A"], d["B"], rows=rows))
    assert np.all(gi[:, N:] == -7)
    want_h = orc.gemm_s4s4_f16(d["A"], d["B"], None, None, rows=rows)
    assert np.array_equal(gh[rows, :N].view(np.uint16), want_h.view(np.uint16))
    assert np.all(gh[:, N:] == -1.0)


def test_s8s8_ring_walk_edge_tile_unaligned_column(qg, orc):
    """A 16-byte-multiple output stride (4112) with N = 4100: the right edge
    tile starts at column N - 256 = 3844, which is not on 16 bytes, so that
    tile must take the narrow stores while the others keep the 16-byte ones."""
    M, N, K, ldc = 2304, 4100, 256, 4112
    _say("s8s8 ring walk unaligned edge column", M, N, K, ldc)
    d = datagen.gemm_s8s8(M, N, K, seed=41, shift=(36, 42))
    Cw = torch.full((M, ldc), 99, dtype=torch.int8, device="cuda")
    qg.qgemm_s8s8_requant(dev(d["A"]), dev(d["B"]), dev(d["bias"]), dev(d["mult"]),
                          dev(d["shift"]), C=Cw[:, :N])
    got = host(Cw)
    rows = _rows(M, 41)
    want = orc.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
    assert np.array_equal(got[rows, :N], want)
    assert np.all(got[:, N:] == 99)


def test_s4s4_ring_walk_edge_tile_unaligned_column(qg, orc):
    """int32 and binary16 outputs with a 4-element-multiple stride (4132) and
    N = 4130: the right edge tile starts at column 3874, off the 16-byte
    (int32) and 8-byte (binary16) alignment of its 4-column stores."""
    M, N, K, ldc = 2304, 4130, 512, 4132
    _say("s4s4 ring walk unaligned edge column", M, N, K, ldc)
    d = datagen.gemm_s4s4(M, N, K, seed=43)
    Ci = torch.full((M, ldc), -7, dtype=torch.int32, device="cuda")
    qg.qgemm_s4s4_i32(dev(d["A"]), dev(d["B"]), C=Ci[:, :N])
    Ch = torch.full((M, ldc), -1.0, dtype=torch.float16, device="cuda")
    qg.qgemm_s4s4_f16(dev(d["A"]), dev(d["B"]), None, None, C=Ch[:, :N])
    gi, gh = host(Ci), host(Ch)
    rows = _rows(M, 43)
    assert np.array_equal(gi[rows, :N], orc.gemm_s4s4_i32(d["A"], d["B"], rows=rows))
    assert np.all(gi[:, N:] == -7)
    want_h = orc.gemm_s4s4_f16(d["A"], d["B"], None, None, rows=rows)
    assert np.array_equal(gh[rows, :N].view(np.uint16), want_h.view(np.uint16))
    assert np.all(gh[:, N:] == -1.0)

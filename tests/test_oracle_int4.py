"""Pins of the oracle's packed-INT4 decode (exhaustive) and the INT4 GEMM
"hello world" of the DeepGEMM INT4 article (www.cf-1.com/news/6060138) §3.2."""
import numpy as np

from conftest import read_golden


def _numpy_decode(byte_vals):
    """Independent decode: let numpy's int8 two's complement sign-extend each
    nibble by placing it in the top half of a byte and shifting back."""
    b = np.asarray(byte_vals, dtype=np.uint8)
    lo = (b << 4).astype(np.uint8).view(np.int8) >> 4
    hi = b.view(np.int8) >> 4
    return lo.astype(np.int64), hi.astype(np.int64)


def test_codes_table(orc):
    rows = read_golden("int4_codes.txt")
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s, 16), int(val_s)
        # code in the low nibble -> element 0, in the high nibble -> element 1
        assert orc.int4_at(np.array([code], np.uint8), 0) == val
        assert orc.int4_at(np.array([code << 4], np.uint8), 1) == val
        # the other nibble of the byte is then 0
        assert orc.int4_at(np.array([code], np.uint8), 1) == 0
        assert orc.int4_at(np.array([code << 4], np.uint8), 0) == 0


def test_exhaustive_256_bytes(orc):
    allb = np.arange(256, dtype=np.uint8)
    lo, hi = _numpy_decode(allb)
    for b in range(256):
        assert orc.int4_at(allb[b:b + 1], 0) == lo[b]
        assert orc.int4_at(allb[b:b + 1], 1) == hi[b]
    # element i of a long row reads byte i // 2
    got = [orc.int4_at(allb, i) for i in range(512)]
    want = np.stack([lo, hi], axis=1).reshape(-1)
    assert np.array_equal(np.array(got), want)


def test_specific_bytes(orc):
    cases = {0x08: (-8, 0), 0x80: (0, -8), 0xF7: (7, -1), 0x7F: (-1, 7), 0x11: (1, 1),
             0x22: (2, 2), 0x88: (-8, -8), 0x00: (0, 0), 0xFF: (-1, -1)}
    for b, (e0, e1) in cases.items():
        row = np.array([b], np.uint8)
        assert (orc.int4_at(row, 0), orc.int4_at(row, 1)) == (e0, e1), hex(b)


def test_hello_world_corrected(orc):
    (M, K, N, ba, bb, want), = read_golden("int4_hello_world.txt")
    M, K, N, want = int(M), int(K), int(N), int(want)
    A = np.full((M, K // 2), int(ba, 16), np.uint8)
    B = np.full((N, K // 2), int(bb, 16), np.uint8)
    C = orc.gemm_s4s4_i32(A, B)
    assert C.shape == (M, N)
    assert np.all(C == want)
    assert want != 2048  # the page's printed value is not reproduced
    acc = orc.gemm_acc(A, B)
    assert np.all(acc == want)

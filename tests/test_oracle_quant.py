"""Pins of the oracle's per-token activation quantizer.

Definition (Ascend FlatQuant operator article, www.zwxr.cn/news/277566,
«per-token 模式»: per token, scale = max|x| / (qmax / clip_ratio) and codes
from x / scale; Voyager quantization article, www.dpshk.com/news/2695434,
§1.1: Q = round(x / scale) + zero_point with round half away from zero).
The codes are decided in IEEE binary32 (the GPU kernel's precision).

The pins: hand-worked tokens, exact ties, clipping, the invariants the
definition implies (sign symmetry, the largest value maps to +-qmax, power-of-
two scaling, monotonicity, the half-step error bound), the float16 / bfloat16
conversions against numpy and torch, and the packed-int4 layout against the
oracle's own int4 decoder.
"""
import numpy as np
import pytest


def test_hand_worked_int8(orc):
    # token 0: max|x| = 127 -> scale 1 exactly; 2.5 is a tie -> 3
    # token 1: all zero -> scale 0, codes 0
    # token 2: max|x| = 2.5 -> scale 2.5/127; 0.5 -> 25.4 -> 25, 1.5 -> 76.2 -> 76
    X = np.array([[1.0, -2.0, 2.5, 127.0],
                  [0.0, 0.0, 0.0, 0.0],
                  [0.5, -0.5, 1.5, -2.5]], np.float32)
    Q, s = orc.quant_per_token(X, bits=8)
    assert np.array_equal(Q, [[1, -2, 3, 127], [0, 0, 0, 0], [25, -25, 76, -127]])
    assert s[0] == 1.0 and s[1] == 0.0 and s[2] == np.float32(2.5) / np.float32(127.0)


def test_hand_worked_int4(orc):
    # token: max|x| = 2.5 -> scale 2.5/7; codes 1.4 -> 1, -1.4 -> -1, 4.2 -> 4, -7
    X = np.array([[0.5, -0.5, 1.5, -2.5]], np.float32)
    Q, s = orc.quant_per_token(X, bits=4)
    # low nibble = even index: bytes (1 | -1 << 4) and (4 | -7 << 4)
    assert Q.tolist() == [[0xF1, 0x94]]
    assert s[0] == np.float32(2.5) / np.float32(7.0)


@pytest.mark.parametrize("bits,qmax", [(8, 127), (4, 7)])
def test_ties_round_away_from_zero(orc, bits, qmax):
    # max|x| = qmax makes the scale exactly 1, so x / scale = x
    ties = [0.5, 1.5, 2.5, qmax - 0.5]
    X = np.array([[qmax] + ties + [-t for t in ties] + [0.0]], np.float32)
    Q, s = orc.quant_per_token(X, bits=bits)
    assert s[0] == 1.0
    codes = Q[0].tolist() if bits == 8 else [orc.int4_at(Q[0], k) for k in range(X.shape[1])]
    want = [qmax] + [int(t + 0.5) for t in ties] + [-int(t + 0.5) for t in ties] + [0]
    assert codes == want


def test_clip_ratio_clamps(orc):
    # clip 0.5 doubles the code range before the clamp: max|x| maps to 254 -> 127
    X = np.array([[-100.0, 10.0, 50.0, 100.0]], np.float32)
    Q, s = orc.quant_per_token(X, bits=8, clip_ratio=0.5)
    assert s[0] == np.float32(100.0) / (np.float32(127.0) / np.float32(0.5))
    assert Q[0].tolist() == [-127, 25, 127, 127]
    Q4, _ = orc.quant_per_token(X, bits=4, clip_ratio=0.5)
    codes = [orc.int4_at(Q4[0], i) for i in range(4)]
    assert codes == [-7, 1, 7, 7]
    # a tiny clip ratio puts x / scale far past 2^31: every nonzero code clamps
    Xt = np.array([[1e-3, -1.0, 0.0, 1.0]], np.float32)
    Qt, _ = orc.quant_per_token(Xt, bits=8, clip_ratio=1e-20)
    assert Qt[0].tolist() == [127, -127, 0, 127]


def _random_tokens(g, M, K):
    X = g.standard_normal((M, K)).astype(np.float32) * g.uniform(0.01, 100, (M, 1)).astype(
        np.float32)
    X[0] = 0.0
    return X


def test_invariants_int8(orc):
    g = np.random.default_rng(3)
    X = _random_tokens(g, 40, 256)
    Q, s = orc.quant_per_token(X, bits=8)
    Qn, sn = orc.quant_per_token(-X, bits=8)
    assert np.array_equal(Qn, -Q) and np.array_equal(sn, s)      # sign symmetry
    assert np.all(np.abs(Q[1:]).max(axis=1) == 127)                # the largest value -> 127
    assert np.all(Q[0] == 0) and s[0] == 0.0
    Q8, s8 = orc.quant_per_token(X * np.float32(8.0), bits=8)     # power-of-two scaling
    assert np.array_equal(Q8, Q) and np.array_equal(s8, s * np.float32(8.0))
    for m in range(1, 40):                                         # monotone within a token
        order = np.argsort(X[m], kind="stable")
        assert np.all(np.diff(Q[m][order].astype(int)) >= 0)
    err = np.abs(X[1:] - Q[1:].astype(np.float64) * s[1:, None])  # half-step error bound
    assert np.all(err <= 0.5 * s[1:, None] * (1 + 1e-5))


def test_int4_layout_and_bound(orc):
    g = np.random.default_rng(4)
    X = _random_tokens(g, 9, 64)
    Q4, s4 = orc.quant_per_token(X, bits=4)
    codes = np.array([[orc.int4_at(Q4[m], k) for k in range(64)] for m in range(9)])
    assert codes.min() >= -7 and codes.max() <= 7
    assert np.all(np.abs(codes[1:]).max(axis=1) == 7)
    err = np.abs(X[1:] - codes[1:] * s4[1:, None].astype(np.float64))
    assert np.all(err <= 0.5 * s4[1:, None] * (1 + 1e-5))


def test_half_and_bfloat_inputs(orc):
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(5)
    X = _random_tokens(g, 12, 128)
    h = X.astype(np.float16)
    Qh, sh = orc.quant_per_token(h, bits=8)
    Qf, sf = orc.quant_per_token(h.astype(np.float32), bits=8)   # numpy's exact widening
    assert np.array_equal(Qh, Qf) and np.array_equal(sh, sf)
    bf = torch.from_numpy(X).to(torch.bfloat16)
    bits_u16 = bf.view(torch.int16).numpy().view(np.uint16)
    Qb, sb = orc.quant_per_token(bits_u16, bits=8, dtype="bfloat16")
    Qw, sw = orc.quant_per_token(bf.float().numpy(), bits=8)       # torch's widening
    assert np.array_equal(Qb, Qw) and np.array_equal(sb, sw)
    for v in [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0xC000, 0x7BFF, 0xFBFF]:
        assert orc.f16_to_f32(v) == float(np.array([v], np.uint16).view(np.float16)[0])


def test_domain(orc):
    X = np.ones((2, 4), np.float32)
    with pytest.raises(orc.OracleDomainError):
        orc.quant_per_token(X, bits=8, clip_ratio=0.0)

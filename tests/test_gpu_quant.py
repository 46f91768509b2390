"""Parity of the per-token activation quantizer's HIP kernel with the oracle.

Codes are compared byte for byte and scales bit for bit: both sides decide
every code in IEEE binary32, so the results are unique.  The cases span the
kernel's register-resident row lengths and the longer rows it streams twice,
every input type (binary32, binary16, bfloat16) and both code widths, strided
rows, zero and degenerate tokens, scales outside the range where the kernel
multiplies by a reciprocal, and inputs built to sit on or next to a rounding
tie.  The full activation workload (8192 tokens x 8192 channels, bfloat16)
is checked in full.
"""
import numpy as np
import pytest

from conv_qgemm_amd import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TORCH_DT = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}
NP_DT = {"float32": np.float32, "float16": np.float16}


@pytest.fixture(scope="module")
def qg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conv_qgemm_amd import qgemm
    return qgemm


def _say(*a):
    print(*a, flush=True)


def _as_type(X32, dtype):
    """(device tensor of dtype, the same values as the oracle takes them).
    The narrowing to 16 bits is torch's round-to-nearest-even; the oracle
    gets the resulting bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(X32)).to(TORCH_DT[dtype])
    if dtype == "bfloat16":
        h = t.view(torch.int16).numpy().view(np.uint16)
    else:
        h = t.numpy()
    return t, h


def _check(qg, orc, X32, dtype, bits, clip=1.0, ldx_pad=0, ldq_pad=0):
    M, K = X32.shape
    t, h = _as_type(X32, dtype)
    if ldx_pad:
        wide = torch.zeros((M, K + ldx_pad), dtype=t.dtype)
        wide[:, :K] = t
        Xd = wide.cuda()[:, :K]
    else:
        Xd = t.cuda()
    qcols = K if bits == 8 else K // 2
    qdt = torch.int8 if bits == 8 else torch.uint8
    Qfull = torch.full((M, qcols + ldq_pad), 0x5A, dtype=qdt, device="cuda")
    Qd = Qfull[:, :qcols]
    sd = torch.full((M + 1,), -1.0, dtype=torch.float32, device="cuda")
    qg.qquant_per_token(Xd, bits=bits, clip_ratio=clip, Q=Qd, scale=sd)
    torch.cuda.synchronize()
    Qw, sw = orc.quant_per_token(h, bits=bits, clip_ratio=clip, dtype=dtype)
    Qg = Qfull.cpu().numpy()
    sg = sd.cpu().numpy()
    bad = np.argwhere(Qg[:, :qcols].view(np.uint8) != Qw.view(np.uint8))
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[0].tolist()}"
    assert np.array_equal(sg[:M].view(np.uint32), sw.view(np.uint32)), "scales differ"
    assert sg[M] == -1.0, "wrote past the scale vector"
    if ldq_pad:
        assert np.all(Qg[:, qcols:].view(np.uint8) == 0x5A), "wrote past the row's codes"


# (M, K) across the kernel's launch shapes (16-byte vectors per row: K / 4
# for binary32, K / 8 for the 16-bit types): one, two or four waves per row,
# 1 to 16 vectors per thread in registers, rows streamed twice past that
# (K 16400 streams binary32, K 32784 every type), and row counts that leave
# a workgroup partly empty
SHAPES = [(1, 16), (3, 48), (7, 208), (5, 1024), (33, 1040), (129, 272), (64, 2064),
          (5, 4112), (3, 8192), (2, 8208), (2, 16384), (3, 16400), (2, 32784)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_quant_shapes(qg, orc, dtype, bits, M, K):
    _say("quant", dtype, bits, M, K)
    X = datagen.activations(M, K, seed=M * 7 + K)
    _check(qg, orc, X, dtype, bits)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("clip", [0.9, 0.5, 0.125])
def test_quant_clip(qg, orc, dtype, bits, clip):
    _say("quant clip", dtype, bits, clip)
    X = datagen.activations(37, 640, seed=11)
    _check(qg, orc, X, dtype, bits, clip=clip)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("bits", [8, 4])
def test_quant_strided(qg, orc, dtype, bits):
    _say("quant strided", dtype, bits)
    X = datagen.activations(19, 528, seed=12)
    _check(qg, orc, X, dtype, bits, ldx_pad=48, ldq_pad=32)


def _special_rows(K):
    g = np.random.default_rng(13)
    rows = []
    rows.append(np.zeros(K))                                  # all zero: scale 0, codes 0
    z = np.zeros(K); z[K // 3] = -3.0; rows.append(z)         # one nonzero
    n = -np.zeros(K); rows.append(n)                          # negative zeros
    rows.append(g.standard_normal(K) * 1e-40)                 # binary32 subnormals
    rows.append(g.standard_normal(K) * 1e-31)                 # scale below 2^-100
    rows.append(g.standard_normal(K) * 1e35)                  # scale above 2^100
    rows.append(g.standard_normal(K) * 3e38 / 5)              # near the binary32 maximum
    c = np.full(K, 2.5); c[::2] = -2.5; rows.append(c)        # constant magnitude
    s = g.standard_normal(K); s[5] = 1e6; rows.append(s)      # one huge outlier
    rows.append(g.standard_normal(K) * 6e-8)                  # binary16 subnormal range
    rows.append(np.clip(g.standard_normal(K) * 3e4, -65504, 65504))  # binary16 maximum
    return np.array(rows)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("bits", [8, 4])
def test_quant_special_values(qg, orc, dtype, bits):
    _say("quant special", dtype, bits)
    X = _special_rows(96)
    if dtype == "float16":
        X = np.clip(X, -65504, 65504)
    with np.errstate(over="ignore", under="ignore"):
        _check(qg, orc, X.astype(np.float32), dtype, bits)


def _near_tie_rows(K, qmax, clip, seed):
    """Rows whose first element sets max|x| = A, the rest sitting on (n + 1/2)
    times the binary32 scale the definition gives for A, and on the floats
    next to those, so that x / scale lies on or next to a rounding tie."""
    g = np.random.default_rng(seed)
    rows = []
    for _ in range(8):
        A = np.float32(2.0 ** g.uniform(-20, 20))
        sc = A / (np.float32(qmax) / np.float32(clip))
        n = g.integers(0, qmax, size=K - 1).astype(np.float32)
        v = (n + np.float32(0.5)) * sc
        step = g.integers(-2, 3, size=K - 1)
        for _ in range(2):
            v = np.where(step > 0, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(step < 0, np.nextafter(v, np.float32(-np.inf)), v)
            step = step - np.sign(step)
        v = np.where(g.integers(0, 2, size=K - 1) == 1, -v, v).astype(np.float32)
        rows.append(np.concatenate([[A], v]).astype(np.float32))
    # x / scale at distances of 2^-17 .. 2^-12 from a half-integer, on both
    # sides of the window inside which the kernel divides exactly
    for _ in range(4):
        A = np.float32(2.0 ** g.uniform(-20, 20))
        sc = A / (np.float32(qmax) / np.float32(clip))
        n = g.integers(0, qmax, size=K - 1)
        d = 2.0 ** g.integers(-17, -11, size=K - 1) * g.choice([-1.0, 1.0], size=K - 1)
        v = ((n + 0.5 + d) * np.float64(sc)).astype(np.float32)
        v = np.where(g.integers(0, 2, size=K - 1) == 1, -v, v)
        rows.append(np.concatenate([[A], np.minimum(np.abs(v), A) * np.sign(v)]))
    # scales that are exact: A = qmax (scale 1) and A = 2 qmax (scale 2)
    for A in (qmax, 2 * qmax):
        t = np.arange(K - 1) % qmax + 0.5
        rows.append(np.concatenate([[A], t * (A // qmax) * np.where(np.arange(K - 1) % 2, -1, 1)]))
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("bits,qmax", [(8, 127), (4, 7)])
@pytest.mark.parametrize("clip", [1.0, 0.75])
def test_quant_near_ties(qg, orc, bits, qmax, clip):
    _say("quant near ties", bits, clip)
    X = _near_tie_rows(1024, qmax, clip, seed=bits * 10 + int(clip * 4))
    if clip != 1.0:
        X = X[:12]  # the exact-scale rows assume clip 1
    _check(qg, orc, X, "float32", bits, clip=clip)


def test_quant_feeds_s8s8(qg, orc):
    """Codes written by the quantizer go straight into the GEMM's A operand
    on the same stream; the chain equals the oracle's chain."""
    _say("quant -> s8s8")
    X = datagen.activations(70, 256, seed=14)
    t, h = _as_type(X, "bfloat16")
    d = datagen.gemm_s8s8(70, 96, 256, seed=15, shift=(36, 42))
    Q, _ = qg.qquant_per_token(t.cuda(), bits=8)
    dv = {k: torch.from_numpy(d[k]).cuda() for k in ("B", "bias", "mult", "shift")}
    C = qg.qgemm_s8s8_requant(Q, dv["B"], dv["bias"], dv["mult"], dv["shift"])
    torch.cuda.synchronize()
    Qw, _ = orc.quant_per_token(h, bits=8, dtype="bfloat16")
    want = orc.gemm_s8s8_requant(Qw, d["B"], d["bias"], d["mult"], d["shift"])
    assert np.array_equal(C.cpu().numpy(), want)


@pytest.mark.parametrize("bits", [8, 4])
def test_workload_quant_a8_full(qg, orc, bits):
    """The 8192 x 8192 bfloat16 activation workload, every code and scale."""
    w = datagen.WORKLOADS["quant_a8"]
    _say("quant workload", w["M"], w["K"], bits)
    X = datagen.workload("quant_a8")["X"]
    _check(qg, orc, X, w["dtype"], bits)

"""The allocation-free asymmetric GEMM (qgemm_s8s8_requant_zp_noalloc)
against the workspace form (qgemm_s8s8_requant_zp) on the same inputs, bit
for bit, on two calls in a row, the second smaller than the first: the
library's per-GPU scratch array keeps the first call's compensation sums, and
the second call must not read any of them.  Both are checked against the
oracle too.  Zero points as the Voyager quantization article
(www.dpshk.com/news/2695434) §1.1 defines them; requantize of the MCU conv
front-end article (news.rkmt.cn/news/16638) §2.3."""
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


def _say(*a):
    print(*a, flush=True)


# (M, N, K, a_zero, b_zero, out_zero, act): the first is the ring kernel
# (>= 128 tiles of 256 x 256), the second the tile kernel, smaller in every
# dimension; the third has b_zero = 0 (no per-row sums)
CALLS = [
    (2304, 4100, 320, -11, 6, 20, (-128, 127)),
    (300, 260, 64, 7, -3, -5, (-5, 127)),
    (96, 80, 128, 12, 0, 4, (-128, 100)),
]


def _one(qg, M, N, K, za, zb, zo, act, seed):
    d = datagen.gemm_s8s8(M, N, K, seed=seed, shift=(36, 42))
    args = [dev(d[k]) for k in ("A", "B", "bias", "mult", "shift")]
    want_ws = qg.qgemm_s8s8_requant_zp(*args, za, zb, zo, act=act)
    C = torch.full((M, N), 77, dtype=torch.int8, device="cuda")
    got = qg.qgemm_s8s8_requant_zp_noalloc(*args, za, zb, zo, C=C, act=act)
    torch.cuda.synchronize()
    got, want_ws = got.cpu().numpy(), want_ws.cpu().numpy()
    assert np.array_equal(got, want_ws)
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 40)), [M - 1]]))
    want = oracle.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"], za, zb,
                                       zo, rows=rows, act=act)
    assert np.array_equal(got[rows], want)


def test_noalloc_matches_workspace_form_two_calls(qg):
    for i, (M, N, K, za, zb, zo, act) in enumerate(CALLS):
        _say("noalloc zp gemm", M, N, K, za, zb, zo, act)
        _one(qg, M, N, K, za, zb, zo, act, seed=50 + i)


def test_noalloc_rejects_oversized_shape(qg):
    # compensation sums of M + N rows beyond the 1 MiB array: rejected on
    # the host before any launch
    A = torch.zeros((16, 16), dtype=torch.int8, device="cuda")
    p = torch.zeros(16, dtype=torch.int32, device="cuda")
    st = qg.lib.qgemm_s8s8_requant_zp_noalloc(A.data_ptr(), 16, A.data_ptr(), 16, p.data_ptr(),
                                              p.data_ptr(), p.data_ptr(), 1, 1, 0, -128, 127,
                                              A.data_ptr(), 64, 262081, 64, 16, None)
    assert st == qg.QG_ERR_INVALID

"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronization), so a caller can capture a sequence of calls and
replay it.  Every replay here runs with the program's own eager work and a
synchronization in between, and is compared bit for bit with the eager
result; the inputs are also rewritten in place between replays, which the
replay must see.
"""
import numpy as np
import pytest

from conv_qgemm_amd import datagen

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def qg():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from conv_qgemm_amd import qgemm
    return qgemm


def _run_graph_case(torch, make_inputs, call, outs=("out",)):
    """make_inputs(seed) -> dict of device tensors (inputs and the outputs
    named in outs); call(d) enqueues the library call writing the outputs."""
    d = make_inputs(1)
    call(d)  # eager first: one-time device setup happens outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(d)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        # new input contents in the captured buffers, eager reference beside
        fresh = make_inputs(10 + r)
        for k, v in fresh.items():
            if k not in outs:
                d[k].copy_(v)
        ref = {k: v.clone() for k, v in d.items()}
        for k in outs:
            ref[k] = torch.empty_like(d[k])
        call(ref)
        for k in outs:
            d[k].fill_(7)
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(d[k].cpu(), ref[k].cpu()), f"replay {r}: {k} differs from eager"
        del junk


def test_graph_s8s8(qg):
    import torch

    def make(seed):
        h = datagen.gemm_s8s8(70, 96, 160, seed, shift=(36, 42))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((70, 96), dtype=torch.int8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qgemm_s8s8_requant(
        d["A"], d["B"], d["bias"], d["mult"], d["shift"], C=d["out"]))


def test_graph_s8s8_large_tile(qg):
    """The direct-to-LDS ring kernel (enough tiles to take that path)."""
    import torch

    def make(seed):
        h = datagen.gemm_s8s8(4096, 2048, 256, seed, shift=(40, 46))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((4096, 2048), dtype=torch.int8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qgemm_s8s8_requant(
        d["A"], d["B"], d["bias"], d["mult"], d["shift"], C=d["out"]))


def test_graph_s4s4(qg):
    import torch

    def make(seed):
        h = datagen.gemm_s4s4(64, 80, 256, seed)
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((64, 80), dtype=torch.int32, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qgemm_s4s4_i32(d["A"], d["B"], C=d["out"]))


def test_graph_w4a8_skinny(qg):
    import torch

    def make(seed):
        h = datagen.gemm_w4a8(16, 512, 1024, seed, shift=(36, 42))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((16, 512), dtype=torch.int8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qgemm_w4a8_requant(
        d["A"], d["B"], d["bias"], d["mult"], d["shift"], C=d["out"]))


@pytest.mark.parametrize("C_in", [64, 32])
def test_graph_conv(qg, C_in):
    """C_in 64 takes the LDS-staged kernel, C_in 32 the implicit-im2col one."""
    import torch

    def make(seed):
        h = datagen.conv_nhwc(2, 9, 11, C_in, 64, 3, 3, seed, shift=(36, 42))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((2, 9, 11, 64), dtype=torch.int8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qconv2d_nhwc_s8_requant(
        d["X"], d["W"], d["bias"], d["mult"], d["shift"], stride=(1, 1), pad=(1, 1),
        Y=d["out"]))


@pytest.mark.parametrize("KH", [3, 5])
def test_graph_dwconv(qg, KH):
    """3x3 takes the matrix-core kernel, 5x5 the direct one."""
    import torch

    def make(seed):
        h = datagen.dwconv_nhwc(2, 9, 11, 64, KH, KH, seed, shift=(36, 42))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((2, 9, 11, 64), dtype=torch.int8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qdwconv2d_nhwc_s8_requant(
        d["X"], d["W"], d["bias"], d["mult"], d["shift"], stride=(1, 1),
        pad=(KH // 2, KH // 2), Y=d["out"]))


@pytest.mark.parametrize("M", [70, 4096])
def test_graph_gemm_zp(qg, M):
    """The compensation-term pass and the GEMM, both captured; the workspace
    is part of the graph's inputs.  M 4096 takes the ring kernel."""
    import torch

    def make(seed):
        h = datagen.gemm_s8s8(M, 2048 if M > 70 else 96, 256, seed, shift=(40, 46))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        n = d["B"].shape[0]
        d["out"] = torch.empty((M, n), dtype=torch.int8, device="cuda")
        d["ws"] = torch.empty(qg.lib.qgemm_s8s8_requant_zp_workspace_size(M, n),
                              dtype=torch.uint8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qgemm_s8s8_requant_zp(
        d["A"], d["B"], d["bias"], d["mult"], d["shift"], -9, 4, 7, C=d["out"],
        workspace=d["ws"]))


@pytest.mark.parametrize("C_in", [64, 32])
def test_graph_conv_zp(qg, C_in):
    import torch

    def make(seed):
        h = datagen.conv_nhwc(2, 9, 11, C_in, 64, 3, 3, seed, shift=(36, 42))
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((2, 9, 11, 64), dtype=torch.int8, device="cuda")
        d["ws"] = torch.empty(qg.lib.qconv2d_nhwc_s8_requant_zp_workspace_size(
            2, 9, 11, 64, 3, 3, 1, 1, 1, 1), dtype=torch.uint8, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qconv2d_nhwc_s8_requant_zp(
        d["X"], d["W"], d["bias"], d["mult"], d["shift"], 13, -2, -5, Y=d["out"],
        workspace=d["ws"]))


def test_graph_s4s4_f16(qg):
    import torch
    g = np.random.default_rng(0)
    sa = torch.from_numpy(g.uniform(1e-3, 1e-2, 64).astype(np.float32)).cuda()
    sb = torch.from_numpy(g.uniform(1e-3, 1e-2, 80).astype(np.float32)).cuda()

    def make(seed):
        h = datagen.gemm_s4s4(64, 80, 256, seed)
        d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
        d["out"] = torch.empty((64, 80), dtype=torch.float16, device="cuda")
        return d

    _run_graph_case(torch, make, lambda d: qg.qgemm_s4s4_f16(d["A"], d["B"], sa, sb, C=d["out"]))


@pytest.mark.parametrize("bits", [8, 4])
def test_graph_quant(qg, bits):
    import torch

    def make(seed):
        X = torch.from_numpy(datagen.activations(40, 1040, seed)).to(torch.bfloat16).cuda()
        cols = 1040 if bits == 8 else 520
        return {"X": X,
                "out": torch.empty((40, cols), dtype=torch.int8 if bits == 8 else torch.uint8,
                                   device="cuda"),
                "scale": torch.empty(40, dtype=torch.float32, device="cuda")}

    _run_graph_case(torch, make, lambda d: qg.qquant_per_token(
        d["X"], bits=bits, Q=d["out"], scale=d["scale"]), outs=("out", "scale"))


def test_graph_matches_oracle(qg, orc):
    """One replayed result also checked against the oracle directly."""
    import torch
    h = datagen.gemm_s8s8(33, 48, 64, 3, shift=(36, 42))
    d = {k: torch.from_numpy(v).cuda() for k, v in h.items()}
    C = torch.empty((33, 48), dtype=torch.int8, device="cuda")
    qg.qgemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], C=C)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qgemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], C=C)
    C.fill_(0)
    g.replay()
    torch.cuda.synchronize()
    want = orc.gemm_s8s8_requant(h["A"], h["B"], h["bias"], h["mult"], h["shift"])
    assert np.array_equal(C.cpu().numpy(), want)

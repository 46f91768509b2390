#!/usr/bin/env python3
"""Benchmark of the quantized GEMM / conv hot path on one MI355X.

One step is one call of each of the five workloads of the problem
statement, which together run every step of the path:
  pointwise  qgemm_s8s8_requant  M=320 N=64 K=64 (1x1 conv, 20x16 pixels)
  s4s4       qgemm_s4s4_i32      M=N=K=4096, raw int32 out
  conv3x3    qconv2d_nhwc_s8_requant  batch 32, 56x56, 64->64, 3x3 s1 p1
  w4a8       qgemm_w4a8_requant  M=16 tokens, K=8192, N=28672 (skinny)
  s8s8       qgemm_s8s8_requant  M=N=K=8192
The other entry points run on their own workloads as extra legs, reported
beside the step but not part of its value:
  dw3x3      qdwconv2d_nhwc_s8_requant  batch 32, 56x56, 64 channels, 3x3 s1 p1
  quant_a8   qquant_per_token    8192 tokens x 8192 channels, bfloat16 -> int8
             codes + float32 scales (the s8s8 A operand; no integer ops)
  w4a8_m64   qgemm_w4a8_requant  M=64 tokens, same weights (skinny, four
             16-token blocks sharing one pass over the weights)
  w4a8_prefill  qgemm_w4a8_requant  M=2048 tokens, same weights (ring kernel)
  conv3x3_zp, s8s8_zp  the asymmetric calls (qconv2d_nhwc_s8_requant_zp,
             qgemm_s8s8_requant_zp) on the same arrays with zero points on
             the input, the weights and the output; their time includes the
             compensation-sum pass
Inputs are seeded synthetic arrays resident in HBM before timing starts.
Each workload rotates through enough copies of its buffers that every call
reads HBM rather than the 256 MB Infinity Cache (the pointwise case is
L2-sized and reported hot).

Two calibration legs measure the board's practical ceilings in the same run
(libqgcalib.so): a read-only HBM stream and an int8 matrix-core stream on
random operands, with the engine clock it ran at.  The GFX clock the driver
reports is sampled during every workload's timed replays.

Prints ONE JSON line: the step's int TOPS as `value` (median per-call
times), per-workload times, TOPS, GB/s and fractions of the published INT8
MFMA and HBM peaks and of the calibrated ceilings, the roofline of the
dominant kernel (HIP events on the launch stream around graph replays of
the timed calls), and the CPU oracle timed on a bounded sample of the step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0       # MI355X dense INT8 MFMA, published (5.0 POP/s)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published (8 TB/s)
METRIC = "int TOPS + % of INT8 MFMA peak (or HBM GB/s % peak) per qgemm config"
ORDER = ["pointwise", "dw3x3", "quant_a8", "w4a8", "w4a8_m64", "conv3x3", "conv3x3_zp", "s4s4",
         "w4a8_prefill", "s8s8", "s8s8_zp"]
# the problem statement's five workloads: one call of each is a step
STEP = ("pointwise", "s4s4", "conv3x3", "w4a8", "s8s8")
MFMA_BOUND = ("s8s8", "s8s8_zp", "s4s4", "conv3x3", "conv3x3_zp", "pointwise", "w4a8_prefill")
HBM_BOUND = ("w4a8", "w4a8_m64", "quant_a8", "dw3x3")
# buffer sets per workload so that the rotation exceeds the Infinity Cache
ROTATE = {"pointwise": 1, "s4s4": 7, "conv3x3": 40, "conv3x3_zp": 40, "dw3x3": 40,
          "quant_a8": 3, "w4a8": 5, "w4a8_m64": 5, "w4a8_prefill": 3, "s8s8": 3, "s8s8_zp": 3}
KERNEL_SOURCES = {
    "s8s8": "conv_qgemm_amd/csrc/k_gemm_dma.hip",
    "s4s4": "conv_qgemm_amd/csrc/k_gemm_dma.hip",
    "pointwise": "conv_qgemm_amd/csrc/k_tile_gemm.hip",
    "conv3x3": "conv_qgemm_amd/csrc/k_conv_halo.hip",
    "w4a8": "conv_qgemm_amd/csrc/k_skinny_w4a8.hip",
    "w4a8_m64": "conv_qgemm_amd/csrc/k_skinny_w4a8.hip",
    "dw3x3": "conv_qgemm_amd/csrc/k_dwconv.hip",
    "quant_a8": "conv_qgemm_amd/csrc/k_quant.hip",
    "s8s8_zp": "conv_qgemm_amd/csrc/k_gemm_dma.hip",
    "w4a8_prefill": "conv_qgemm_amd/csrc/k_gemm_dma.hip",
    "conv3x3_zp": "conv_qgemm_amd/csrc/k_conv_halo.hip",
}


def shape_of(name):
    from conv_qgemm_amd import datagen
    return datagen.WORKLOADS[name]


def ops_and_bytes(name):
    """(int ops = 2 * MACs, algorithmic bytes: inputs once, outputs once,
    plus 12 bytes per output channel of bias / multiplier / shift)."""
    w = shape_of(name)
    if w["kind"] == "quant":
        eb = {"float32": 4, "float16": 2, "bfloat16": 2}[w["dtype"]]
        return 0, w["M"] * w["K"] * eb + w["M"] * w["K"] * w["bits"] // 8 + 4 * w["M"]
    if w["kind"] == "dwconv":
        Ho, Wo = w["H"], w["W"]  # 3x3 s1 p1 keeps the size
        pix = w["batch"] * Ho * Wo
        macs = pix * w["C"] * w["KH"] * w["KW"]
        by = w["batch"] * w["H"] * w["W"] * w["C"] + w["KH"] * w["KW"] * w["C"] + \
            12 * w["C"] + pix * w["C"]
        return 2 * macs, by
    if w["kind"] == "conv":
        Ho, Wo = w["H"], w["W"]  # 3x3 s1 p1 keeps the size
        pix = w["batch"] * Ho * Wo
        K = w["KH"] * w["KW"] * w["C_in"]
        macs = pix * w["C_out"] * K
        by = w["batch"] * w["H"] * w["W"] * w["C_in"] + w["C_out"] * K + 12 * w["C_out"] + \
            pix * w["C_out"]
        return 2 * macs, by
    M, N, K = w["M"], w["N"], w["K"]
    macs = M * N * K
    if w["kind"] == "s8s8":
        by = M * K + N * K + M * N + 12 * N
    elif w["kind"] == "s4s4":
        by = M * K // 2 + N * K // 2 + 4 * M * N
    else:  # w4a8
        by = M * K + N * K // 2 + M * N + 12 * N
    return 2 * macs, by


def code_text(src):
    """C++ source with its comments removed and each run of whitespace made
    one space: what the compiler sees, so that a comment-only edit keeps the
    counters taken on the kernel.  String and character literals are kept
    whole (an asm string may hold '//')."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def src_sha(path):
    """Fingerprint of a kernel's code (its source and the shared device
    header, comments and layout aside)."""
    h = hashlib.sha256()
    for p in (path, "conv_qgemm_amd/csrc/dev_common.hpp"):
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None when it is absent or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if not line.startswith("traffic "):
            continue
        kv = dict(x.split("=", 1) for x in line.split()[1:])
        if kv.get("workload") != name:
            continue
        if kv.get("src_sha") != src_sha(KERNEL_SOURCES[name]):
            return None
        return int(float(kv["bytes_per_launch"]))
    return None


class Case:
    """Device buffers (rotated copies) and the call of one workload."""

    def __init__(self, name, torch, qgemm, datagen):
        self.name = name
        self.q = qgemm
        d = datagen.workload(name)
        self.host = d
        nrot = ROTATE[name]
        dev = lambda a: torch.from_numpy(a).cuda()
        w = shape_of(name)
        if w["kind"] == "quant":
            base = {"X": torch.from_numpy(d["X"]).to(getattr(torch, w["dtype"])).cuda()}
        else:
            base = {k: dev(v) for k, v in d.items()}
        self.sets = []
        for r in range(nrot):
            s = {k: (v if r == 0 else v.clone()) for k, v in base.items()}
            if w["kind"] == "quant":
                s["Q"] = torch.empty((w["M"], w["K"] * w["bits"] // 8),
                                     dtype=torch.int8 if w["bits"] == 8 else torch.uint8,
                                     device="cuda")
                s["scale"] = torch.empty(w["M"], dtype=torch.float32, device="cuda")
            elif w["kind"] == "conv":
                s["Y"] = torch.empty((w["batch"], w["H"], w["W"], w["C_out"]), dtype=torch.int8,
                                     device="cuda")
            elif w["kind"] == "dwconv":
                s["Y"] = torch.empty((w["batch"], w["H"], w["W"], w["C"]), dtype=torch.int8,
                                     device="cuda")
            elif w["kind"] == "s4s4":
                s["C"] = torch.empty((w["M"], w["N"]), dtype=torch.int32, device="cuda")
            else:
                s["C"] = torch.empty((w["M"], w["N"]), dtype=torch.int8, device="cuda")
            if "zp" in w:
                if w["kind"] == "conv":
                    nb = qgemm.lib.qconv2d_nhwc_s8_requant_zp_workspace_size(
                        w["batch"], w["H"], w["W"], w["C_out"], w["KH"], w["KW"],
                        w["stride"][0], w["stride"][1], w["pad"][0], w["pad"][1])
                else:
                    nb = qgemm.lib.qgemm_s8s8_requant_zp_workspace_size(w["M"], w["N"])
                s["ws"] = torch.empty(nb, dtype=torch.uint8, device="cuda")
            self.sets.append(s)
        self.ops, self.bytes = ops_and_bytes(name)
        # SHA-256 over the generated host arrays (names sorted), so that a
        # result names the exact inputs it was measured on
        import numpy as np
        h = hashlib.sha256()
        for k in sorted(d):
            h.update(k.encode())
            h.update(np.ascontiguousarray(d[k]).tobytes())
        self.input_sha = h.hexdigest()

    def __call__(self, i):
        s = self.sets[i % len(self.sets)]
        q = self.q
        if self.name == "s4s4":
            return q.qgemm_s4s4_i32(s["A"], s["B"], C=s["C"])
        if self.name in ("w4a8", "w4a8_m64", "w4a8_prefill"):
            return q.qgemm_w4a8_requant(s["A"], s["B"], s["bias"], s["mult"], s["shift"], C=s["C"])
        if self.name == "s8s8_zp":
            za, zb, zo = shape_of(self.name)["zp"]
            return q.qgemm_s8s8_requant_zp(s["A"], s["B"], s["bias"], s["mult"], s["shift"], za,
                                           zb, zo, C=s["C"], workspace=s["ws"])
        if self.name == "conv3x3_zp":
            za, zb, zo = shape_of(self.name)["zp"]
            return q.qconv2d_nhwc_s8_requant_zp(s["X"], s["W"], s["bias"], s["mult"], s["shift"],
                                                za, zb, zo, stride=(1, 1), pad=(1, 1), Y=s["Y"],
                                                workspace=s["ws"])
        if self.name == "quant_a8":
            return q.qquant_per_token(s["X"], bits=shape_of("quant_a8")["bits"], Q=s["Q"],
                                      scale=s["scale"])
        if self.name == "dw3x3":
            return q.qdwconv2d_nhwc_s8_requant(s["X"], s["W"], s["bias"], s["mult"], s["shift"],
                                               stride=(1, 1), pad=(1, 1), Y=s["Y"])
        if self.name == "conv3x3":
            return q.qconv2d_nhwc_s8_requant(s["X"], s["W"], s["bias"], s["mult"], s["shift"],
                                             stride=(1, 1), pad=(1, 1), Y=s["Y"])
        return q.qgemm_s8s8_requant(s["A"], s["B"], s["bias"], s["mult"], s["shift"], C=s["C"])


def cpu_baseline(names, frac=16):
    """The CPU oracle, as it stands, on 1/frac of every workload of the step:
    every frac-th output row (GEMMs), pixel (conv), weight row (w4a8) or
    token (quantizer); every (16 frac)-th row of the W4A8 prefill.  Wall
    seconds and GMAC/s per workload, and the step's ops over the total
    seconds as `value`."""
    import numpy as np

    import oracle
    from conv_qgemm_amd import datagen

    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    total_ops, total_t, parts, per = 0, 0.0, [], {}
    for name in names:
        d = datagen.workload(name)
        w = shape_of(name)
        ops, _ = ops_and_bytes(name)
        t0 = time.perf_counter()
        if w["kind"] == "s8s8" and "zp" in w:
            rows = np.arange(0, w["M"], frac)
            oracle.gemm_s8s8_requant_zp(d["A"], d["B"], d["bias"], d["mult"], d["shift"],
                                        *w["zp"], rows=rows)
            part = len(rows) / w["M"]
        elif w["kind"] == "s8s8":
            rows = np.arange(0, w["M"], frac)
            oracle.gemm_s8s8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
            part = len(rows) / w["M"]
        elif w["kind"] == "s4s4":
            rows = np.arange(0, w["M"], frac)
            oracle.gemm_s4s4_i32(d["A"], d["B"], rows=rows)
            part = len(rows) / w["M"]
        elif w["kind"] == "w4a8" and w["M"] > 64:
            rows = np.arange(0, w["M"], frac * 16)
            oracle.gemm_w4a8_requant(d["A"], d["B"], d["bias"], d["mult"], d["shift"], rows=rows)
            part = len(rows) / w["M"]
        elif w["kind"] == "w4a8":
            cols = np.arange(0, w["N"], frac)
            oracle.gemm_w4a8_requant(d["A"], d["B"][cols], d["bias"][cols], d["mult"][cols],
                                     d["shift"][cols])
            part = len(cols) / w["N"]
        elif w["kind"] == "quant":
            import torch
            rows = np.arange(0, w["M"], frac)
            Xs = torch.from_numpy(d["X"][rows]).to(getattr(torch, w["dtype"]))
            if w["dtype"] == "bfloat16":
                Xs = Xs.view(torch.int16).numpy().view(np.uint16)
            else:
                Xs = Xs.numpy()
            t0 = time.perf_counter()  # the conversion to the input type is not the oracle's
            oracle.quant_per_token(Xs, bits=w["bits"], dtype=w["dtype"])
            part = len(rows) / w["M"]
        elif w["kind"] == "dwconv":
            npix = w["batch"] * w["H"] * w["W"]
            pix = np.arange(0, npix, frac)
            oracle.dwconv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                            pix=pix)
            part = len(pix) / npix
        elif "zp" in w:
            npix = w["batch"] * w["H"] * w["W"]
            pix = np.arange(0, npix, frac)
            oracle.conv2d_nhwc_s8_requant_zp(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                             *w["zp"], pix=pix)
            part = len(pix) / npix
        else:
            npix = w["batch"] * w["H"] * w["W"]
            pix = np.arange(0, npix, frac)
            oracle.conv2d_nhwc_s8_requant(d["X"], d["W"], d["bias"], d["mult"], d["shift"],
                                          pix=pix)
            part = len(pix) / npix
        dt = time.perf_counter() - t0
        total_ops += ops * part
        total_t += dt
        parts.append(f"{name}:{part:.4f}")
        per[name] = {"seconds": round(dt, 3), "fraction": round(part, 4),
                     "gmac_s": round(ops / 2 * part / dt / 1e9, 2)}
    return {"value": total_ops / total_t / 1e12, "unit": "TOPS", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(total_t, 2), "per_config": per,
            "sample": f"every {frac}th output row/pixel/weight row/token of each workload of one "
                      f"step ({', '.join(parts)} of the outputs)"}


def hbm_copy_gbs(torch, nbytes=1 << 30, iters=10):
    """Achieved bandwidth of a plain device-to-device copy (read + write)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9


def _calib_lib():
    import ctypes
    path = os.path.join(ROOT, "conv_qgemm_amd", "libqgcalib.so")
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.qgc_stream_read.argtypes = [P, I64, P, I32, I32, P]
    lib.qgc_stream_read.restype = I32
    lib.qgc_mfma_stream.argtypes = [P, I32, P, P, I32, I32, P]
    lib.qgc_mfma_stream.restype = I32
    lib.qgc_wall_clock_khz.argtypes = []
    lib.qgc_wall_clock_khz.restype = I32
    return lib


def vendor_comparison(torch, M=8192, N=8192, K=8192, reps=10, seed=7):
    """AMD's hipBLASLt int8 GEMM (int8 operands, int32 output, no requantize)
    on the s8s8 workload's shape, every solution the library offers for it
    timed (libqgvendor.so: 2 untimed calls, then the median of `reps` eager
    calls between HIP events per solution), and 16 elements of the best
    solution's output checked exactly."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "conv_qgemm_amd", "libqgvendor.so"))
    P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.qgv_int8_gemm_search.argtypes = [P, P, P, I64, I64, I64, P, I64, I32, P,
                                         ctypes.POINTER(D), ctypes.POINTER(D),
                                         ctypes.POINTER(I32), ctypes.c_char_p, I32,
                                         ctypes.c_char_p, I32]
    lib.qgv_int8_gemm_search.restype = I32
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    A = torch.randint(-128, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    B = torch.randint(-128, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    C = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    heur, best, n = D(-1), D(-1), I32(0)
    bname, hname = ctypes.create_string_buffer(512), ctypes.create_string_buffer(512)
    st = torch.cuda.current_stream()
    rc = lib.qgv_int8_gemm_search(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K,
                                  ws.data_ptr(), ws.numel(), reps, ctypes_stream(st),
                                  ctypes.byref(heur), ctypes.byref(best), ctypes.byref(n),
                                  bname, 512, hname, 512)
    torch.cuda.synchronize()
    if rc != 0:
        raise RuntimeError(f"qgv_int8_gemm_search: {rc}")
    rows = torch.randint(0, M, (16,), generator=g, device="cuda")
    cols = torch.randint(0, N, (16,), generator=g, device="cuda")
    want = (A[rows].to(torch.int64) * B[cols].to(torch.int64)).sum(dim=1)
    ok = int((C[rows, cols].to(torch.int64) == want).sum())
    ops = 2.0 * M * N * K
    return {"library": "hipBLASLt", "problem": f"int8 {M}x{N}x{K}, int32 out, no requantize",
            "heuristic_us": round(heur.value, 2),
            "best_us": round(best.value, 2), "best_tops": round(ops / best.value / 1e6, 1),
            "solutions_timed": n.value, "best_kernel": bname.value.decode()[:160],
            "heuristic_kernel": hname.value.decode()[:160],
            "checked": f"{ok} of 16 elements exact",
            "timing": f"median of {reps} eager calls per solution between HIP events"}


def read_calibration(torch, reps=5):
    """Best read-only streaming rates (GB/s) over a few launch shapes, with
    16-byte loads, grid-stride, `unroll` loads in flight per thread:
      read_gb_s          a 1 GiB buffer (4x the Infinity Cache) per launch;
      read_gb_s_117mb    a 117,440,512-byte buffer per launch (the skinny
                         W4A8 weight matrix), five copies in rotation so
                         that each launch reads HBM: the like-for-like
                         ceiling of a bandwidth-bound kernel of that size,
                         launch and ramp included."""
    lib = _calib_lib()
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    out = {}
    for key, nbytes, ncopy, nrep in (("read_gb_s", 1 << 30, 1, reps),
                                     ("read_gb_s_117mb", 117440512, 5, 20)):
        bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
                for _ in range(ncopy)]
        best = (0.0, None)
        for grid in (2048, 4096, 8192, 16384):
            for unroll in (4, 8):
                def go(i):
                    rc = lib.qgc_stream_read(bufs[i % ncopy].data_ptr(), nbytes, sink.data_ptr(),
                                             grid, unroll, ctypes_stream(st))
                    if rc != 0:
                        raise RuntimeError(f"qgc_stream_read: hip error {rc}")
                for i in range(ncopy):
                    go(i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for i in range(nrep):
                    go(i)
                e1.record(st)
                torch.cuda.synchronize()
                gbs = nbytes * nrep / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if gbs > best[0]:
                    best = (gbs, f"grid {grid} x 256 threads, {unroll} x 16-byte loads in flight")
        out[key] = round(best[0], 1)
        out[key.replace("gb_s", "shape")] = best[1]
        del bufs
    return out


def mfma_calibration(torch, cus, iters=20000, reps=5, seed=99):
    """int8 matrix-core ceiling on random operands, 256 accumulator registers
    per wave, 4 waves per CU, one workgroup per CU, for two MFMA shapes:
    v_mfma_i32_32x32x32_i8 over 4x4 tiles and v_mfma_i32_16x16x64_i8 over 8x8
    tiles (the same MACs per round: `iters` rounds of the first, iters/2 of
    the second); the median of `reps` launches of ~5 ms each.  Under the
    power limit the two run at different clocks; the faster is the ceiling.
    The clock is the shader-clock counter over the constant-rate counter
    around the loop (s_memtime / s_memrealtime), times the latter's rate."""
    import numpy as np
    lib = _calib_lib()
    g = np.random.default_rng(seed)
    ops = torch.from_numpy(g.integers(-128, 127, size=cus * 4 * 16 * 64 * 16, endpoint=True,
                                      dtype=np.int8)).cuda()
    clk = torch.zeros(4 * cus, dtype=torch.int64, device="cuda")
    sink = torch.zeros(cus * 256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    wall_khz = lib.qgc_wall_clock_khz()
    shapes = {}
    for shape, name, it, macs in ((0, "32x32x32", iters, 16 * 32768),
                                  (1, "16x16x64", iters // 2, 64 * 16384)):
        res = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = lib.qgc_mfma_stream(ops.data_ptr(), it, clk.data_ptr(), sink.data_ptr(), cus,
                                     shape, ctypes_stream(st))
            e1.record(st)
            if rc != 0:
                raise RuntimeError(f"qgc_mfma_stream: hip error {rc}")
            torch.cuda.synchronize()
            if r == 0:
                continue  # warm-up launch
            t = e0.elapsed_time(e1) * 1e-3
            c = clk.cpu().numpy().reshape(cus, 4).astype(np.float64)
            ratio = (c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1)
            res.append((cus * 4 * it * macs * 2 / t / 1e12, float(np.median(ratio))))
        res.sort()
        tops, ratio = res[len(res) // 2]
        shapes[name] = {"tops": round(tops, 1),
                        "clock_mhz": round(ratio * wall_khz / 1e3, 1) if wall_khz else None,
                        "rounds": it}
    best = max(shapes, key=lambda k: shapes[k]["tops"])
    return {"mfma_random_tops": shapes[best]["tops"],
            "mfma_random_frac_of_peak": round(shapes[best]["tops"] / PEAK_INT8_TOPS, 4),
            "mfma_clock_mhz": shapes[best]["clock_mhz"],
            "mfma_shape": best,
            "mfma_shapes": shapes,
            "wall_clock_khz": wall_khz,
            "shape": f"{cus} workgroups x 4 waves, 256 accumulator registers per wave, "
                     f"random int8 operands, median of {reps} launches per MFMA shape; "
                     f"the faster shape is the ceiling"}


def ctypes_stream(st):
    """The raw hipStream_t of a torch stream, for a ctypes call."""
    return st.cuda_stream


class ClockSampler:
    """The GFX clock and socket power the driver reports (amdsmi GPU
    metrics: the mean of the per-XCD current_gfxclks, current_socket_power),
    sampled every few ms on a host thread; means over a time window.  Absent
    (None) where amdsmi cannot be opened."""

    def __init__(self, period=0.004):
        import threading
        self.samples = []
        self.ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            if self._read() is None:
                return
            self.ok = True
        except Exception:
            return
        self._stop = False
        self._period = period
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = m.get("current_gfxclks")
        clks = [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 10000] \
            if isinstance(clks, (list, tuple)) else []
        if not clks:
            return None
        pw = m.get("current_socket_power")
        pw = float(pw) if isinstance(pw, (int, float)) and 0 < pw < 100000 else float("nan")
        return sum(clks) / len(clks), pw

    def _run(self):
        while not self._stop:
            try:
                r = self._read()
                if r is not None:
                    self.samples.append((time.perf_counter(), r[0], r[1]))
            except Exception:
                pass
            time.sleep(self._period)

    def mean(self, t0, t1):
        """(mean MHz, mean W, samples) over [t0, t1]."""
        v = [(c, w) for t, c, w in self.samples if t0 <= t <= t1]
        if not v:
            return None, None, 0
        w = [x[1] for x in v if x[1] == x[1]]
        return (round(sum(x[0] for x in v) / len(v), 1),
                round(sum(w) / len(w), 1) if w else None, len(v))

    def close(self):
        if self.ok:
            self._stop = True
            self._t.join(timeout=1)
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass


def _csv_rows(path):
    import csv
    import glob
    files = [path] if os.path.isfile(path) else sorted(
        glob.glob(os.path.join(path, "**", "*.csv"), recursive=True))
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def summarize_trace(stats_csv, title, cmd):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel summary."""
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in _csv_rows(stats_csv):
        if "AverageNs" not in r:
            continue
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    return "\n".join(lines)


def summarize_pmc(name, fetch_dir, write_dir, copy_bytes=1 << 30):
    """One traffic line for `name` from two rocprofv3 --pmc runs of
    `bench.py --config name` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).
    The dispatches of the workload's kernel (KERNEL_NAMES) are averaged; the
    1 GiB device copy of hbm_copy_gbs() in the same run calibrates the
    counter (factor = known bytes / what the counter reads for that copy)."""
    out = {}
    kn = KERNEL_NAMES[name]
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        work, copies = [], []
        for r in _csv_rows(d):
            if r.get("Counter_Name") != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            if "copy" in r["Kernel_Name"].lower():
                copies.append(v)
            elif kn in r["Kernel_Name"]:
                work.append(v)
        if not work or not copies:
            raise SystemExit(f"no {counter} rows for the workload or the copy kernel in {d}")
        calib = copy_bytes / max(copies)
        out[counter] = (sum(work) / len(work), calib)
    (f, cf), (w, cw) = out["FETCH_SIZE"], out["WRITE_SIZE"]
    total = f * cf + w * cw
    return (f"traffic workload={name} src_sha={src_sha(KERNEL_SOURCES[name])} "
            f"bytes_per_launch={int(total)} fetch_bytes_raw={int(f)} write_bytes_raw={int(w)} "
            f"calib_fetch={cf:.4f} calib_write={cw:.4f}")


LABELS = {"pointwise": "pointwise s8s8 320x64x64", "s4s4": "s4s4 4096^3 -> i32",
          "conv3x3": "conv3x3 NHWC 32x56x56x64->64",
          "dw3x3": "depthwise 3x3 NHWC 32x56x56x64",
          "quant_a8": "per-token quant bf16 8192x8192 -> int8",
          "w4a8": "w4a8 skinny 16x28672x8192", "s8s8": "s8s8 8192^3",
          "w4a8_m64": "w4a8 skinny 64x28672x8192",
          "w4a8_prefill": "w4a8 prefill 2048x28672x8192",
          "conv3x3_zp": "conv3x3 with zero points", "s8s8_zp": "s8s8 8192^3 with zero points"}


# kernel of each workload, as it appears in a rocprofv3 kernel name
KERNEL_NAMES = {"s8s8": "k_gemm_dma<8, 0,", "s8s8_zp": "k_gemm_dma<8, 2,",
                "w4a8_prefill": "k_gemm_dma<3, 0,", "s4s4": "k_gemm_dma<4, 1,",
                "conv3x3": "k_conv_halo<3, 3, false>", "conv3x3_zp": "k_conv_halo<3, 3, true>",
                "w4a8": "k_skinny_w4a8", "w4a8_m64": "k_skinny_w4a8",
                "dw3x3": "k_dwconv3x3<1, false>", "quant_a8": "k_quant", "pointwise": "k_tile"}


def summarize_counters(name, *dirs, n_xcd=8, n_simd=1024):
    """One line per workload from rocprofv3 --pmc runs of `bench.py --config
    name`: each counter averaged over the workload kernel's dispatches, plus
    derived figures where their counters are present:
      clock_mhz   = GRBM_GUI_ACTIVE / n_xcd / dispatch duration (the engine
                    clock while the kernel ran; GRBM counts per XCD), for
                    dispatches of 200 us or more
      mfma_busy   = SQ_VALU_MFMA_BUSY_CYCLES / n_simd / (GRBM_GUI_ACTIVE /
                    n_xcd): share of the kernel's cycles the matrix pipe
                    issues in
      lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      tcp_* stall shares = the TCP counter / 256 CUs / (GRBM_GUI_ACTIVE / n_xcd)"""
    import collections
    kn = KERNEL_NAMES[name]
    vals = collections.defaultdict(list)
    durs = []
    for d in dirs:
        for r in _csv_rows(d):
            if "Counter_Name" not in r or kn not in r["Kernel_Name"]:
                continue
            vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                durs.append((float(r["Counter_Value"]),
                             float(r["End_Timestamp"]) - float(r["Start_Timestamp"])))
    if not vals:
        raise SystemExit(f"no dispatches of {kn} in {dirs}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    out = [f"counters workload={name} kernel=\"{kn}\""]
    if durs:
        g = sum(x for x, _ in durs) / len(durs) / n_xcd
        t_us = sum(t for _, t in durs) / len(durs) / 1e3
        # GRBM_GUI_ACTIVE also counts a few thousand cycles around the
        # dispatch, so the clock is only given for long dispatches
        if t_us >= 200:
            out.append(f"clock_mhz={sum(x / n_xcd / t for x, t in durs) / len(durs) * 1e3:.0f}")
        out.append(f"dispatch_us={t_us:.1f}")
        out.append(f"grbm_active_per_xcd={g:.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            out.append(f"mfma_busy_pct={100 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / n_simd / g:.1f}")
        for k in ("TCP_PENDING_STALL_CYCLES", "TCP_TCR_TCP_STALL_CYCLES",
                  "TCP_UTCL1_STALL_INFLIGHT_MAX", "TCP_UTCL1_SERIALIZATION_STALL",
                  "TA_ADDR_STALLED_BY_TC_CYCLES"):
            if k in avg:
                out.append(f"{k.lower()}_pct={100 * avg[k] / 256 / g:.1f}")
    if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
        out.append(f"lds_conflict_pct={100 * avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.1f}")
    out += [f"{k.lower()}={v:.0f}" for k, v in sorted(avg.items()) if k != "GRBM_GUI_ACTIVE"]
    return " ".join(out)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        print(summarize_counters(sys.argv[2], *sys.argv[3:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        print(summarize_trace(sys.argv[2], sys.argv[3], sys.argv[4]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        print(summarize_pmc(sys.argv[2], sys.argv[3], sys.argv[4]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="all", help="all, or a comma list of " + ",".join(ORDER))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-calib", action="store_true", help="skip the calibration legs")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the hipBLASLt comparison on the s8s8 shape")
    ap.add_argument("--cpu-frac", type=int, default=2)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; runs on more than one GPU are not "
              "part of it (across GPUs the path would shard the output channels, each GPU "
              "streaming only its own weight columns)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from conv_qgemm_amd import datagen
    if not os.path.exists(os.path.join(ROOT, "conv_qgemm_amd", "libqgemm.so")):
        import __graft_entry__
        __graft_entry__.build()
    from conv_qgemm_amd import qgemm

    names = ORDER if args.config == "all" else args.config.split(",")
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cases = [Case(n, torch, qgemm, datagen) for n in names]
    torch.cuda.synchronize()
    clock = ClockSampler()

    # Timed region: each workload runs as its own phase, lightest first, so
    # that a workload is not measured in the power state a heavier one leaves
    # behind.  A phase is W warm-up calls, then K back-to-back eager calls
    # between two HIP events on the launch stream, then the same K calls
    # captured in a HIP graph, replayed once untimed and then 20 times with
    # an event between replays.  The median replay, divided by K, is the
    # per-launch GPU time without the Python binding's per-call host cost
    # (which decides the launch-bound pointwise case and is hidden behind
    # the GPU for the others); the first replay and the p99 are reported
    # beside it.
    stream = torch.cuda.current_stream()
    eager, graphed, spread, windows = {}, {}, {}, {}
    nb = 20  # timed replays of the K-call graph

    def timed(fn):
        s0 = torch.cuda.current_stream()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s0)
        fn()
        b.record(s0)
        return a, b

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in cases:
        for i in range(args.warmup):
            c(i)
        eager[c.name] = timed(lambda: [c(i) for i in range(args.steps)])
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                c(i)
        g.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        bmarks = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
        bmarks[0].record(stream)
        for r in range(nb):
            g.replay()
            bmarks[r + 1].record(stream)
        torch.cuda.synchronize()
        windows[c.name] = (w0, time.perf_counter())
        graphed[c.name] = bmarks
        # 20 more eager calls with an event after each give the spread of
        # single launches (median, max); they enter no average
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
        marks[0].record(stream)
        for i in range(20):
            c(i)
            marks[i + 1].record(stream)
        spread[c.name] = marks
        torch.cuda.synchronize()
        del g
    wall = time.perf_counter() - t0

    calib = {}
    if not args.no_calib:
        try:
            calib.update(read_calibration(torch))
            w0 = time.perf_counter()
            calib.update(mfma_calibration(torch, cus))
            mhz, watts, _ = clock.mean(w0, time.perf_counter())
            calib["mfma_smi_gfxclk_mhz"] = mhz
            calib["mfma_smi_socket_w"] = watts
        except (OSError, RuntimeError) as e:
            calib["error"] = str(e)
    try:
        copy_gbs = round(hbm_copy_gbs(torch), 1)
    except RuntimeError:
        copy_gbs = None
    vendor = None
    if not args.no_vendor and "s8s8" in names:
        try:
            vendor = vendor_comparison(torch)
        except (OSError, RuntimeError) as e:
            vendor = {"error": str(e)}
    clock.close()

    per = {}
    for c in cases:
        bm = graphed[c.name]
        bt = [bm[r].elapsed_time(bm[r + 1]) * 1e-3 / args.steps for r in range(nb)]
        first = bt[0]
        bts = sorted(bt)
        b_med = bts[len(bts) // 2]
        b_p99 = bts[min(len(bts) - 1, int(0.99 * len(bts)))]
        a, b = eager[c.name]
        avg_eager = a.elapsed_time(b) * 1e-3 / args.steps
        m = spread[c.name]
        times = sorted(m[i].elapsed_time(m[i + 1]) * 1e-3 for i in range(len(m) - 1))
        tops = c.ops / b_med / 1e12
        gbs = c.bytes / b_med / 1e9
        mhz, watts, nsamp = clock.mean(*windows[c.name])
        e = {"us_median": round(b_med * 1e6, 2),
             "us_first_replay": round(first * 1e6, 2),
             "us_batch_p99": round(b_p99 * 1e6, 2),
             "us_avg_eager": round(avg_eager * 1e6, 2),
             "us_single_median": round(times[len(times) // 2] * 1e6, 2),
             "us_single_max": round(times[-1] * 1e6, 2), "tops": round(tops, 2),
             "gb_s": round(gbs, 1),
             "pct_int8_mfma_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
             "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
             "ops": c.ops, "alg_bytes": c.bytes,
             "smi_gfxclk_mhz": mhz, "smi_socket_w": watts, "smi_samples": nsamp,
             "buffer_sets": ROTATE[c.name], "input_sha256": c.input_sha}
        if c.name in HBM_BOUND and calib.get("read_gb_s"):
            e["pct_of_read_rate"] = round(100 * gbs / calib["read_gb_s"], 1)
        if c.name in ("w4a8", "w4a8_m64") and calib.get("read_gb_s_117mb"):
            e["pct_of_read_rate_117mb"] = round(100 * gbs / calib["read_gb_s_117mb"], 1)
        if c.name in MFMA_BOUND and calib.get("mfma_random_tops") and c.name != "pointwise":
            e["pct_of_mfma_calib"] = round(100 * tops / calib["mfma_random_tops"], 1)
        per[c.name] = e

    # one step = one call of each of the five workloads (median per-call
    # times); warm-up calls are outside
    step = [n for n in STEP if n in per] or list(per)
    step_s = sum(per[n]["us_median"] for n in step) * 1e-6
    step_ops = sum(cases[names.index(n)].ops for n in step)
    value = step_ops / step_s / 1e12

    # the roofline describes the dominant single kernel of the step: the
    # longest of its workloads
    dom = max(step, key=lambda n: per[n]["us_median"])
    if dom in MFMA_BOUND:
        achieved = per[dom]["tops"]
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": round(achieved / PEAK_INT8_TOPS, 4)}
    else:
        achieved = per[dom]["gb_s"]
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(dom)
    roof["time"] = "median of 20 graph replays of the timed calls, per call"

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "qgemm step: " + " + ".join(LABELS[n] for n in step),
                   "extra_legs": [LABELS[n] for n in names if n not in step],
                   "parallelism": "single GPU", "seeds": "numpy PCG64 1..8",
                   "timing": f"per workload: {args.warmup} warm-up calls; "
                             f"{args.steps} back-to-back calls issued eagerly from Python "
                             f"(us_avg_eager); the same {args.steps} calls captured in a "
                             f"HIP graph, replayed once untimed and {nb} times between "
                             f"HIP events (us_median, which value and roofline use; "
                             f"us_first_replay; us_batch_p99: per call over the {nb} "
                             f"replays); single-launch spread from 20 more eager calls; "
                             f"wall {wall:.3f} s for all phases"},
        "per_config": {n: per[n] for n in step},
        "extra": {n: per[n] for n in names if n not in step},
        "roofline": roof,
        "calibration": calib,
        "hbm_copy_gb_s": copy_gbs,
    }
    if vendor is not None:
        if "best_us" in vendor:
            vendor["this_kernel_us"] = per["s8s8"]["us_median"]
        out["vendor_int8_gemm"] = vendor
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(step, args.cpu_frac)
    print(json.dumps(out))


if __name__ == "__main__":
    main()

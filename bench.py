#!/usr/bin/env python3
"""Benchmark of the quantized GEMM / conv hot path on one MI355X.

One step is one call of every entry point on its workload:
  pointwise  qgemm_s8s8_requant  M=320 N=64 K=64 (1x1 conv, 20x16 pixels)
  s4s4       qgemm_s4s4_i32      M=N=K=4096, raw int32 out
  conv3x3    qconv2d_nhwc_s8_requant  batch 32, 56x56, 64->64, 3x3 s1 p1
  w4a8       qgemm_w4a8_requant  M=16 tokens, K=8192, N=28672 (skinny)
  w4a8_prefill  qgemm_w4a8_requant  M=2048 tokens, same weights (tiled)
  dw3x3      qdwconv2d_nhwc_s8_requant  batch 32, 56x56, 64 channels, 3x3 s1 p1
  quant_a8   qquant_per_token    8192 tokens x 8192 channels, bfloat16 -> int8
             codes + float32 scales (the s8s8 A operand; no integer ops)
  s8s8       qgemm_s8s8_requant  M=N=K=8192
  conv3x3_zp, s8s8_zp  the asymmetric calls (qconv2d_nhwc_s8_requant_zp,
             qgemm_s8s8_requant_zp) on the same arrays with zero points on
             the input, the weights and the output; their time includes the
             compensation-sum pass
Inputs are seeded synthetic arrays resident in HBM before timing starts.
Each workload rotates through enough copies of its buffers that every call
reads HBM rather than the 256 MB Infinity Cache (the pointwise case is
L2-sized and reported hot).

Prints ONE JSON line: whole-step int TOPS as `value`, per-workload times,
TOPS, GB/s and fractions of the INT8 MFMA and HBM peaks, the roofline of the
dominant kernel (HIP events on the launch stream around a graph replay of
the timed calls), and the CPU oracle timed on a bounded sample of the same
step.
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
ORDER = ["pointwise", "dw3x3", "quant_a8", "w4a8", "conv3x3", "conv3x3_zp", "s4s4",
         "w4a8_prefill", "s8s8", "s8s8_zp"]
# buffer sets per workload so that the rotation exceeds the Infinity Cache
ROTATE = {"pointwise": 1, "s4s4": 7, "conv3x3": 40, "conv3x3_zp": 40, "dw3x3": 40,
          "quant_a8": 3, "w4a8": 5, "w4a8_prefill": 3, "s8s8": 3, "s8s8_zp": 3}
KERNEL_SOURCES = {
    "s8s8": "conv_qgemm_amd/csrc/k_gemm_dma.hip",
    "s4s4": "conv_qgemm_amd/csrc/k_gemm_dma.hip",
    "pointwise": "conv_qgemm_amd/csrc/k_tile_gemm.hip",
    "conv3x3": "conv_qgemm_amd/csrc/k_conv_halo.hip",
    "w4a8": "conv_qgemm_amd/csrc/k_skinny_w4a8.hip",
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


def src_sha(path):
    h = hashlib.sha256()
    for p in (path, "conv_qgemm_amd/csrc/dev_common.hpp"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
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
        if self.name in ("w4a8", "w4a8_prefill"):
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
    Every dispatch that is not a copy kernel belongs to the workload; the
    1 GiB device copy of hbm_copy_gbs() in the same run calibrates the
    counter (factor = known bytes / what the counter reads for that copy)."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        work, copies = [], []
        for r in _csv_rows(d):
            if r.get("Counter_Name") != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            (copies if "copy" in r["Kernel_Name"].lower() else work).append(v)
        if not work or not copies:
            raise SystemExit(f"no {counter} rows for the workload or the copy kernel in {d}")
        calib = copy_bytes / max(copies)
        out[counter] = (sum(work) / len(work), calib)
    (f, cf), (w, cw) = out["FETCH_SIZE"], out["WRITE_SIZE"]
    total = f * cf + w * cw
    return (f"traffic workload={name} src_sha={src_sha(KERNEL_SOURCES[name])} "
            f"bytes_per_launch={int(total)} fetch_bytes_raw={int(f)} write_bytes_raw={int(w)} "
            f"calib_fetch={cf:.4f} calib_write={cw:.4f}")


def main():
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
    ap.add_argument("--cpu-frac", type=int, default=2)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; runs on more than one GPU are not "
              "part of it (the path shards by output channel, see the design notes)",
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
    cases = [Case(n, torch, qgemm, datagen) for n in names]
    torch.cuda.synchronize()

    # Timed region: each workload runs as its own phase, lightest first, so
    # that a workload is not measured in the power state a heavier one leaves
    # behind.  A phase is W warm-up calls, then K back-to-back eager calls
    # between two HIP events on the launch stream, then the same K calls
    # captured in a HIP graph, replayed once untimed and then 20 times with
    # an event between replays.  The first timed replay (exactly K calls) is
    # the per-launch GPU time without the Python binding's per-call host cost,
    # which decides the launch-bound pointwise case and is hidden behind the
    # GPU for the others; all 20 give the median and p99 over batches.
    stream = torch.cuda.current_stream()
    eager, graphed, spread = {}, {}, {}
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
        bmarks = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
        bmarks[0].record(stream)
        for r in range(nb):
            g.replay()
            bmarks[r + 1].record(stream)
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
    gpu_step = sum(m[0].elapsed_time(m[1]) for m in graphed.values()) * 1e-3 / args.steps

    per = {}
    total_ops = 0
    for c in cases:
        bm = graphed[c.name]
        avg = bm[0].elapsed_time(bm[1]) * 1e-3 / args.steps
        bt = sorted(bm[r].elapsed_time(bm[r + 1]) * 1e-3 / args.steps for r in range(nb))
        b_med = bt[len(bt) // 2]
        b_p99 = bt[min(len(bt) - 1, int(0.99 * len(bt)))]
        a, b = eager[c.name]
        avg_eager = a.elapsed_time(b) * 1e-3 / args.steps
        m = spread[c.name]
        times = sorted(m[i].elapsed_time(m[i + 1]) * 1e-3 for i in range(len(m) - 1))
        med = times[len(times) // 2]
        p99 = times[-1]
        tops = c.ops / avg / 1e12
        gbs = c.bytes / avg / 1e9
        per[c.name] = {"us_avg": round(avg * 1e6, 2),
                       "us_batch_median": round(b_med * 1e6, 2),
                       "us_batch_p99": round(b_p99 * 1e6, 2),
                       "us_avg_eager": round(avg_eager * 1e6, 2),
                       "us_single_median": round(med * 1e6, 2),
                       "us_single_max": round(p99 * 1e6, 2), "tops": round(tops, 2),
                       "gb_s": round(gbs, 1),
                       "pct_int8_mfma_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
                       "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                       "ops": c.ops, "alg_bytes": c.bytes,
                       "buffer_sets": ROTATE[c.name], "input_sha256": c.input_sha}
        total_ops += c.ops
    # one step = one timed call of every workload; warm-up calls are outside
    ms_per_step = gpu_step * 1e3
    value = total_ops / gpu_step / 1e12

    # the roofline describes the dominant single kernel: the longest of the
    # workloads that are one kernel launch (the asymmetric calls add a
    # compensation-sum pass in front of theirs)
    single = [n for n in per if not n.endswith("_zp")] or list(per)
    dom = max(single, key=lambda n: per[n]["us_avg"])
    mfma_bound = dom in ("s8s8", "s8s8_zp", "s4s4", "conv3x3", "conv3x3_zp", "pointwise",
                         "w4a8_prefill")
    if mfma_bound:
        achieved = per[dom]["tops"]
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": round(achieved / PEAK_INT8_TOPS, 4)}
    else:
        achieved = per[dom]["gb_s"]
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(dom)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "qgemm step: " + " + ".join(
            {"pointwise": "pointwise s8s8 320x64x64", "s4s4": "s4s4 4096^3 -> i32",
             "conv3x3": "conv3x3 NHWC 32x56x56x64->64",
             "dw3x3": "depthwise 3x3 NHWC 32x56x56x64",
             "quant_a8": "per-token quant bf16 8192x8192 -> int8",
             "w4a8": "w4a8 skinny 16x28672x8192", "s8s8": "s8s8 8192^3",
             "w4a8_prefill": "w4a8 prefill 2048x28672x8192",
             "conv3x3_zp": "conv3x3 with zero points", "s8s8_zp": "s8s8 8192^3 with zero points"}[n]
            for n in names),
                   "parallelism": "single GPU", "seeds": "numpy PCG64 1..7",
                   "timing": f"per workload: {args.warmup} warm-up calls; "
                             f"{args.steps} back-to-back calls issued eagerly from Python "
                             f"(us_avg_eager); the same {args.steps} calls captured in a "
                             f"HIP graph, replayed once untimed and {nb} times between "
                             f"HIP events (us_avg: the first timed replay, which value "
                             f"and roofline use; us_batch_median / us_batch_p99: per "
                             f"call over the {nb} replays); single-launch spread from "
                             f"20 more eager calls; wall {wall:.3f} s for all phases"},
        "per_config": per,
        "roofline": roof,
    }
    try:
        out["hbm_copy_gb_s"] = round(hbm_copy_gbs(torch), 1)
    except RuntimeError:
        out["hbm_copy_gb_s"] = None
    # the HBM-bound workloads against the rate a plain device copy reaches in
    # the same run (torch's reductions, the only plain streaming reads at
    # hand, read slower than these kernels, so the copy is the calibration)
    for n in ("w4a8", "quant_a8"):
        if n in per and out["hbm_copy_gb_s"]:
            per[n]["pct_of_copy_rate"] = round(100 * per[n]["gb_s"] / out["hbm_copy_gb_s"], 1)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(names, args.cpu_frac)
    print(json.dumps(out))


if __name__ == "__main__":
    main()

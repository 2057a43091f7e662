"""Benchmark of the MXFP4 W4A8 linear layer on one MI355X.

Step (the headline, timed K times after W warm-up steps): one decode pass of
the merged gate_up projection (N = 2 x 17408, K = 5120, MXFP4 weights
requantized on the GPU from NVFP4 with one global divisor per partition, then
repacked once into matrix-core fragment order), for each batch M in
{1, 8, 16, 64}: per-token fp8 quantization of a bf16 [M, K] activation, then the
block-scaled W4A8 GEMM -> bf16 [M, N] on the fragment-order weights, one call
of the linear entry point per M (at M = 1 one launch: the quantization runs in
the split-K decode kernel's prologue; M = 8 the quant kernel and the decode
kernel; M = 16 and 64 the quant kernel and the tiled kernel).  The step's four
linears read four different copies of the weight out of eight (95 MB each,
758 MB in all, three times the 256 MB Infinity Cache; step s uses copies
4s .. 4s + 3 mod 8), so between two reads of a copy seven others stream
through and every weight byte of a step comes from HBM (with one copy per step
the later linears found much of the weight still in the cache).  Each step is
one HIP graph replay (one graph per pair of copy sets), so host launch latency
is not in the timed region.

value = algorithmic HBM bytes of the step / step time (GB/s): per M the MXFP4
weight (codes + e8m0) plus bf16 activations read, e4m3 activations written and
read back, token scales, and the bf16 output.

Also reported, each from its own short timed loop (HIP events on the stream the
kernels run on): the decode GEMM per M, with the roofline taken on the decode
kernel at M = 1 (one kernel per call there); the prefill GEMM (M = 4096) in
TFLOP/s; the full-layer requant in GB/s for the three exponent rules, and
the bf16 / fp8-per-channel -> MXFP4 encoders on the same shape; W4A4 (MXFP4
activations) on the same weights, prefill and decode; the
down_proj decode and prefill; the int4 g128 variant; and the row-major weight
layout's GEMM for comparison.
cpu_baseline: the CPU oracle timed on a bounded sample of the same step.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

METRIC = "W4A8 MXFP4 GEMM: decode HBM GB/s (M≤64), prefill TFLOPS (M=4096); requant GB/s"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0        # MI355X dense MXFP4 (fp4 x fp4 block-scaled MFMA)
DECODE_MS = (1, 8, 16, 64)
COPIES = 8


TRAFFIC_RECORD = os.path.join(HERE, "profiles", "pdec_gate_up_m1_traffic.md")
ROOFLINE_SOURCE = os.path.join(HERE, "w4a8_gemm_amd", "csrc", "gemm_prepared.hip")
ROOFLINE_GRID = 139392          # pdec_kernel launch at gate_up M = 1: 726 workgroups x 192 threads
CALIB_BYTES = 1 << 30           # plain device-to-device copy used to scale the HBM counters


def _source_hash(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic_record():
    """HBM bytes per launch of the roofline kernel from the committed counter
    record, or None when the kernel's source has changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = dict(line.split(": ", 1) for line in f.read().splitlines()
                       if line.startswith(("traffic_bytes: ", "kernel_source_sha256: ")))
    except OSError:
        return None
    if rec.get("kernel_source_sha256", "").strip() != _source_hash(ROOFLINE_SOURCE):
        return None
    return int(rec["traffic_bytes"])


def decode_bytes(M, N, K):
    """Algorithmic bytes of act quant + GEMM at one M."""
    w = N * K // 2 + N * K // 32
    act = M * K * 2 + M * K + M * 4          # bf16 read, e4m3 written, scale written
    gemm_in = M * K + M * 4                  # e4m3 and scales read by the GEMM
    out = M * N * 2
    return w + act + gemm_in + out


def gemm_bytes(M, N, K):
    return N * K // 2 + N * K // 32 + M * K + M * 4 + M * N * 2


def requant_bytes(rows, K):
    return rows * (K // 2 + K // 16 + K // 2 + K // 32)


class Timer:
    """Average duration of `fn` (which enqueues work on the current stream),
    measured with HIP events on that stream around `reps` back-to-back calls."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps):
        t = self.torch
        s = t.cuda.current_stream()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(s)
        for i in range(reps):
            fn(i)
        b.record(s)
        b.synchronize()
        return a.elapsed_time(b) / reps * 1e-3   # seconds per call


def graph_of(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm (lazy module loading) outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill/requant/int4 loops")
    ap.add_argument("--cpu-rows", type=int, default=34816, help="weight rows in the oracle sample")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="only the launches the HBM counters are read on: a 1 GiB device copy "
                         "(calibration) and the roofline kernel (run under rocprofv3 --pmc)")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) "
                         "into the traffic record under profiles/")
    args = ap.parse_args()
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a8_gemm_amd as w4
    from w4a8_gemm_amd import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    w4.lib()
    dev = torch.device("cuda:0")
    timer = Timer(torch)
    log = lambda *m: print("[bench]", *m, file=sys.stderr, flush=True)

    # ---------------- inputs (resident in HBM before any timing) ----------------
    log("generating gate_up NVFP4 (2 x 17408 x 5120)")
    g = synth.gate_up()
    N, K = g["N"], g["K"]
    nv_p = torch.from_numpy(g["nv_packed"]).to(dev)
    nv_s = torch.from_numpy(g["nv_scale"]).to(dev)
    wp, we = w4.requant_nvfp4_to_mxfp4(nv_p, nv_s, g["part_rows"], g["part_divisor"],
                                       mode="mse", row_chunk=4096)
    pcopies = [w4.mxfp4_prepare(wp, we) for _ in range(COPIES)]
    xs_bf16 = {M: torch.from_numpy(synth.acts(M, K, seed=(1, M), spread=10.0).view(np.int16))
               .view(torch.bfloat16).to(dev) for M in DECODE_MS}
    x8 = {M: torch.empty((M, K), dtype=torch.uint8, device=dev) for M in DECODE_MS}
    xsc = {M: torch.empty((M,), dtype=torch.float32, device=dev) for M in DECODE_MS}
    out = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in DECODE_MS}
    pws = w4.Workspace(max(DECODE_MS), N, K, "prepared", dev)
    torch.cuda.synchronize()

    def gemm(M, c):
        w4.mxfp4_gemm_prepared(x8[M], xsc[M], pcopies[c], out=out[M], workspace=pws)

    if args.pmc_probe:
        pmc_probe(torch, w4, timer, graph_of, gemm, x8, xsc, xs_bf16, dev, log)
        return

    def step(c):
        # the linear on bf16 activations: the per-token quantization runs in
        # the decode kernel's prologue where it fits (M = 1), else its own
        # kernel before the GEMM; each M on its own weight copy
        for i, M in enumerate(DECODE_MS):
            w = pcopies[(len(DECODE_MS) * c + i) % COPIES]
            w4.mxfp4_linear_prepared(xs_bf16[M], w, out=out[M], workspace=pws, x8=x8[M], xs=xsc[M])

    graphs = [graph_of(torch, lambda c=c: step(c)) for c in range(COPIES)]
    step_bytes = sum(decode_bytes(M, N, K) for M in DECODE_MS)

    # ---------------- headline: K steps ----------------
    for i in range(args.warmup):
        graphs[i % COPIES].replay()
    torch.cuda.synchronize()
    t_step = timer(lambda i: graphs[i % COPIES].replay(), args.steps)
    value = step_bytes / t_step / 1e9
    log(f"step {t_step * 1e3:.4f} ms, {value:.1f} GB/s")

    # ---------------- decode GEMM kernel durations (roofline) ----------------
    per_m = {}
    R = 8 * COPIES         # launches per graph: the gap between graph replays (~8 us) spreads thin
    for M in DECODE_MS:
        def gemms(M=M):
            for r in range(R):
                gemm(M, r % COPIES)
        gg = graph_of(torch, gemms)
        gg.replay()
        dt = timer(lambda i: gg.replay(), max(2, args.steps // 4)) / R
        per_m[M] = dt
        log(f"decode GEMM M={M}: {dt * 1e6:.2f} us, {gemm_bytes(M, N, K) / dt / 1e9:.1f} GB/s")
    # roofline: the split-K decode kernel at M = 1, the largest share of the
    # step and a single kernel per GEMM call (no reduction pass)
    b1 = gemm_bytes(1, N, K)
    achieved = b1 / per_m[1] / 1e9
    roofline = {"bound": "hbm",
                "kernel": "pdec_kernel<1,2,0,4> (fragment-order split-K decode), gate_up M=1; "
                          "average over graph replays of 64 launches rotating 8 weight copies",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic_record(),
                "bytes_per_launch": b1, "avg_launch_us": round(per_m[1] * 1e6, 3),
                "gemm_call_us_by_M": {str(M): round(per_m[M] * 1e6, 3) for M in DECODE_MS},
                "gemm_call_gbps_by_M": {str(M): round(gemm_bytes(M, N, K) / per_m[M] / 1e9, 1)
                                        for M in DECODE_MS}}

    extra = {}
    if not args.no_extra:
        extra = extra_measurements(torch, w4, synth, timer, graph_of, log, nv_p, nv_s, g, wp, we,
                                   pcopies, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth, g, args.cpu_rows, log)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 x e2m1 (e8m0 block scale), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "decode gate_up: merged MXFP4 linear N=2x17408 K=5120 "
                               "(requantized from NVFP4, per-partition divisors), "
                               "M in {1,8,16,64}, fp8 per-token act quant + GEMM per M "
                               "(fragment-order weights)",
                   "N": N, "K": K, "M": list(DECODE_MS), "weight_copies_rotated": COPIES,
                   "step_bytes": step_bytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def pmc_probe(torch, w4, timer, graph_of, gemm, x8, xsc, xs_bf16, dev, log):
    """Launches for the HBM byte counters: a plain device-to-device copy of
    CALIB_BYTES (read and written once: the counters' scale), then 16
    launches of the roofline kernel (gate_up, M = 1, rotating the weight
    copies), each stream-ordered and separate."""
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(7)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w4.quant_act_fp8_per_token(xs_bf16[1], out=x8[1], scale=xsc[1])
    for r in range(16):
        gemm(1, r % COPIES)
    torch.cuda.synchronize()
    log("pmc probe done")


def pmc_summarize(fetch_dir, write_dir):
    """Traffic record of the roofline kernel from two rocprofv3 --pmc runs of
    `bench.py --pmc-probe`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of
    the roofline kernel's launches, each scaled by the factor the same counter
    reads on the calibration copy (CALIB_BYTES read and written)."""
    import csv
    import glob

    def per_dispatch(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = list(csv.DictReader(open(files[0])))
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            key = r["Dispatch_Id"]
            name, grid = r["Kernel_Name"], int(r["Grid_Size"])
            v = acc.setdefault(key, [name, grid, 0.0])
            v[2] += float(r["Counter_Value"])
        return list(acc.values())

    def pick(recs):
        copies = [v for n, g, v in recs if "copy" in n.lower() and v > 0]
        kern = [v for n, g, v in recs if "pdec_kernel" in n and g == ROOFLINE_GRID]
        if not copies or not kern:
            raise SystemExit("calibration copy or roofline kernel dispatches not found")
        return max(copies), kern

    fc, fk = pick(per_dispatch(fetch_dir, "FETCH_SIZE"))
    wc, wk = pick(per_dispatch(write_dir, "WRITE_SIZE"))
    f_scale = fc * 1024 / CALIB_BYTES          # counter bytes per true byte read
    w_scale = wc * 1024 / CALIB_BYTES          # counter bytes per true byte written
    fetch = sum(fk) / len(fk) * 1024 / f_scale
    write = sum(wk) / len(wk) * 1024 / w_scale
    algo = gemm_bytes(1, 34816, 5120)
    lines = [
        "# HBM traffic of pdec_kernel, gate_up M = 1 (roofline kernel of bench.py)",
        "",
        "Commands (repository root, one MI355X):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_fetch -o run -- python -u bench.py --pmc-probe",
        "    rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_write -o run -- python -u bench.py --pmc-probe",
        "    python bench.py --pmc-summarize gpurun_out/pmc_fetch gpurun_out/pmc_write",
        "",
        f"Calibration: a {CALIB_BYTES} B device-to-device copy reads FETCH_SIZE {fc:.0f} KiB "
        f"(scale {f_scale:.4f}) and WRITE_SIZE {wc:.0f} KiB (scale {w_scale:.4f}).",
        f"Roofline kernel: {len(fk)} / {len(wk)} dispatches, mean FETCH_SIZE {sum(fk) / len(fk):.0f} KiB, "
        f"mean WRITE_SIZE {sum(wk) / len(wk):.0f} KiB.",
        f"Scaled HBM bytes per launch: read {fetch:.0f}, written {write:.0f}; "
        f"algorithmic bytes {algo} (ratio {(fetch + write) / algo:.4f}).",
        "",
        f"traffic_bytes: {int(round(fetch + write))}",
        f"kernel_source_sha256: {_source_hash(ROOFLINE_SOURCE)}",
    ]
    with open(TRAFFIC_RECORD, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _timed_graph(torch, timer, graph_of, calls, reps):
    """Average duration of one call: `calls` is a list of closures replayed as
    one graph; the graph is replayed `reps` times after one untimed replay."""
    gg = graph_of(torch, lambda: [c() for c in calls])
    gg.replay()
    return timer(lambda i: gg.replay(), reps) / len(calls)


def extra_measurements(torch, w4, synth, timer, graph_of, log, nv_p, nv_s, g, wp, we, pcopies, dev):
    N, K = g["N"], g["K"]
    res = {}
    # prefill: M = 4096 against the gate_up weight (fragment order, tiled kernel)
    M = 4096
    xb = torch.from_numpy(synth.acts(M, K, seed=3).view(np.int16)).view(torch.bfloat16).to(dev)
    x8, xs = w4.quant_act_fp8_per_token(xb)
    o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * M * N * K
    dt = _timed_graph(torch, timer, graph_of,
                      [lambda r=r: w4.mxfp4_gemm_prepared(x8, xs, pcopies[r], out=o) for r in range(4)], 5)
    res["prefill_gemm"] = {"M": M, "N": N, "K": K, "kernel": "pf_kernel<256>", "us": round(dt * 1e6, 2),
                           "tflops": round(flops / dt / 1e12, 1),
                           "frac_of_fp8_peak": round(flops / dt / 1e12 / FP8_PEAK_TFLOPS, 4)}
    log("prefill", res["prefill_gemm"])
    aq = timer(lambda i: w4.quant_act_fp8_per_token(xb, out=x8, scale=xs), 5)
    res["act_quant_prefill"] = {"M": M, "K": K, "us": round(aq * 1e6, 2),
                                "gbps": round((M * K * 3 + M * 4) / aq / 1e9, 1)}
    # W4A4 (MXFP4 activations, OCP rule) on the same prepared weights: the
    # activation quant and the fp4 x fp4 GEMM, prefill M = 4096 and decode M = 1
    xa4, xe4 = w4.quant_act_mxfp4(xb)
    aq4 = timer(lambda i: w4.quant_act_mxfp4(xb), 5)
    dt4 = _timed_graph(torch, timer, graph_of,
                       [lambda r=r: w4.w4a4_gemm_prepared(xa4, xe4, pcopies[r], out=o) for r in range(4)], 5)
    res["w4a4"] = {"prefill_M4096": {"us": round(dt4 * 1e6, 2), "tflops": round(flops / dt4 / 1e12, 1),
                                     "frac_of_fp4_peak": round(flops / dt4 / 1e12 / FP4_PEAK_TFLOPS, 4)},
                   "act_quant_mxfp4_M4096_us": round(aq4 * 1e6, 2)}
    # decode-sized M: the split-K decode kernel with fp4 activations
    ws4 = w4.Workspace(32, N, K, "w4a4", dev)
    for Md in (1, 32):
        xad, xed = w4.quant_act_mxfp4(xb[:Md].contiguous())
        od = torch.empty((Md, N), dtype=torch.bfloat16, device=dev)
        dtd = _timed_graph(torch, timer, graph_of,
                           [lambda r=r: w4.w4a4_gemm_prepared(xad, xed, pcopies[r], out=od, workspace=ws4)
                            for r in range(len(pcopies))], 10)
        bd = N * K // 2 + N * K // 32 + Md * (K // 2 + K // 32) + 2 * Md * N
        res["w4a4"][f"decode_M{Md}"] = {"us": round(dtd * 1e6, 2), "gbps": round(bd / dtd / 1e9, 1)}
    log("w4a4", res["w4a4"])
    del xa4, xe4
    # the row-major weight layout (no repack), for comparison: M = 1 and 4096
    rm = {}
    rcopies = [(wp, we)] + [(wp.clone(), we.clone()) for _ in range(7)]
    rws = w4.Workspace(1, N, K, "mxfp4", dev)
    x1, s1 = w4.quant_act_fp8_per_token(xb[:1].contiguous())
    o1 = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
    dt1 = _timed_graph(torch, timer, graph_of,
                       [lambda r=r: w4.mxfp4_gemm(x1, s1, rcopies[r][0], rcopies[r][1], out=o1, workspace=rws)
                        for r in range(len(rcopies))], 10)
    rm["decode_M1"] = {"us": round(dt1 * 1e6, 2), "gbps": round(gemm_bytes(1, N, K) / dt1 / 1e9, 1)}
    dtp = _timed_graph(torch, timer, graph_of,
                       [lambda r=r: w4.mxfp4_gemm(x8, xs, rcopies[r][0], rcopies[r][1], out=o) for r in range(2)], 3)
    rm["prefill_M4096"] = {"us": round(dtp * 1e6, 2), "tflops": round(flops / dtp / 1e12, 1)}
    res["rowmajor_layout_gemm"] = rm
    log("row-major layout", rm)
    del o, xb, rcopies
    # full-layer requant, three rules, ROW_CHUNK passes and one pass per partition
    src = [(nv_p, nv_s), (nv_p.clone(), nv_s.clone())]
    outs = [(torch.empty_like(wp), torch.empty_like(we)) for _ in range(2)]
    rq = {}
    for mode in ("ocp", "noclip", "mse"):
        for chunk in (4096, 0):
            def run(i, mode=mode, chunk=chunk):
                p, s = src[i % 2]
                op, oe = outs[i % 2]
                w4.requant_nvfp4_to_mxfp4(p, s, g["part_rows"], g["part_divisor"], mode=mode,
                                          row_chunk=chunk, out_packed=op, out_e8m0=oe)
            rg = [graph_of(torch, lambda i=i: run(i)) for i in range(2)]
            dt = timer(lambda i: rg[i % 2].replay(), 6)
            rq[f"{mode}_chunk{chunk}"] = {"us": round(dt * 1e6, 1),
                                          "gbps": round(requant_bytes(N, K) / dt / 1e9, 1)}
    res["requant_full_layer"] = rq
    log("requant", rq)
    del src, outs
    # bf16 and fp8 per-channel weights of the same shape -> MXFP4 (the requant
    # encoder with other input stages), two input copies alternating
    lq = {}
    wb = torch.from_numpy(synth.bf16_weight(N, K).view(np.int16)).view(torch.bfloat16).to(dev)
    bsrc = [wb, wb.clone()]
    del wb
    f8 = synth.fp8ch_weight(N, K)
    w8 = torch.from_numpy(f8["w8"]).to(dev)
    rs = torch.from_numpy(f8["row_scale"]).to(dev)
    fsrc = [(w8, rs), (w8.clone(), rs.clone())]
    del w8, f8
    outs = [(torch.empty_like(wp), torch.empty_like(we)) for _ in range(2)]
    for mode in ("ocp", "mse"):
        def run_b(i, mode=mode):
            w4.quant_bf16_to_mxfp4(bsrc[i % 2], mode=mode, out_packed=outs[i % 2][0], out_e8m0=outs[i % 2][1])

        def run_f(i, mode=mode):
            w4.quant_fp8ch_to_mxfp4(fsrc[i % 2][0], fsrc[i % 2][1], mode=mode, out_packed=outs[i % 2][0],
                                    out_e8m0=outs[i % 2][1])
        for name, run, nbytes in (("bf16", run_b, N * K * 2 + N * K // 2 + N * K // 32),
                                  ("fp8ch", run_f, N * K + 4 * N + N * K // 2 + N * K // 32)):
            rg = [graph_of(torch, lambda i=i, run=run: run(i)) for i in range(2)]
            dt = timer(lambda i: rg[i % 2].replay(), 6)
            lq[f"{name}_{mode}"] = {"us": round(dt * 1e6, 1), "gbps": round(nbytes / dt / 1e9, 1)}
    res["load_quant_full_layer"] = lq
    log("bf16 / fp8 -> mxfp4", lq)
    del bsrc, fsrc, outs
    # down_proj (K = 17408), fragment-order weights, eight copies
    d = synth.down_proj()
    dw = torch.from_numpy(d["w_packed"]).to(dev)
    de = torch.from_numpy(d["w_e8m0"]).to(dev)
    pdc = [w4.mxfp4_prepare(dw, de) for _ in range(8)]
    pdws = w4.Workspace(64, d["N"], d["K"], "prepared", dev)
    pdp = {}
    for M in (1, 16, 64, 4096):
        xb = torch.from_numpy(synth.acts(M, d["K"], seed=(2, M)).view(np.int16)).view(torch.bfloat16).to(dev)
        a8, asc = w4.quant_act_fp8_per_token(xb)
        oo = torch.empty((M, d["N"]), dtype=torch.bfloat16, device=dev)
        reps = 8 if M <= 64 else 2
        dt = _timed_graph(torch, timer, graph_of,
                          [lambda r=r: w4.mxfp4_gemm_prepared(a8, asc, pdc[r], out=oo, workspace=pdws)
                           for r in range(reps)], 10 if M <= 64 else 3)
        b = gemm_bytes(M, d["N"], d["K"])
        ent = {"us": round(dt * 1e6, 2), "gbps": round(b / dt / 1e9, 1),
               "frac_of_hbm": round(b / dt / 1e9 / HBM_PEAK_GBS, 4)}
        if M > 64:
            fl = 2.0 * M * d["N"] * d["K"]
            ent["tflops"] = round(fl / dt / 1e12, 1)
            ent["frac_of_fp8_peak"] = round(fl / dt / 1e12 / FP8_PEAK_TFLOPS, 4)
        pdp[str(M)] = ent
    res["down_proj_prepared"] = pdp
    log("down_proj prepared", pdp)
    del pdc, dw, de
    # int4 g128 (symmetric, then with zero points) and int5 g128, fragment order, eight copies
    def to_dev(a, half=False):
        t = torch.from_numpy(a.view(np.int16) if half else a)
        return (t.view(torch.float16) if half else t).to(dev)

    def int_family(q, prep, gemm, kind, extra_bits):
        copies = [prep(q) for _ in range(8)]
        ws = w4.Workspace(2048, q["N"], q["K"], kind, dev)
        out = {}
        for M in (1, 16, 64, 2048):
            xb = torch.from_numpy(synth.acts(M, q["K"], seed=(4, M)).view(np.int16)).view(torch.bfloat16).to(dev)
            a8, asc = w4.quant_act_fp8_per_token(xb)
            oo = torch.empty((M, q["N"]), dtype=torch.bfloat16, device=dev)
            reps = 8 if M <= 64 else 2
            dt = _timed_graph(torch, timer, graph_of,
                              [lambda r=r: gemm(a8, asc, copies[r], out=oo, workspace=ws)
                               for r in range(reps)], 10 if M <= 64 else 3)
            # codes (4 or 5 bits), fp16 scale + zero nibble per group, activations, output
            b = (q["N"] * q["K"] * extra_bits // 8 + q["N"] * q["K"] // 64 + M * q["K"] + M * 4
                 + M * q["N"] * 2)
            ent = {"us": round(dt * 1e6, 2), "gbps": round(b / dt / 1e9, 1),
                   "frac_of_hbm": round(b / dt / 1e9 / HBM_PEAK_GBS, 4)}
            if M > 64:
                fl = 2.0 * M * q["N"] * q["K"]
                ent["tflops"] = round(fl / dt / 1e12, 1)
                ent["frac_of_fp8_peak"] = round(fl / dt / 1e12 / FP8_PEAK_TFLOPS, 4)
            out[str(M)] = ent
        del copies
        return out

    i4 = int_family(synth.int4(), lambda q: w4.int4g128_prepare_fragments(
        to_dev(q["qweight_kn"]), to_dev(q["qzeros"]), to_dev(q["scales"], True)),
        w4.int4g128_gemm_prepared, "int4_prepared", 4)
    res["int4_g128"] = i4
    log("int4", i4)
    i4z = int_family(synth.int4_zp(), lambda q: w4.int4g128_zp_prepare_fragments(
        to_dev(q["qweight_kn"]), to_dev(q["qzeros"]), to_dev(q["scales"], True)),
        w4.int4g128_zp_gemm_prepared, "int4_zp_prepared", 4)
    res["int4_g128_zp"] = i4z
    log("int4 zp", i4z)
    i5 = int_family(synth.int5(), lambda q: w4.int5g128_prepare_fragments(
        to_dev(q["qweight_kn"]), to_dev(q["qweight_hi"]), to_dev(q["qzeros"]), to_dev(q["scales"], True)),
        w4.int5g128_gemm_prepared, "int5_prepared", 5)
    res["int5_g128"] = i5
    log("int5", i5)
    return res


def cpu_baseline(synth, g, rows, log):
    """The CPU oracle (as it stands) on a sample of the headline step: the same
    activations for M in {1, 8, 16, 64}, against the first `rows` weight rows."""
    import oracle
    N, K = g["N"], g["K"]
    rows = min(rows, N)
    half = rows // 2
    sel = np.r_[0:half, N // 2:N // 2 + rows - half]
    mp, me, _ = oracle.requant_nvfp4_to_mxfp4(g["nv_packed"][sel], g["nv_scale"][sel],
                                              [half, rows - half], g["part_divisor"], mode="mse")
    xs = {M: synth.acts(M, K, seed=(1, M), spread=10.0) for M in DECODE_MS}
    t0 = time.perf_counter()
    for M in DECODE_MS:
        a8, s = oracle.quant_act_fp8(xs[M])
        oracle.mxfp4_gemm(a8, s, mp, me)
    dt = time.perf_counter() - t0
    b = sum(decode_bytes(M, rows, K) for M in DECODE_MS)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    res = {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds": round(dt, 2),
           "sample": f"headline step on {rows} of {N} weight rows (both partitions), "
                     "M in {1,8,16,64}: oracle fp8 act quant + fp64 GEMM reference"}
    log("cpu baseline", res)
    return res


if __name__ == "__main__":
    main()

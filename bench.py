#!/usr/bin/env python3
"""Benchmark of the MXFP8 path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. fused Gemma RMSNorm -> MXFP8 of x [1024, 6144] (linear + swizzled scales),
  2. per-rank down_proj chain: BF16 activations [32768, 3072] quantised on the fly (swizzled
     scales) and multiplied by pre-quantised weights [6144, 3072] -> BF16 [32768, 6144] in 4
     row chunks,
  3. the same for o_proj with K = 2048.
Inputs are resident in HBM before the timed region. `value` is the step's GEMM work
(2 M N K summed over both GEMMs) divided by the step time, so the quantisers and the norm
count against it. The timed steps record HIP events on the launch stream around the K = 3072
GEMM only (the roofline kernel; six events per step cost about 1% of the step); the per-kernel
breakdown comes from as many steps again, run right after with events around every kernel.

Prints one JSON line. `--sweep` instead prints one JSON line per GEMM / quantiser shape of
the pages' sweeps (each timed in isolation with a 512 MiB cache flush between launches).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM TFLOP/s (K=2048/3072, N=6144, M=1k-32k) + % MFMA peak; quant GB/s"
PEAK_MFMA_FP8_TFLOPS = 5000.0   # MI355X dense FP8/MXFP8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
N_MODEL = 6144
M_CHAIN = 32768
K_DOWN, K_O = 3072, 2048
NORM_ROWS = 1024
CHUNKS = 4


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sweep", action="store_true", help="per-shape GEMM/quantiser lines instead of the step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one 1 GiB device-to-device copy first (the reference kernel that scales the "
                        "FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    return p.parse_args()


# HBM traffic of one launch of the K=3072 GEMM, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by the factor that maps the
# counter of a 1 GiB copy onto 1 GiB. Valid only for the kernel code it was taken on
# (gemm_code_sha256).
GEMM_TRAFFIC = {
    "source_sha256": "e6b96aea36e5a662e0b56db1d332fd69cfc18d062228c53482eb1b698d67f96e",
    "fetch_kib": 457283.0, "write_kib": 393356.5,
    "fetch_factor": 2.0, "write_factor": 1.0,
}


def gemm_code_sha256():
    """SHA-256 of gemm.hip with comments and whitespace removed: the kernel code the traffic
    figures belong to (a comment edit does not invalidate them, a code edit does)."""
    import hashlib
    import re
    src = os.path.join(ROOT, "quant_mxfp8_gemm_amd", "csrc", "gemm.hip")
    try:
        text = open(src).read()
    except OSError:
        return None
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return hashlib.sha256("".join(text.split()).encode()).hexdigest()


def gemm_traffic_bytes():
    sha = gemm_code_sha256()
    t = GEMM_TRAFFIC
    if t["source_sha256"] != sha or t["fetch_kib"] is None or t["write_kib"] is None:
        return None
    return int(round((t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"]) * 1024))


def gemm_bytes(m, n, k):
    """Algorithmic HBM bytes of one GEMM: A and B codes, both scale sets, BF16 C."""
    return m * k + n * k + (m + n) * (k // 32) + 2 * m * n


def quant_bytes(rows, k, layouts=1):
    """Algorithmic bytes of the quantiser: BF16 in, E4M3 out, one byte per 32 per scale layout."""
    return rows * k * 2 + rows * k + layouts * rows * (k // 32)


def norm_bytes(rows, h):
    return rows * h * 2 + h * 2 + rows * h + 2 * rows * (h // 32)


def cpu_baseline(target_s):
    """The oracle, untuned, on the host cores: the same chain on the first rows of the batch."""
    import numpy as np
    import oracle
    import synth

    def bits(t):
        return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)

    w_d = synth.weights_bf16(N_MODEL, K_DOWN, seed=1)
    w_o = synth.weights_bf16(N_MODEL, K_O, seed=1)
    qd, _, sd = oracle.quantize(bits(w_d))
    qo, _, so = oracle.quantize(bits(w_o))
    x, w = synth.norm_inputs_bf16(NORM_ROWS, N_MODEL)

    def run(rows):
        a_d = synth.activations_bf16(rows, K_DOWN, seed=0)
        a_o = synth.activations_bf16(rows, K_O, seed=0)
        t0 = time.perf_counter()
        oracle.rmsnorm_quant(bits(x[:max(1, rows * NORM_ROWS // M_CHAIN)]), bits(w), float(np.float32(1e-6)))
        qa, _, sa = oracle.quantize(bits(a_d))
        oracle.gemm(qa, sa, oracle.SWIZZLED, qd, sd, oracle.SWIZZLED)
        qa, _, sa = oracle.quantize(bits(a_o))
        oracle.gemm(qa, sa, oracle.SWIZZLED, qo, so, oracle.SWIZZLED)
        return time.perf_counter() - t0

    probe_rows = 16
    t = run(probe_rows)
    rows = int(max(probe_rows, min(M_CHAIN, probe_rows * target_s / max(t, 1e-3))))
    rows = max(16, rows // 16 * 16)
    t = run(rows)
    flops = 2.0 * rows * N_MODEL * (K_DOWN + K_O)
    cores = oracle.num_threads()
    # the same code on one thread, on a sample a sixteenth the size
    prev = oracle.set_num_threads(1)
    rows1 = max(16, rows // 16 // 16 * 16)
    t1 = run(rows1)
    oracle.set_num_threads(prev)
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"first {rows} of {M_CHAIN} rows of the step (norm rows scaled alike), fp64 oracle, "
                      f"{t:.1f} s",
            "one_thread": {"value": 2.0 * rows1 * N_MODEL * (K_DOWN + K_O) / t1 / 1e12, "unit": "TFLOP/s",
                           "sample": f"first {rows1} rows, {t1:.1f} s"}}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the reduce-scatter that would follow the chunked GEMM is not part of it).", file=sys.stderr)
        sys.exit(2)

    import torch

    import quant_mxfp8_gemm_amd as mx
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mx.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.sweep:
        return sweep(args, mx, synth, torch, dev)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- resident inputs (untimed): activations, norm input, pre-quantised weights
    x, w = synth.norm_inputs_bf16(NORM_ROWS, N_MODEL)
    x, w = x.to(dev), w.to(dev)
    a_d = synth.activations_bf16(M_CHAIN, K_DOWN, seed=0).to(dev)
    a_o = synth.activations_bf16(M_CHAIN, K_O, seed=0).to(dev)
    wq_d, _, ws_d = mx.quantize(synth.weights_bf16(N_MODEL, K_DOWN, seed=1).to(dev), linear=False)
    wq_o, _, ws_o = mx.quantize(synth.weights_bf16(N_MODEL, K_O, seed=1).to(dev), linear=False)
    # outputs, allocated once
    nq = (torch.empty((NORM_ROWS, N_MODEL), dtype=torch.uint8, device=dev),
          torch.empty((NORM_ROWS, N_MODEL // 32), dtype=torch.uint8, device=dev),
          torch.empty(mx.scale_bytes(NORM_ROWS, N_MODEL, mx.SWIZZLED), dtype=torch.uint8, device=dev))
    qd = (torch.empty((M_CHAIN, K_DOWN), dtype=torch.uint8, device=dev), None,
          torch.empty(mx.scale_bytes(M_CHAIN, K_DOWN, mx.SWIZZLED), dtype=torch.uint8, device=dev))
    qo = (torch.empty((M_CHAIN, K_O), dtype=torch.uint8, device=dev), None,
          torch.empty(mx.scale_bytes(M_CHAIN, K_O, mx.SWIZZLED), dtype=torch.uint8, device=dev))
    c_d = torch.empty((M_CHAIN, N_MODEL), dtype=torch.bfloat16, device=dev)
    c_o = torch.empty((M_CHAIN, N_MODEL), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    n_ev = 6
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    roof_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]

    def step(ev=None, roof=None):
        if ev:
            ev[0].record()
        mx.rmsnorm_quant(x, w, 1e-6, out=nq)
        if ev:
            ev[1].record()
        mx.quantize(a_d, linear=False, out=qd)
        if ev:
            ev[2].record()
        if roof:
            roof[0].record()
        mx.gemm(qd[0], qd[2], mx.SWIZZLED, wq_d, ws_d, mx.SWIZZLED, out=c_d, num_chunks=CHUNKS)
        if roof:
            roof[1].record()
        if ev:
            ev[3].record()
        mx.quantize(a_o, linear=False, out=qo)
        if ev:
            ev[4].record()
        mx.gemm(qo[0], qo[2], mx.SWIZZLED, wq_o, ws_o, mx.SWIZZLED, out=c_o, num_chunks=CHUNKS)
        if ev:
            ev[5].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(roof=roof_ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] {args.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)
    # per-kernel breakdown: the same steps again, events around every kernel (not timed)
    for i in range(args.steps):
        step(ev=events[i])
    torch.cuda.synchronize()

    def avg(a, b):
        return sum(events[i][a].elapsed_time(events[i][b]) for i in range(args.steps)) / args.steps / 1e3

    def pct(a, b):
        """Median, p10 and p90 of one kernel's event durations over the timed steps (seconds)."""
        ts = sorted(events[i][a].elapsed_time(events[i][b]) / 1e3 for i in range(args.steps))
        return ts[len(ts) // 2], ts[len(ts) // 10], ts[min(len(ts) - 1, (9 * len(ts)) // 10)]

    t_norm, t_qd, t_gd, t_qo, t_go = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4), avg(4, 5)
    # the roofline kernel from the timed steps themselves
    t_roof = sum(roof_ev[i][0].elapsed_time(roof_ev[i][1]) for i in range(args.steps)) / args.steps / 1e3
    ms_step = elapsed / args.steps * 1e3
    flops_d = 2.0 * M_CHAIN * N_MODEL * K_DOWN
    flops_o = 2.0 * M_CHAIN * N_MODEL * K_O
    value = (flops_d + flops_o) / (elapsed / args.steps) / 1e12
    achieved = flops_d / t_roof / 1e12
    kernels = {
        "rmsnorm_quant_1024x6144": {"us": t_norm * 1e6, "GB/s": norm_bytes(NORM_ROWS, N_MODEL) / t_norm / 1e9,
                                    "frac_hbm": norm_bytes(NORM_ROWS, N_MODEL) / t_norm / 1e9 / PEAK_HBM_GBS},
        "quantize_32768x3072": {"us": t_qd * 1e6, "GB/s": quant_bytes(M_CHAIN, K_DOWN) / t_qd / 1e9,
                                "frac_hbm": quant_bytes(M_CHAIN, K_DOWN) / t_qd / 1e9 / PEAK_HBM_GBS},
        "gemm_32768x6144x3072": {"us": t_gd * 1e6, "TFLOP/s": flops_d / t_gd / 1e12,
                                 "frac_mfma": flops_d / t_gd / 1e12 / PEAK_MFMA_FP8_TFLOPS},
        "quantize_32768x2048": {"us": t_qo * 1e6, "GB/s": quant_bytes(M_CHAIN, K_O) / t_qo / 1e9,
                                "frac_hbm": quant_bytes(M_CHAIN, K_O) / t_qo / 1e9 / PEAK_HBM_GBS},
        "gemm_32768x6144x2048": {"us": t_go * 1e6, "TFLOP/s": flops_o / t_go / 1e12,
                                 "frac_mfma": flops_o / t_go / 1e12 / PEAK_MFMA_FP8_TFLOPS},
    }
    # median / p10 / p90 of each kernel's event durations (microseconds) beside the means above
    for name, (a, b) in (("rmsnorm_quant_1024x6144", (0, 1)), ("quantize_32768x3072", (1, 2)),
                         ("gemm_32768x6144x3072", (2, 3)), ("quantize_32768x2048", (3, 4)),
                         ("gemm_32768x6144x2048", (4, 5))):
        med, p10, p90 = pct(a, b)
        kernels[name].update({"us_median": med * 1e6, "us_p10": p10 * 1e6, "us_p90": p90 * 1e6})
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "per-rank MXFP8 chain M=32768 (quantise BF16 activations + GEMM, "
                               "K=3072 down_proj and K=2048 o_proj, N=6144, 4 row chunks, 128x4-swizzled "
                               "UE8M0 scales) + fused Gemma RMSNorm quantiser [1024, 6144]",
                   "m": M_CHAIN, "n": N_MODEL, "k": [K_DOWN, K_O], "num_chunks": CHUNKS,
                   "norm_rows": NORM_ROWS, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_FP8_TFLOPS, 4),
                     "traffic": gemm_traffic_bytes(),
                     "kernel": "gemm 32768x6144x3072", "us": round(t_roof * 1e6, 3)},
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def sweep(args, mx, synth, torch, dev):
    # evict the 256 MB MALL and the L2 with a 512 MiB read (a read leaves no dirty lines behind
    # whose write-back would be charged to the next timed kernel)
    flush = torch.ones(64 << 20, dtype=torch.int64, device=dev)
    flush_out = torch.empty((), dtype=torch.int64, device=dev)

    def timed(fn, iters):
        ts = []
        for _ in range(iters):
            torch.sum(flush, dim=0, out=flush_out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        ts.sort()
        return ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]

    # K = 2048 mid-M shapes with both scale layouts (swizzled is the workload's: the step
    # quantises its activations that way)
    shapes = [(32, 2048, mx.LINEAR, 1), (128, 2048, mx.LINEAR, 1)] \
        + [(m, 2048, mx.LINEAR, 4) for m in (512, 768, 1024, 1536, 2048, 4096)] \
        + [(m, 2048, mx.SWIZZLED, 4) for m in (2048, 4096)] \
        + [(m, 3072, mx.SWIZZLED, 4) for m in (1024, 4096, 8192, 16384, 32768)] + [(32768, 2048, mx.SWIZZLED, 4)]
    wq = {}
    for k in (2048, 3072):
        q, sl, ss = mx.quantize(synth.weights_bf16(N_MODEL, k, seed=1).to(dev))
        wq[k] = (q, {mx.LINEAR: sl, mx.SWIZZLED: ss})
    for m, k, layout, chunks in shapes:
        a = synth.activations_bf16(m, k, seed=0).to(dev)
        qa, sl, ss = mx.quantize(a)
        sa = {mx.LINEAR: sl, mx.SWIZZLED: ss}[layout]
        c = torch.empty((m, N_MODEL), dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup):
            mx.gemm(qa, sa, layout, wq[k][0], wq[k][1][layout], layout, out=c, num_chunks=chunks)
        med, p10, p90 = timed(lambda: mx.gemm(qa, sa, layout, wq[k][0], wq[k][1][layout], layout, out=c,
                                               num_chunks=chunks), max(args.steps, 10))
        tf = 2.0 * m * N_MODEL * k / med / 1e12
        print(json.dumps({"kind": "gemm", "m": m, "n": N_MODEL, "k": k, "layout": "swizzled" if layout else "linear",
                          "num_chunks": chunks, "us_median": round(med * 1e6, 2), "us_p10": round(p10 * 1e6, 2),
                          "us_p90": round(p90 * 1e6, 2), "TFLOP/s": round(tf, 1),
                          "frac_mfma": round(tf / PEAK_MFMA_FP8_TFLOPS, 4),
                          "GB/s": round(gemm_bytes(m, N_MODEL, k) / med / 1e9, 1)}), flush=True)
        if m == 32768:
            out = (torch.empty_like(qa), None, torch.empty_like(ss))
            med, p10, p90 = timed(lambda: mx.quantize(a, linear=False, out=out), max(args.steps, 10))
            gbs = quant_bytes(m, k) / med / 1e9
            print(json.dumps({"kind": "quantize", "rows": m, "k": k, "us_median": round(med * 1e6, 2),
                              "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}), flush=True)
        del a, qa, sl, ss, c
    x, w = synth.norm_inputs_bf16(NORM_ROWS, N_MODEL)
    x, w = x.to(dev), w.to(dev)
    med, p10, p90 = timed(lambda: mx.rmsnorm_quant(x, w, 1e-6), max(args.steps, 10))
    gbs = norm_bytes(NORM_ROWS, N_MODEL) / med / 1e9
    print(json.dumps({"kind": "rmsnorm_quant", "rows": NORM_ROWS, "hidden": N_MODEL, "us_median": round(med * 1e6, 2),
                      "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}), flush=True)
    # residual add + norm quantiser (the decode fusion without its all-reduce)
    for rows in (128, NORM_ROWS):
        xr, wr = synth.norm_inputs_bf16(rows, N_MODEL)
        xr, wr = xr.to(dev), wr.to(dev)
        res = synth.normal_bf16((rows, N_MODEL), sigma=2.0, seed=9).to(dev)
        med, p10, p90 = timed(lambda: mx.add_rmsnorm_quant(xr, res, wr, 1e-6), max(args.steps, 10))
        nbytes = norm_bytes(rows, N_MODEL) + 4 * rows * N_MODEL  # + residual read and write
        gbs = nbytes / med / 1e9
        print(json.dumps({"kind": "add_rmsnorm_quant", "rows": rows, "hidden": N_MODEL,
                          "us_median": round(med * 1e6, 2), "GB/s": round(gbs, 1),
                          "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}), flush=True)
    # fused dense GEMM1: gate_up [2 * 3072, 6144] GEMM + SiLU(gate) * up + MXFP8 quantisation
    inter, hidden = K_DOWN, N_MODEL
    wq_gu, _, ws_gu = mx.quantize(synth.weights_bf16(2 * inter, hidden, seed=1).to(dev), linear=False)
    for m in (1024, 4096, 32768):
        qa, _, sa = mx.quantize(synth.activations_bf16(m, hidden, seed=0).to(dev), linear=False)
        out = (torch.empty((m, inter), dtype=torch.uint8, device=dev), None,
               torch.empty(mx.scale_bytes(m, inter, mx.SWIZZLED), dtype=torch.uint8, device=dev))
        for _ in range(args.warmup):
            mx.gemm_silu_mul_quant(qa, sa, mx.SWIZZLED, wq_gu, ws_gu, mx.SWIZZLED, out=out)
        med, p10, p90 = timed(lambda: mx.gemm_silu_mul_quant(qa, sa, mx.SWIZZLED, wq_gu, ws_gu, mx.SWIZZLED, out=out),
                              max(args.steps, 10))
        tf = 2.0 * m * 2 * inter * hidden / med / 1e12
        print(json.dumps({"kind": "gemm_silu_mul_quant", "m": m, "n": 2 * inter, "k": hidden,
                          "us_median": round(med * 1e6, 2), "us_p10": round(p10 * 1e6, 2), "us_p90": round(p90 * 1e6, 2),
                          "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / PEAK_MFMA_FP8_TFLOPS, 4)}), flush=True)
        del qa, sa, out
    # the platform's own MXFP8 GEMM on the headline shape, for context: torch._scaled_mm with
    # E8M0 block scales (served by hipBLASLt), same codes and scale values as this library's run
    try:
        m, k = M_CHAIN, K_DOWN
        qa, sl, _ = mx.quantize(synth.activations_bf16(m, k, seed=0).to(dev), swizzled=False)
        qb, tl, _ = mx.quantize(synth.weights_bf16(N_MODEL, k, seed=1).to(dev), swizzled=False)
        fa, fb = qa.view(torch.float8_e4m3fn), qb.view(torch.float8_e4m3fn)
        e8a, e8b = sl.view(torch.float8_e8m0fnu), tl.view(torch.float8_e8m0fnu)
        vendor = lambda: torch._scaled_mm(fa, fb.t(), scale_a=e8a, scale_b=e8b, out_dtype=torch.bfloat16)
        vendor()
        med, p10, p90 = timed(vendor, max(args.steps, 10))
        tf = 2.0 * m * N_MODEL * k / med / 1e12
        print(json.dumps({"kind": "vendor_scaled_mm_mxfp8", "m": m, "n": N_MODEL, "k": k,
                          "us_median": round(med * 1e6, 2), "TFLOP/s": round(tf, 1),
                          "frac_mfma": round(tf / PEAK_MFMA_FP8_TFLOPS, 4)}), flush=True)
        del qa, qb, sl, tl
    except Exception as e:  # the vendor path is context only
        print(json.dumps({"kind": "vendor_scaled_mm_mxfp8", "error": repr(e)[:200]}), flush=True)
    # swizzle after a row gather: linear scales of the gathered activation -> 128x4 layout
    for rows, k in ((NORM_ROWS, N_MODEL), (M_CHAIN, K_DOWN)):
        s_lin = torch.randint(0, 256, (rows, k // 32), dtype=torch.uint8, device=dev)
        s_out = torch.empty(mx.scale_bytes(rows, k, mx.SWIZZLED), dtype=torch.uint8, device=dev)
        med, p10, p90 = timed(lambda: mx.swizzle_scales(s_lin, out=s_out), max(args.steps, 10))
        gbs = (s_lin.numel() + s_out.numel()) / med / 1e9
        print(json.dumps({"kind": "swizzle_scales", "rows": rows, "k": k, "us_median": round(med * 1e6, 2),
                          "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}), flush=True)


if __name__ == "__main__":
    main()

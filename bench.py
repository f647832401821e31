"""Benchmark: one step = one fftconv_fwd call over a whole synthetic batch.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all] [--pass fwd|bwd|taps]

Prints ONE JSON line (stdout).  By default (--workload all) every one of the
five configurations the metric spans (N = 1K .. 4M) is measured in turn:
ungated_fp32_n1k, gated_fp16_n1k, gated_bf16_n16k, ungated_fp16_n1m and
partial_sparse_n4m.  The line's headline (value, ms_per_step, config,
roofline, cpu_baseline) is the largest, partial_sparse_n4m; the list
"workloads" holds the same figures for all five, and "target_n16k" compares
the N = 16K configuration with half of the HBM peak.

Inputs are seeded synthetic data already resident in HBM; the filter is
prepared once before timing (it depends only on k).  `value` is B*H*N
elements per second over the K timed steps.  The roofline object reports the
algorithmic HBM bytes of one forward call divided by the call's average
duration, timed with HIP events on the stream the library launches on; the
HBM traffic and matrix-core utilisation come from the committed rocprofv3
counter summaries (profiles/) when they were taken on the current kernel
sources.  The cpu_baseline object times the CPU oracle (route F) on a bounded
sample of the same workload on this host's cores, and compares the GPU's
output with it on that sample (relL2, worst sequence, max-abs).

With --pass bwd one step is one fftconv_bwd call (fftconv_bwd_short for the
short-filter workload) producing du, dk, dw, dv instead;
with --pass taps one fftconv_fwd_taps call (the filter transformed from its L
time-domain taps inside the call).  Those lines name their own metric and carry
no CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_fft_convolution_amd as fc  # noqa: E402
from long_fft_convolution_amd import synth  # noqa: E402

METRIC = "FFT-conv fwd B·H·N elems/s + % HBM peak (rocprof), N=1K..4M, 1 GPU"
HBM_PEAK_GBS = 8000.0


# The GPU's clock ramps up over several milliseconds of sustained work: calls right after an
# idle period run 10-20 % slower.  Warm-up therefore runs the requested W steps and, beyond
# them, keeps stepping (untimed) until at least this much wall time has passed, so that the
# K timed steps see the steady clock.
MIN_WARMUP_S = 0.2


def warm_up(step, warmup: int, dev) -> int:
    """Run `warmup` steps, then more until MIN_WARMUP_S has passed; return the count run."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < MIN_WARMUP_S:
        step()
        n += 1
        if n >= warmup and n % 8 == 0:
            torch.cuda.synchronize(dev)
    torch.cuda.synchronize(dev)
    return n


ELEM = {"f32": 4, "f16": 2, "bf16": 2}
KERNEL_SOURCES = ["fused.hip", "multipass.hip", "pair_mfma.hip", "pair16k.hip", "eqlinear.hip", "cmfma.hpp",
                  "fft_device.hpp", "fft_stages.hpp",
                  "fftconv_internal.hpp", "api.cpp"]


def path_of(w: synth.Workload):
    """(kernel name, compute dtype, arithmetic) of the path fftconv_fwd takes for w."""
    mm = "fp16 MFMA operands, fp32 accumulation"
    if w.short:
        return "pair1k_kernel (windows of 2048, hop 1024)", "f16", mm
    if w.dtype in ("f16", "bf16") and w.N == 1024:
        return "pair1k_kernel", "f16", mm
    if w.dtype in ("f16", "bf16") and 2048 <= w.N <= 16384:
        return "pair16k_kernel", "f16", mm
    if w.N <= 16384:
        return "fused_conv_kernel", "f32", "fp32 (VALU)"
    if w.dtype == "f32":
        return "mp_pass1+mp_pass2+mp_pass3 (one call)", "f32", "fp32 (VALU)"
    if w.N >= 1 << 21:   # N1 = N / 8192 >= 256: column passes on the matrix cores too
        return ("mp_pass1c+mp_pass2m+mp_pass3c (one call)", "f16",
                f"fp16 MFMA operands, fp32 accumulation; {w.dtype} intermediate")
    return ("mp_pass1+mp_pass2m+mp_pass3 (one call)", "f16",
            "column passes fp32 (VALU); row pass fp16 MFMA operands, fp32 accumulation; "
            f"{w.dtype} intermediate")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w: synth.Workload) -> int:
    """What one forward call must move: u (+ w, v) read, out written, K_f read once
    per channel (only the kept blocks when the mask zeroes some)."""
    e = ELEM[w.dtype]
    act = w.B * w.H * w.N * e * (4 if w.gated else 2)
    if w.short:   # the spectrum of a 1024-sample window: 2048 bins per channel
        return int(act + w.H * 2048 * 4)
    bin_bytes = 8 if w.dtype == "f32" else 4
    keep = 1.0 if w.mask_keep_blocks is None else w.mask_keep_blocks / 128.0
    return int(act + w.H * w.N * bin_bytes * keep)


def bwd_algorithmic_bytes(w: synth.Workload, has_w: bool, has_v: bool) -> int:
    """What one backward call must move: dy, u (+ w, v) read, du (+ dw, dv) written,
    dk written, the spectrum read once per channel."""
    e = ELEM[w.dtype]
    nact = 3 + (2 if has_w else 0) + (2 if has_v else 0)
    spec = w.H * 2048 * 4 if w.short else w.H * (w.N + 1) * (8 if w.dtype == "f32" else 4)
    return int(w.B * w.H * w.N * e * nact + w.H * w.L * e + spec)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        p = os.path.join(ROOT, "long_fft_convolution_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _profile_json(name: str):
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    return d if d.get("kernel_source_hash") == kernel_source_hash() else None


def measured_traffic(workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources (else None)."""
    d = _profile_json(f"traffic_{workload}.json")
    return None if d is None else d.get("hbm_bytes_per_launch")


def measured_mfma(workload: str, ms_per_call: float):
    """Matrix-core figures per call from the committed rocprofv3 SQ counters of the
    current kernel sources (else None): fp16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_F16,
    512 flops per unit) over the timed call duration against the 2.5 PFLOP/s dense
    fp16 peak, and the counters' busy fraction SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x 256 CUs)."""
    d = _profile_json(f"counters_{workload}.json")
    if d is None:
        return None
    flops = d.get("mfma_f16_flops_per_call")
    out = {"peak_tflops": 2500.0, "flops_per_call": flops, "busy_frac": d.get("mfma_busy_frac")}
    if flops is not None:
        out["achieved_tflops"] = flops / (ms_per_call / 1e3) / 1e12
        out["frac"] = out["achieved_tflops"] / 2500.0
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl: synth.Workload, inp: synth.Inputs, out: torch.Tensor, budget_s: float = 8.0):
    """Time oracle.fft_conv (route F, float64) on leading batch rows (or channels when
    B = 1), sized to about budget_s of work on this host's threads, and compare the
    GPU's output `out` with the oracle's on that sample."""
    import oracle

    def sample(n):
        if wl.B > 1:
            sl = (slice(0, n), slice(None))
            kk, mm = inp.k, inp.mask
        else:
            sl = (slice(None), slice(0, n))
            kk, mm = inp.k[:n], None if inp.mask is None else inp.mask[:n]
        f64 = lambda t: None if t is None else t[sl].to(torch.float64).numpy()
        return sl, (f64(inp.u), kk.to(torch.float64).numpy(), f64(inp.w), f64(inp.v), mm)

    def run(n):
        sl, (uu, kk, ww, vv, mm) = sample(n)
        t0 = time.perf_counter()
        y = oracle.fft_conv(uu, kk, ww, vv, mask=mm)
        return time.perf_counter() - t0, uu.shape[0] * uu.shape[1], sl, y

    units = wl.B if wl.B > 1 else wl.H
    cores = oracle.max_threads()
    per_unit = wl.H if wl.B > 1 else 1            # sequences per sampled unit
    n = min(units, max(1, -(-cores // per_unit)))   # fill the threads once
    dt, nseq, sl, y = run(n)
    if dt < 0.5 * budget_s and n < units:
        n = int(min(units, max(n + 1, n * budget_s / max(dt, 1e-9))))
        dt, nseq, sl, y = run(n)
    got = out[sl].double().cpu().numpy()
    seq = oracle.seq_rel_l2(got, y)
    mabs = oracle.max_abs(got, y)
    what = "batch rows" if wl.B > 1 else "channels"
    return {"value": nseq * wl.N / dt, "unit": "elems/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n} of {units} {what} ({nseq} sequences) of {wl.name}, route F float64, {dt:.1f} s",
            "parity_on_sample": {"rel_l2": oracle.rel_l2(got, y), "worst_seq_rel_l2": float(seq.max()),
                                 "max_abs": mabs, "max_abs_rel": mabs / float(np.abs(y).max()),
                                 "sequences": int(seq.size)}}


FIVE = ["ungated_fp32_n1k", "gated_fp16_n1k", "gated_bf16_n16k", "ungated_fp16_n1m", "partial_sparse_n4m"]
HEADLINE = "partial_sparse_n4m"
TARGET_N16K = "gated_bf16_n16k"


def time_steps(step, steps: int, dev) -> float:
    """ms per step over `steps` back-to-back calls between two HIP events on the
    stream the library launches on (torch's current stream); no event between calls,
    which would add its own gap to every call."""
    stream = torch.cuda.current_stream(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize(dev)
    return t0.elapsed_time(t1) / steps


def measure_fwd(wl: synth.Workload, args, dev, with_cpu: bool):
    """One workload's forward figures (a dict of the bench line's fields)."""
    log(f"bench: generating {wl.name} (B={wl.B} H={wl.H} N={wl.N} L={wl.L} {wl.dtype})")
    inp = synth.generate_workload(wl.name)
    u = inp.u.to(dev)
    k = inp.k.to(dev)
    w = None if inp.w is None else inp.w.to(dev)
    v = None if inp.v is None else inp.v.to(dev)
    mask = None if inp.mask is None else torch.from_numpy(inp.mask).to(dev)
    out = torch.empty_like(u)
    if wl.short:
        K_f = torch.empty(fc.fftconv_short_filter_bytes(wl.H, u.dtype), dtype=torch.uint8, device=dev)
        fc.fftconv_prepare_short_filter(k, K_f)
        ws = None
    else:
        K_f = fc.alloc_filter(wl.H, wl.N, u.dtype, dev)
        fc.fftconv_prepare_filter(k, wl.N, K_f, fc.alloc_workspace(1, wl.H, wl.N, u.dtype, dev))
        ws = fc.alloc_workspace(wl.B, wl.H, wl.N, u.dtype, dev)
    torch.cuda.synchronize(dev)

    def step():
        if wl.short:
            fc.fftconv_fwd_short(u, K_f, w, v, out, wl.L)
        else:
            fc.fftconv_fwd(u, K_f, w, v, out, wl.L, mask, ws)

    n_warm = warm_up(step, args.warmup, dev)
    ms = time_steps(step, args.steps, dev)
    elems = wl.B * wl.H * wl.N
    alg = algorithmic_bytes(wl)
    achieved = alg / (ms / 1e3) / 1e9
    kernel, cdtype, arith = path_of(wl)
    log(f"bench: {wl.name}: {n_warm} warm-up steps, {ms * 1e3:.1f} us/step, {elems / (ms / 1e3):.3e} elems/s, "
        f"{achieved:.0f} GB/s algorithmic ({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")
    if args.calibrate_copy:
        # a plain elementwise copy kernel of known size: reads and writes n*4 bytes
        n = (alg // 2) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize(dev)
        log(f"bench: calibration copy kernel moved {n * 4} bytes each way")
        del src, dst
    traffic = measured_traffic(wl.name)
    rec = {
        "workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "L_filter": wl.L, "gated": wl.gated,
        "storage": wl.dtype, "dtype": cdtype, "arithmetic": arith, "mask_keep_blocks": wl.mask_keep_blocks,
        "ms_per_step": ms, "value": elems / (ms / 1e3), "unit": "elems/s", "warmup_steps_run": n_warm,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_over_algorithmic": None if traffic is None else traffic / alg,
                     "algorithmic_bytes": alg, "kernel_ms": ms, "mfma": measured_mfma(wl.name, ms)},
        "cpu_baseline": None,
    }
    if with_cpu:
        log(f"bench: {wl.name}: timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(wl, inp, out)
        c = rec["cpu_baseline"]
        log(f"bench: {wl.name}: oracle {c['value']:.3e} elems/s on {c['cores']} threads ({c['sample']}); "
            f"sample relL2 {c['parity_on_sample']['rel_l2']:.2e}, worst sequence "
            f"{c['parity_on_sample']['worst_seq_rel_l2']:.2e}")
    del u, k, w, v, mask, out, K_f, ws, inp
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="minimum untimed steps; more run until 0.2 s has passed (the count run is reported)")
    ap.add_argument("--workload", default="all",
                    choices=["all"] + sorted(synth.WORKLOADS) + sorted(synth.EQ_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "taps"], default="fwd",
                    help="time the forward call (default), the backward call, or the forward "
                         "call from time-domain taps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain device copy of the activation bytes (counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(sequences are independent: (b, h) would be sharded across devices)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")

    if args.workload in synth.EQ_WORKLOADS:
        return bench_eqlinear(args)
    if args.which != "fwd":
        wl = synth.WORKLOADS[HEADLINE if args.workload == "all" else args.workload]
        if wl.short and args.which == "taps":
            log("bench: the short-filter path takes a prepared filter only (no taps call)")
            return 2
        return bench_other(args, wl, dev)

    names = FIVE if args.workload == "all" else [args.workload]
    recs = [measure_fwd(synth.WORKLOADS[n], args, dev, not args.no_cpu_baseline) for n in names]
    head = next((r for r in recs if r["workload"] == HEADLINE), recs[-1])
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": head["warmup_steps_run"],
        "warmup_min": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) activations, decaying random filter)",
        "config": {"workload": head["workload"], "B": head["B"], "H": head["H"], "N": head["N"],
                   "L_filter": head["L_filter"], "gated": head["gated"], "storage": head["storage"],
                   "arithmetic": head["arithmetic"], "mask_keep_blocks": head["mask_keep_blocks"],
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "workloads": recs,
    }
    t = next((r for r in recs if r["workload"] == TARGET_N16K), None)
    if t is not None:
        line["target_n16k"] = {"workload": TARGET_N16K, "frac": t["roofline"]["frac"], "target_frac": 0.5,
                               "met": t["roofline"]["frac"] >= 0.5,
                               "elems_per_s": t["value"], "target_elems_per_s": 4.44e11}
    print(json.dumps(line), flush=True)


def bench_other(args, wl, dev):
    """--pass bwd / taps on one workload."""
    inp = synth.generate_workload(wl.name)
    u = inp.u.to(dev)
    k = inp.k.to(dev)
    w = None if inp.w is None else inp.w.to(dev)
    v = None if inp.v is None else inp.v.to(dev)
    mask = None if inp.mask is None else torch.from_numpy(inp.mask).to(dev)
    if wl.short:
        K_f = torch.empty(fc.fftconv_short_filter_bytes(wl.H, u.dtype), dtype=torch.uint8, device=dev)
        fc.fftconv_prepare_short_filter(k, K_f)
    else:
        K_f = fc.alloc_filter(wl.H, wl.N, u.dtype, dev)
        fc.fftconv_prepare_filter(k, wl.N, K_f, fc.alloc_workspace(1, wl.H, wl.N, u.dtype, dev))
    torch.cuda.synchronize(dev)
    if args.which == "bwd":
        return bench_bwd(args, wl, dev, u, K_f, w, v, mask)
    return bench_taps(args, wl, dev, u, k, w, v, mask)


def bench_eqlinear(args):
    """One step = one fftconv_eqlinear_fwd call (the group-axis circular convolution)."""
    wl = synth.EQ_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"bench: generating {wl.name} (N={wl.N} T={wl.T} C_in={wl.C_in} C_out={wl.C_out} {wl.dtype})")
    x_h, W_h = synth.generate_eq(wl.name)
    x, W = x_h.to(dev), W_h.to(dev)
    W_f = torch.empty(fc.fftconv_eqlinear_weight_bytes(wl.T, wl.C_out, wl.C_in, x.dtype), dtype=torch.uint8,
                      device=dev)
    fc.fftconv_eqlinear_prepare(W, W_f)
    y = torch.empty((wl.N, wl.T, wl.C_out), dtype=x.dtype, device=dev)
    n_warm = warm_up(lambda: fc.fftconv_eqlinear_fwd(x, W_f, y), args.warmup, dev)
    ms = time_steps(lambda: fc.fftconv_eqlinear_fwd(x, W_f, y), args.steps, dev)
    e = ELEM[wl.dtype]
    alg = wl.N * wl.T * (wl.C_in + wl.C_out) * e + W_f.numel()
    # matrix-core work: per token, f = 0 and T/2 are real products, the T/2 - 1 others complex (4 real)
    flops = 2.0 * wl.N * wl.C_in * wl.C_out * (2 + 4 * (wl.T // 2 - 1))
    value = wl.N * wl.T * wl.C_in / (ms / 1e3)
    achieved = alg / (ms / 1e3) / 1e9
    tflops = flops / (ms / 1e3) / 1e12
    # the bound: HBM for fp16 operands (dense fp16 peak 2.5 PFLOP/s), the fp32 matrix cores
    # (157.3 TFLOP/s dense) for fp32, whichever takes longer at its peak
    mfma_peak = 157.3 if wl.dtype == "f32" else 2500.0
    bound = "mfma" if flops / (mfma_peak * 1e12) > alg / (HBM_PEAK_GBS * 1e9) else "hbm"
    log(f"bench: {ms * 1e3:.1f} us/step, {value:.3e} elems/s, {achieved:.0f} GB/s algorithmic "
        f"({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s), MFMA {tflops:.1f} TFLOP/s ({tflops / mfma_peak:.1%} of {mfma_peak})")
    if args.calibrate_copy:
        n = (alg // 2) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize(dev)
        log(f"bench: calibration copy kernel moved {n * 4} bytes each way")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle.eqlinear import eqlinear_tokens
        n = 256
        xx, WW = x_h[:n].double().numpy(), W_h.double().numpy()
        t = time.perf_counter()
        eqlinear_tokens(xx, WW, np.arange(n))
        dt = time.perf_counter() - t
        cpu = {"value": n * wl.T * wl.C_in / dt, "unit": "elems/s", "cores": torch.get_num_threads(),
               "kind": "oracle", "sample": f"{n} of {wl.N} tokens of {wl.name}, float64 numpy, {dt:.2f} s"}
    rec = {
        "metric": "group-axis circular conv fwd N*T*C_in elems/s + % HBM peak, 1 GPU",
        "value": value, "unit": "elems/s", "n_gpus": 1, "steps": args.steps, "warmup": n_warm,
        "warmup_min": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "f16",
        "data": "synthetic (seeded N(0,1) activations, N(0, 1/(T C_in)) weights)",
        "config": {"workload": wl.name, "N": wl.N, "T": wl.T, "C_in": wl.C_in, "C_out": wl.C_out,
                   "storage": wl.dtype,
                   "arithmetic": ("fp32 MFMA operands, fp32 accumulation" if wl.dtype == "f32"
                                  else "fp16 MFMA operands, fp32 accumulation"),
                   "parallelism": "single GPU"},
        "roofline": ({"bound": "hbm", "kernel": "eqlinear_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name),
                      "algorithmic_bytes": int(alg), "kernel_ms": ms, "mfma_tflops": tflops}
                     if bound == "hbm" else
                     {"bound": "mfma", "kernel": "eqlinear32_kernel", "achieved": tflops, "peak": mfma_peak,
                      "unit": "TFLOP/s", "frac": tflops / mfma_peak, "traffic": measured_traffic(wl.name),
                      "algorithmic_flops": flops, "algorithmic_bytes": int(alg), "kernel_ms": ms,
                      "hbm_gbs": achieved}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_bwd(args, wl, dev, u, K_f, w, v, mask):
    """One step = one fftconv_bwd call (fftconv_bwd_short for the short-filter path)
    producing du, dk, dw, dv."""
    g = torch.Generator().manual_seed(4242)
    dy = torch.randn(u.shape, generator=g, dtype=torch.float32).to(u.dtype).to(dev)
    du = torch.empty_like(u)
    dk = torch.empty((wl.H, wl.L), dtype=u.dtype, device=dev)
    dw = torch.empty_like(u) if w is not None else None
    dv = torch.empty_like(u) if v is not None else None
    ws = None if wl.short else torch.empty(fc.fftconv_bwd_workspace_bytes(wl.B, wl.H, wl.N, u.dtype),
                                           dtype=torch.uint8, device=dev)

    def step():
        if wl.short:
            fc.fftconv_bwd_short(dy, u, K_f, w, v, du, dk, dw, dv, wl.L)
        else:
            fc.fftconv_bwd(dy, u, K_f, w, v, du, dk, dw, dv, wl.L, mask, ws)

    n_warm = warm_up(step, args.warmup, dev)
    log(f"bench: {n_warm} warm-up steps")
    ms_per_step = time_steps(step, args.steps, dev)
    elems = wl.B * wl.H * wl.N
    alg = bwd_algorithmic_bytes(wl, w is not None, v is not None)
    achieved = alg / (ms_per_step / 1e3) / 1e9
    log(f"bench: bwd {ms_per_step * 1e3:.1f} us/step, {elems / (ms_per_step / 1e3):.3e} elems/s")
    rec = {
        "metric": "FFT-conv bwd (du, dk, dw, dv) B·H·N elems/s, 1 GPU",
        "value": elems / (ms_per_step / 1e3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "warmup_min": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_of(wl)[1],
        "data": "synthetic (seeded N(0,1) activations and output gradient, decaying random filter)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "L_filter": wl.L,
                   "gated": wl.gated, "storage": wl.dtype, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": ("fftconv_bwd_short" if wl.short else "fftconv_bwd")
                     + " (several launches)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes": alg, "kernel_ms": ms_per_step},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def bench_taps(args, wl, dev, u, k, w, v, mask):
    """One step = one fftconv_fwd_taps call: the spectrum of the L taps is formed inside
    the call (into its workspace), then the forward kernels run on it."""
    out = torch.empty_like(u)
    ws = torch.empty(fc.fftconv_fwd_taps_workspace_bytes(wl.B, wl.H, wl.N, u.dtype), dtype=torch.uint8,
                     device=dev)

    def step():
        fc.fftconv_fwd_taps(u, k, w, v, out, ws, mask)

    n_warm = warm_up(step, args.warmup, dev)
    log(f"bench: {n_warm} warm-up steps")
    ms_per_step = time_steps(step, args.steps, dev)
    elems = wl.B * wl.H * wl.N
    e = ELEM[wl.dtype]
    # the forward call's bytes with the L taps read in place of the spectrum
    alg = wl.B * wl.H * wl.N * e * (4 if wl.gated else 2) + wl.H * wl.L * e
    achieved = alg / (ms_per_step / 1e3) / 1e9
    log(f"bench: taps {ms_per_step * 1e3:.1f} us/step, {elems / (ms_per_step / 1e3):.3e} elems/s")
    rec = {
        "metric": "FFT-conv fwd from time-domain taps B·H·N elems/s, 1 GPU",
        "value": elems / (ms_per_step / 1e3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "warmup_min": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_of(wl)[1],
        "data": "synthetic (seeded N(0,1) activations, decaying random filter)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "L_filter": wl.L,
                   "gated": wl.gated, "storage": wl.dtype,
                   "mask_keep_blocks": wl.mask_keep_blocks, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "fftconv_fwd_taps (prepare and forward launches)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": alg,
                     "kernel_ms": ms_per_step},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

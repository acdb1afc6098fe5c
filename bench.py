"""Benchmark of the Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload d24_bf16]
                    [--no-cpu-baseline] [--power SECONDS] [--copy-calibration]

A step is one muon_step_batched call over every matrix of the workload
(momentum, norm, Newton-Schulz, write-back), with weights, gradients and
momenta resident in HBM before the timed region.  Prints one JSON line.

The roofline object is for the kernel class with the largest share of the
timed region; per-launch durations come from HIP events the library
records around each launch on the launch stream (muon_timing_*).  Its
traffic is the HBM bytes per launch from the rocprofv3 FETCH_SIZE /
WRITE_SIZE summary under profiles/, reported only while the kernel sources
hash to the values recorded there (null otherwise).
`roofline.measured_peak` is the achievable rate on the same box: the
library's register-only MFMA loop on random operands (`muon_mfma_probe`)
for the products, a torch device copy for HBM-bound kernels.
The cpu_baseline is the CPU oracle timed on a bounded sample of the same
workload on this host.  The `adamw` object times the other half of the
hybrid optimizer, AdamW on the d24 parameters that are not transformer
matrices; it is reported beside the Muon step and not counted in `value`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "Muon steps/sec on d24-like stack; NS TFLOP/s and % bf16 MFMA peak"

WORKLOAD_TEXT = {
    "d24_bf16": "d24-like stack: 24 layers x {Q,K,V,O 1536x1536, up 1536x6144, down 6144x1536} = 144 bf16 "
                "matrices, rank-16 + N(0,1) gradients, 5 quintic NS steps, bf16 MFMA",
    "lm3p8b_bf16": "3.8B-like stack: 32 layers x {Q,O 3072x3072, K,V 3072x1024, up 3072x12288, "
                   "down 12288x3072} = 192 bf16 matrices, N(0,1) gradients, 5 quintic NS steps",
    "gpt2s_attn768_bf16": "12 x 768x768 bf16, 5 quintic NS steps",
    "single256_f32": "1 x 256x256 f32, 5 cubic NS steps, f32 MFMA",
    "stress_mixed_bf16": "64 mixed-aspect bf16 matrices from {512..8192}^2, 10 quintic NS steps, split-bf16",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d24_bf16")
    ap.add_argument("--layers", type=int, default=None,
                    help="truncate the layer stack (d24_bf16 with 3 layers is one GPU's share of 8: "
                         "12 x 1536^2 + 3 up + 3 down)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=6,
                    help="layers in the oracle's sample (about 10-15 s of host work for d24)")
    ap.add_argument("--launch-mode", choices=("auto", "grids", "chain"), default="auto",
                    help="Newton-Schulz launches: the library's choice, one grid per phase, or one persistent chain")
    ap.add_argument("--tile-mode", choices=("auto", "large", "small"), default="auto",
                    help="tile size of the Newton-Schulz products: the library's choice, "
                         "large (bf16 256, fp32 128) or small (bf16 128, fp32 64)")
    ap.add_argument("--no-adamw", action="store_true",
                    help="skip timing the AdamW half of the hybrid optimizer (d24 non-matrix parameters)")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, run steps for SECONDS more while amd-smi samples the "
                         "socket power and the shader clocks (reported as `power`; off by default)")
    ap.add_argument("--power-zero-data", type=float, default=0.0, metavar="SECONDS",
                    help="at the end, zero the gradients and momenta (every product then multiplies "
                         "zeros, with the same memory traffic) and time and sample the step for SECONDS "
                         "(reported as `power_zero_data`; a diagnostic of how the data sets the clock)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB device-to-device once (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU layout is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from muon_newton_schulz_02_amd import binding as mb
    from muon_newton_schulz_02_amd import workloads as wlm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = wlm.workload(args.workload, layers=args.layers)
    n = len(wl.specs)
    print(f"[bench] generating {args.workload}: {n} matrices, {wl.elements} elements", file=sys.stderr,
          flush=True)
    ws, ms, gs = [], [], []
    for i in range(n):
        w, m = wlm.initial_state(wl, i, device=dev)
        ws.append(w)
        ms.append(m)
        gs.append(wlm.gradient(wl, i, 0, device=dev))
    torch.cuda.synchronize()
    # keep host copies of the oracle's sample before the weights move
    sample_idx = []
    if not args.no_cpu_baseline:
        per_layer = 6 if args.workload in ("d24_bf16", "lm3p8b_bf16") else 1
        sample_idx = list(range(min(n, per_layer * args.cpu_layers)))
    sample = [(ws[i].float().cpu().numpy(), gs[i].float().cpu().numpy(), ms[i].cpu().numpy())
              for i in sample_idx]

    sargs = mb.StepArgs(ws, gs, ms, precision=wl.precision)
    kw = dict(lr=float(np.float32(wl.lr)), beta=wl.beta, nesterov=int(wl.nesterov), ns_coeffs=wl.coeffs,
              ns_steps=wl.ns_steps, scale_rule=wl.scale_rule)
    stream = torch.cuda.current_stream()
    mode = {"auto": mb.LAUNCH_AUTO, "grids": mb.LAUNCH_PHASE_GRIDS, "chain": mb.LAUNCH_CHAIN}[args.launch_mode]
    tiles = {"auto": mb.TILES_AUTO, "large": mb.TILES_LARGE, "small": mb.TILES_SMALL}[args.tile_mode]

    def step():
        if mode == mb.LAUNCH_AUTO and tiles == mb.TILES_AUTO:
            mb.muon_step_batched(sargs, **kw, stream=stream)
        else:
            mb.muon_step_batched_v2(sargs, **kw, stream=stream, launch_mode=mode, tile_mode=tiles)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    mb.muon_timing_enable(True)
    mb.muon_timing_read()  # clear
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = mb.muon_timing_read()
    mb.muon_timing_enable(False)
    ms_total = marks[0].elapsed_time(marks[-1])
    ms_step = ms_total / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    pct = {f"p{q}": round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)}
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (event), wall {wall / args.steps * 1e3:.3f} ms",
          file=sys.stderr, flush=True)
    # the same steps again without the per-launch events of the timing hook
    # (they add a few microseconds per launch, visible on the small workloads)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step_plain = e0.elapsed_time(e1) / args.steps

    power = sample_power(args.power, step, torch) if args.power > 0 else None

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------ accounting
    k = wl.ns_steps
    nominal, alg = ns_flops([(s.rows, s.cols) for s in wl.specs], k, wl.coeffs[2] != 0.0)
    elems = wl.elements
    gbytes = 2 if wl.grad_dtype == torch.bfloat16 else 4
    pbytes = 2 if wl.param_dtype == torch.bfloat16 else 4
    # momentum kernel: read g and M, write M, write U once (algorithmic)
    alg_bytes_mom = elems * (gbytes + 4 + 4 + 2)
    peak_mfma = PEAK_F32_TFLOPS if wl.precision == mb.NS_F32 else PEAK_BF16_TFLOPS

    kernels = {}
    steps = args.steps
    for name, (tot_ms, launches) in kern.items():
        if launches == 0:
            continue
        avg_ms = tot_ms / launches
        entry = {"launches_per_step": launches / steps, "avg_ms": round(avg_ms, 5),
                 "share": round(tot_ms / ms_total, 4)}
        if name in alg or name == "chain":
            # one chain launch runs every step of the Newton-Schulz iteration
            flops_launch = sum(alg.values()) if name == "chain" else alg[name] / k
            tf = flops_launch / (avg_ms * 1e-3) / 1e12
            entry.update({"bound": "mfma", "tflops": round(tf, 2), "frac": round(tf / peak_mfma, 4)})
        elif name == "momentum":
            gbs = alg_bytes_mom / (avg_ms * 1e-3) / 1e9
            entry.update({"bound": "hbm", "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)})
        kernels[name] = entry
    dom = max(kernels, key=lambda x: kernels[x]["share"])
    d = kernels[dom]
    traffic = measured_traffic(args.workload if args.layers is None else None, dom)
    if d.get("bound") == "mfma":
        roofline = {"bound": "mfma", "kernel": dom, "achieved": d["tflops"], "peak": peak_mfma,
                    "unit": "TFLOP/s", "frac": d["frac"], "traffic": traffic}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": d.get("gbs"), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": d.get("frac"), "traffic": traffic}
    ns_ms = sum(kern[x][0] for x in ("gram", "poly", "combine", "chain")) / steps
    ns_exec = sum(alg.values())
    ns_chain = {"nominal_tflop_per_step": round(nominal / 1e12, 4),
                "ms_per_step": round(ns_ms, 4),
                "nominal_tflops": round(nominal / (ns_ms * 1e-3) / 1e12, 2),
                "nominal_frac": round(nominal / (ns_ms * 1e-3) / 1e12 / peak_mfma, 4),
                "algorithmic_tflops": round(ns_exec / (ns_ms * 1e-3) / 1e12, 2),
                "algorithmic_frac": round(ns_exec / (ns_ms * 1e-3) / 1e12 / peak_mfma, 4)}

    adamw = None
    if not args.no_adamw and args.workload == "d24_bf16" and args.layers is None:
        adamw = time_adamw(args, mb, wlm, torch, dev, stream)
    copy_gbs = hbm_copy_gbs(torch, dev, stream)
    mfma_tflops = mfma_probe_tflops(mb, torch, dev, stream)
    if roofline["bound"] == "hbm":
        roofline["measured_peak"] = round(copy_gbs, 1)
    elif wl.precision != mb.NS_F32:   # the probe measures the bf16 rate
        roofline["measured_peak"] = round(mfma_tflops, 1)
    if roofline.get("measured_peak") and roofline.get("achieved"):
        roofline["frac_of_measured"] = round(roofline["achieved"] / roofline["measured_peak"], 4)
    if wl.precision != mb.NS_F32:
        ns_chain["algorithmic_frac_of_measured"] = round(ns_exec / (ns_ms * 1e-3) / 1e12 / mfma_tflops, 4)
    for entry in [kernels.get("momentum"), adamw]:
        if entry and entry.get("gbs"):
            entry["frac_of_copy"] = round(entry["gbs"] / copy_gbs, 4)

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if sample:
        cpu = cpu_baseline(wl, sample, sample_idx, kw, n)

    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 4),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms_percentiles": pct,
        "ms_per_step_without_kernel_events": round(ms_step_plain, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.precision == mb.NS_BF16 else ("f32" if wl.precision == mb.NS_F32 else "bf16x3"),
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT.get(args.workload, args.workload) if args.layers is None else
                   f"{args.workload} truncated to {args.layers} layers", "name": args.workload,
                   "matrices": n, "elements": elems, "ns_steps": k, "coeffs": list(wl.coeffs),
                   "matrices_per_s": round(n * 1e3 / ms_step, 1), "parallelism": "1 GPU",
                   "launch_mode": args.launch_mode, "tile_mode": args.tile_mode},
        "roofline": roofline,
        "ns_chain": ns_chain,
        "kernels": kernels,
        "adamw": adamw,
        "hbm_copy_gbs": round(copy_gbs, 1),
        "mfma_probe_tflops": round(mfma_tflops, 1),
        "cpu_baseline": cpu,
    }
    if power is not None:
        out["power"] = power
    if args.power_zero_data > 0:
        for t in gs + ms:
            t.zero_()
        torch.cuda.synchronize()
        for _ in range(3):
            step()
        z0, z1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        z0.record(stream)
        for _ in range(args.steps):
            step()
        z1.record(stream)
        torch.cuda.synchronize()
        zero = sample_power(args.power_zero_data, step, torch)
        zero["ms_per_step"] = round(z0.elapsed_time(z1) / args.steps, 4)
        out["power_zero_data"] = zero
    print(json.dumps(out))


def ns_flops(shapes, ns_steps, c_nonzero):
    """Flops of `ns_steps` Newton-Schulz steps over matrices of the given
    (rows, cols): nominal, 4 m^2 n + 2 m^3 per step and matrix (m <= n; the
    A^2 term dropped when c = 0), and algorithmic per product, the symmetric
    products counting their unique entries once: GRAM m (m + 1) n, POLY
    m^2 (m + 1), COMBINE 2 m^2 n."""
    nominal = 0.0
    alg = {"gram": 0.0, "poly": 0.0, "combine": 0.0}
    for rows, cols in shapes:
        m_, n_ = min(rows, cols), max(rows, cols)
        nominal += (4.0 * m_ * m_ * n_ + (2.0 * m_ ** 3 if c_nonzero else 0.0)) * ns_steps
        alg["gram"] += float(m_) * (m_ + 1) * n_ * ns_steps
        alg["poly"] += (float(m_) * (m_ + 1) * m_ * ns_steps) if c_nonzero else 0.0
        alg["combine"] += 2.0 * m_ * m_ * n_ * ns_steps
    return nominal, alg


def parse_amd_smi_metric(txt):
    """Socket power (W) and the mean of the shader clocks gfx_0 .. (MHz) from
    `amd-smi metric -g 0 -p -c --json` output."""
    d = json.loads(txt)
    d = d[0] if isinstance(d, list) else d
    d = d.get("gpu_data", [d])[0] if isinstance(d, dict) and "gpu_data" in d else d
    pw = d["power"]["socket_power"]
    pw = pw["value"] if isinstance(pw, dict) else pw
    clk = [v["clk"]["value"] for k, v in d["clock"].items()
           if k.startswith("gfx_") and isinstance(v.get("clk"), dict) and isinstance(v["clk"]["value"], (int, float))]
    return float(pw), sum(clk) / len(clk)


def sample_power(seconds, step, torch, period=0.4):
    """Socket power and shader clock while the step runs back to back: amd-smi
    (`metric -p -c --json`) is sampled from a thread; the first second is
    skipped.  Returns means over the samples, or an error string."""
    import subprocess
    import threading

    samples, stop = [], threading.Event()

    def sampler():
        stop.wait(1.0)
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"],
                                   capture_output=True, text=True, timeout=10)
                if r.returncode == 0:
                    samples.append(parse_amd_smi_metric(r.stdout))
            except Exception:  # noqa: BLE001 - a failed sample is skipped
                pass
            stop.wait(period)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return {"error": "no amd-smi sample"}
    return {"socket_power_w": round(sum(p for p, _ in samples) / len(samples), 1),
            "socket_power_w_min": min(p for p, _ in samples), "socket_power_w_max": max(p for p, _ in samples),
            "gfx_clock_mhz": round(sum(c for _, c in samples) / len(samples), 1), "samples": len(samples),
            "seconds": seconds, "tool": "amd-smi metric -g 0 -p -c --json"}


def mfma_probe_tflops(mb, torch, dev, stream, iterations=200000, launches=4):
    """Achievable dense bf16 MFMA rate on random data: the library's
    register-only MFMA loop on every SIMD, one untimed launch (the clock
    settles under the load) and `launches` timed with events (about 35 ms
    each)."""
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    mb.muon_mfma_probe(iterations, sink, stream=stream)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    flops = 0.0
    for _ in range(launches):
        flops += mb.muon_mfma_probe(iterations, sink, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    tf = flops / (start.elapsed_time(stop) * 1e-3) / 1e12
    print(f"[bench] mfma probe: {tf:.0f} TFLOP/s dense bf16", file=sys.stderr, flush=True)
    return tf


def hbm_copy_gbs(torch, dev, stream, nbytes=1 << 30, reps=5):
    """Achievable HBM bandwidth for a read + write stream: torch's device copy
    of `nbytes`, bytes read plus bytes written per second."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    stop.record(stream)
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (start.elapsed_time(stop) * 1e-3) / 1e9
    print(f"[bench] device copy: {gbs:.0f} GB/s (read + write)", file=sys.stderr, flush=True)
    del src, dst
    return gbs


def time_adamw(args, mb, wlm, torch, dev, stream):
    """Time muon_adamw_batched on the d24 AdamW set (the parameters Muon does
    not take), `args.steps` calls after `args.warmup`, with the step number
    advancing; reported beside the Muon step, not part of its value."""
    wl = wlm.adamw_workload()
    print(f"[bench] generating {wl.name}: {len(wl.specs)} tensors, {wl.elements} elements", file=sys.stderr,
          flush=True)
    ps, gs, ms, vs = [], [], [], []
    for i in range(len(wl.specs)):
        p, m, v = wlm.adamw_state(wl, i, dev)
        ps.append(p)
        ms.append(m)
        vs.append(v)
        gs.append(wlm.adamw_gradient(wl, i, 0, dev))
    aargs = mb.AdamwArgs(ps, gs, ms, vs)
    kw = dict(lr=wl.lr[0], beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps, lr_per_tensor=wl.lr_per_tensor(),
              wd_per_tensor=wl.wd_per_tensor(), stream=stream)
    t = wl.step
    for _ in range(args.warmup):
        mb.muon_adamw_batched(aargs, step=t, **kw)
        t += 1
    torch.cuda.synchronize()
    mb.muon_timing_enable(True)
    mb.muon_timing_read()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        mb.muon_adamw_batched(aargs, step=t, **kw)
        t += 1
    stop.record(stream)
    torch.cuda.synchronize()
    kern = mb.muon_timing_read()
    mb.muon_timing_enable(False)
    ms_call = start.elapsed_time(stop) / args.steps
    k_ms, k_n = kern["adamw"]
    avg = k_ms / max(k_n, 1)
    bpe = 2 * (ps[0].element_size() + 4 + 4) + gs[0].element_size()   # p, m, v read and written; g read
    alg_bytes = wl.elements * bpe
    gbs = alg_bytes / (avg * 1e-3) / 1e9
    print(f"[bench] adamw: {ms_call:.3f} ms/call, kernel {avg:.3f} ms, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    del aargs, ps, gs, ms, vs
    return {"workload": "d24 non-matrix parameters: lm_head, token embedding and 12 value embeddings "
                        "(32768x1536 each) + 2 x 24 scalars, bf16 p and g, fp32 moments",
            "elements": wl.elements, "tensors": len(wl.specs), "ms_per_call": round(ms_call, 4),
            "kernel_avg_ms": round(avg, 5), "bytes_per_element": bpe, "algorithmic_gb": round(alg_bytes / 1e9, 3),
            "bound": "hbm", "gbs": round(gbs, 1), "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("d24_bf16", "adamw")}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ns_gemm_d24_bf16_hbm.md")
CSRC = os.path.join(ROOT, "muon_newton_schulz_02_amd", "csrc")


def _src_hash(*names):
    """sha256 prefix of the kernel sources' code: `//` comments, trailing blanks
    and empty lines removed, so that a comment edit keeps the hash."""
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(CSRC, nm), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE summary of
    the d24 workload, or None when that summary was taken on other kernel sources (or another
    workload)."""
    if workload != "d24_bf16" or not os.path.exists(TRAFFIC_FILE):
        return None
    line = None
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if ln.strip().startswith("traffic:"):
                line = ln.strip()[len("traffic:"):]
    if line is None:
        return None
    kv = dict(tok.split("=", 1) for tok in line.split())
    if kernel == "momentum":
        src, key = _src_hash("elementwise.hip", "numeric.h", "muon_internal.h"), "elementwise_src"
    elif kernel == "adamw":
        src, key = _src_hash("adamw.hip", "numeric.h", "muon_internal.h"), "adamw_src"
    else:
        src, key = _src_hash("ns_gemm.hip", "ns_tile.h", "numeric.h", "muon_internal.h"), "gemm_src"
    if src != kv.get(key) or kernel not in kv:
        return None
    return float(kv[kernel])


def _host_description():
    """CPU model, logical CPUs and the BLAS library (with its thread count)
    that NumPy calls, as this host reports them."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, os.cpu_count() or 1
    try:
        import numpy  # noqa: F401  (loads the BLAS the oracle calls)
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api')} {p.get('version')} ({p.get('architecture')})"
                threads = int(p.get("num_threads", threads))
                break
    except Exception:  # noqa: BLE001
        pass
    return model, os.cpu_count(), blas, threads


def _config1_one_thread(orc, wlm):
    """The oracle on the single 256 x 256 binary32 configuration (5 cubic
    steps), BLAS held to one thread: steps per second."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    wl = wlm.workload("single256_f32")
    w, m = (t.numpy() for t in wlm.initial_state(wl, 0))
    g = wlm.gradient(wl, 0).numpy()
    kw = dict(lr=float(np.float32(wl.lr)), beta=wl.beta, nesterov=wl.nesterov, coeffs=wl.coeffs,
              steps=wl.ns_steps)
    with threadpool_limits(limits=1):
        orc.muon_step(w, g, m, **kw)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            orc.muon_step(w, g, m, **kw)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    return {"workload": "single256_f32 (1 x 256x256 f32, 5 cubic NS steps)", "threads": 1,
            "value": round(1.0 / dt, 2), "unit": "steps/s", "ms_per_step": round(dt * 1e3, 3)}


def cpu_baseline(wl, sample, sample_idx, kw, n_total):
    """Time the float64 oracle on the sample; scale by nominal FLOPs to a full step."""
    import oracle as orc
    from muon_newton_schulz_02_amd import workloads as wlm

    model, ncpu, blas, threads = _host_description()
    t0 = time.perf_counter()
    for w, g, m in sample:
        orc.muon_step(w, g, m, lr=kw["lr"], beta=kw["beta"], nesterov=bool(kw["nesterov"]),
                      coeffs=kw["ns_coeffs"], steps=kw["ns_steps"], scale_rule=kw["scale_rule"],
                      param_bf16=str(wl.param_dtype) == "torch.bfloat16")
    dt = time.perf_counter() - t0

    def cost(s):
        m_, n_ = min(s.rows, s.cols), max(s.rows, s.cols)
        return 4.0 * m_ * m_ * n_ + 2.0 * m_ ** 3

    frac = sum(cost(wl.specs[i]) for i in sample_idx) / sum(cost(s) for s in wl.specs)
    step_s = dt / frac
    out = {"value": round(1.0 / step_s, 6), "unit": "steps/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(sample)} of {n_total} matrices (first layers), float64 NumPy oracle, "
                     f"{dt:.2f} s, scaled by nominal NS FLOPs ({frac:.4f} of the step) to the full step",
           "seconds_per_step": round(step_s, 3), "cpu_model": model, "logical_cpus": ncpu, "blas": blas}
    try:
        out["config1_one_thread"] = _config1_one_thread(orc, wlm)
    except Exception as e:  # noqa: BLE001
        out["config1_one_thread"] = {"error": str(e)}
    return out


if __name__ == "__main__":
    main()

#!/usr/bin/env python
"""Benchmark: the online 4-bit activation path and the W4A4 + low-rank linear at the
FLUX.1-like joint-block shape, on one MI355X.

One step = the whole hot path over one batch, for each of the block's three linears
(qkv 3072->9216, fc1 3072->12288, fc2 12288->3072, M = 4608 tokens):
    kq_transform_quantize_lowrank   centre each token, RPBH-32 rotation, MXFP4 quantize +
                                    pack, and T = X L1^T (rank 32, fp16)
    kq_w4a4_linear_t                Y = Xq Wq^T + T L2^T + mu wbar^T (scaled-FP4 MFMA, fp16 out)
Weights are folded once (offline, untimed).  Inputs are seeded synthetic activations
(Gaussian + per-token adaLN-like shift N(0, 4^2) + 12 outlier channels x50) already
resident in HBM; the activation buffers rotate over enough copies (>= 1 GiB) that no step
reads them from the 256 MB last-level cache.

Prints ONE JSON line.  The step time comes from two HIP events around the timed steps, on
the stream the kernels run on, with nothing between the launches; before the warm-up steps
each rotated input set goes through one step, so that none is first touched while timed.  Per-launch durations:
10 untimed launches, then 50 timed ones in 5 groups of 10 back to back between two events,
each group queued behind a short device-side sleep so that the GPU never waits for the
host (a launch through the binding costs about 11 us of host time, more than some of the
kernels); the figure is the median of the group means, which matches the profiler's kernel
durations.  Activations (and, for the GEMM, the packed activation codes, T and mu) rotate
over >= 1 GiB of copies in these passes too.  The other configurations (CogVideoX-like,
PixArt-like, SANA-like) are timed the same way, per launch.  The "traffic" fields come
from the HBM byte counters recorded in profiles/ for the same kernel source (null when the
source has changed since).  The shader clock is measured by the library's clock probe on a
second stream while the GEMMs run, and the matrix-core peak is also given at that clock.
The vendor library's MXFP4 GEMM (hipBLASLt, through torch._scaled_mm) is timed beside this
library's GEMM on the same packed operands, as a comparison outside the step, and the library's
FP4 matrix-core probe measures what the matrix cores sustain with no memory traffic at all.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "act transform+quant GB/s and W4A4+LR linear TFLOPS at FLUX shape, % of roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA at the 2.4 GHz peak engine clock
PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA at 2.4 GHz
PEAK_CLOCK_MHZ = 2400.0
SLEEP_CYCLES = 2_000_000       # device-side sleep that lets the host queue a group of launches


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_flops(M, K, N, r, center):
    """Algorithmic flops of one linear: 4-bit product, both low-rank projections, rank-1."""
    return 2 * M * N * K + 2 * M * r * (K + N) + (2 * M * N if center else 0)


def gemm_flops(M, K, N, r, center):
    """Flops inside the W4A4 kernel launch: 4-bit product, low-rank up-projection, rank-1."""
    return 2 * M * N * K + 2 * M * N * r + (2 * M * N if center else 0)


def composite_floor_s(M, K, N, r):
    """Time of the linear (down-projection + GEMM) at the peaks: the 4-bit product at the
    MXFP4 peak plus both fp16 low-rank projections at the fp16 peak."""
    return 2 * M * N * K / (PEAK_FP4_TFLOPS * 1e12) + 2 * M * r * (K + N) / (PEAK_FP16_TFLOPS * 1e12)


def transform_bytes(M, K, center, fmt="mxfp4"):
    """Algorithmic HBM bytes of transform+quantize: fp16 in, 4-bit codes + E8M0 scales out
    (2 + 0.5 + 1/32 bytes per element), plus the fp16 mean per token when centring."""
    return M * K * 2 + M * K // 2 + M * K // 32 + (2 * M if center else 0)


def gemm_bytes(M, K, N, r, center):
    """Algorithmic HBM bytes of one W4A4 launch: both packed operands with their E8M0
    scales, T, L2, mu, wbar, and the fp16 output."""
    return (M + N) * (K // 2 + K // 32) + 2 * M * r + 2 * N * r + (2 * M + 2 * N if center else 0) + 2 * M * N


# source files whose kernels the recorded counters describe
_TRAFFIC_SOURCES = {
    "w4a4_gemm": ["w4a4_gemm.hip", "kq_device.hpp"],
    "transform": ["transform_quant.hip", "kq_device.hpp"],
}


def source_digest(kind):
    h = hashlib.sha256()
    for f in _TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, "w4a4_post_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kind):
    """HBM bytes per launch by layer, from the counter summary in profiles/, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_flux.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            m = re.match(r"\s*traffic-record:\s+kind=(\S+)\s+source=(\S+)\s+(.*)$", line)
            if m and m.group(1) == kind and m.group(2) == source_digest(kind):
                return {k: float(v) for k, v in (kv.split("=") for kv in m.group(3).split())}
    return None


def cpu_baseline(cfg_idx, rows, col_frac=4):
    """Time the float64 oracle (as it stands) on a bounded sample of the workload: `rows`
    tokens and 1/col_frac of the output columns of every linear; the transform+quantize and
    the linear are timed separately."""
    import synth
    from oracle import linear, pipeline
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = synth.CONFIGS[cfg_idx]
    flops = tq_bytes = 0
    t_tq = t_lin = 0.0
    for li, (name, K, N) in enumerate(cfg["layers"]):
        Ns = N // col_frac
        X = synth.activations(rows, K, cfg_idx, cfg["sigma_mu"], cfg["frames"])
        W, L1, L2 = synth.weights(K, N, cfg_idx, li, cfg["rank"])
        W, L2 = W[:Ns], L2[:Ns]
        xf = synth.xform_for(cfg_idx, li, K)
        fw = pipeline.fold_weights(W, xf, cfg["wfmt"])          # offline, not timed
        t0 = time.perf_counter()
        a = pipeline.transform_quantize(X, xf, cfg["fmt"], cfg["center"])
        t1 = time.perf_counter()
        linear.w4a4_linear(a["codes"], a["scales"], fw["wcodes"], fw["wscales"], X, L1, L2,
                           a["mu"], fw["wbar"] if cfg["center"] else None)
        t2 = time.perf_counter()
        t_tq += t1 - t0
        t_lin += t2 - t1
        flops += layer_flops(rows, K, Ns, cfg["rank"], cfg["center"])
        tq_bytes += transform_bytes(rows, K, cfg["center"])
    secs = t_tq + t_lin
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "transform_quant_s": round(t_tq, 3), "transform_quant_GBps": round(tq_bytes / t_tq / 1e9, 4),
            "linear_s": round(t_lin, 3), "linear_TFLOPs": flops / t_lin / 1e12,
            "sample": f"{rows} tokens x 1/{col_frac} of the output columns of each of the "
                      f"{len(cfg['layers'])} linears (full K): float64 transform+quantize ({t_tq:.1f} s) and "
                      f"dequantize+matmul linear ({t_lin:.1f} s), weight fold excluded"}


class Timer:
    """Per-launch durations that the host cannot bias (see the module docstring)."""

    def __init__(self, torch, n=50, warm=10, groups=5):
        self.torch, self.n, self.warm, self.groups = torch, n, warm, groups

    def __call__(self, fn):
        torch = self.torch
        for i in range(self.warm):
            fn(i)
        torch.cuda.synchronize()
        per = self.n // self.groups
        means = []
        k = self.warm
        for _ in range(self.groups):
            torch.cuda._sleep(SLEEP_CYCLES)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(per):
                fn(k)
                k += 1
            b.record()
            torch.cuda.synchronize()
            means.append(a.elapsed_time(b) / per)
        means.sort()
        return means[len(means) // 2]          # ms


def probe_clock(torch, kq, run=None, spin_us=300, samples=5):
    """Median shader clock in MHz from the library's clock probe (one wavefront counting
    shader cycles against the 100 MHz reference counter), launched on a stream of its own
    while `run()` keeps the GPU busy on the current stream (or on an idle GPU)."""
    side = torch.cuda.Stream()
    vals = []
    for _ in range(samples):
        out = torch.empty((2,), dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()
        if run is not None:
            for _ in range(4):          # about a millisecond of work first: the clock settles under load
                run()
        kq.clock_probe(spin_us, out=out, stream=side)
        if run is not None:
            for _ in range(4):
                run()
        torch.cuda.synchronize()
        cyc, ticks = (int(v) for v in out.tolist())
        if ticks > 0:
            vals.append(100.0 * cyc / ticks)
    vals.sort()
    return round(vals[len(vals) // 2], 1) if vals else None


def mfma_probe(torch, kq, codes, iters=1200, reps=5):
    """The scaled FP4 matrix cores with nothing else to do (kq_mfma_fp4_probe): one workgroup
    of four wavefronts per compute unit (one per SIMD, as the GEMM runs), each issuing
    sixteen independent 32x32x64 products per round on real activation codes; median rate
    over `reps` launches, each timed alone between two events, and the shader clock while it
    runs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus
    flops = 64 * iters * wgs * 2 * 32 * 32 * 64
    out = torch.empty((4 * wgs,), dtype=torch.float32, device=codes.device)
    kq.mfma_fp4_probe(iters, wgs, codes, out=out)
    torch.cuda.synchronize()
    rates = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        kq.mfma_fp4_probe(iters, wgs, codes, out=out)
        b.record()
        torch.cuda.synchronize()
        rates.append(flops / (a.elapsed_time(b) * 1e-3) / 1e12)
    rates.sort()
    mhz = probe_clock(torch, kq, lambda: kq.mfma_fp4_probe(iters, wgs, codes, out=out))
    return {"TFLOPs": round(rates[len(rates) // 2], 1), "frac_of_peak": round(rates[len(rates) // 2] / PEAK_FP4_TFLOPS, 4),
            "shader_mhz": mhz, "workgroups": wgs, "iters": iters,
            "method": "kq_mfma_fp4_probe: one workgroup of four wavefronts per compute unit, 16 independent "
                      "scaled FP4 32x32x64 products per wavefront and round, no memory traffic, operands from "
                      "the step's packed activation codes; median of 5 launches"}


def rotation_count(set_bytes):
    return max(2, math.ceil((1 << 30) / set_bytes))


def kron_config(torch, kq, synth, timer, cfg_idx, dev):
    """Per-launch timings of a Kronecker-transform MXFP4 configuration (no centring): the
    transform alone, the transform fused with the rank-32 down-projection (one kernel, X
    read once), and the W4A4 GEMM with the up-projection in its epilogue."""
    cfg = synth.CONFIGS[cfg_idx]
    M, r = cfg["M"], cfg["rank"]
    widths = sorted({K for _, K, _ in cfg["layers"]})
    X0 = {K: torch.from_numpy(synth.activations(M, K, cfg_idx, cfg["sigma_mu"], cfg["frames"])).to(dev) for K in widths}
    R = rotation_count(sum(x.numel() * 2 for x in X0.values()))
    Xs = [X0] + [{K: x.clone() for K, x in X0.items()} for _ in range(R - 1)]
    out = []
    for li, (name, K, N) in enumerate(cfg["layers"]):
        W, L1, L2 = synth.weights(K, N, cfg_idx, li, r)
        A, B = synth.kron_factors(cfg_idx, li)
        xf = kq.Xform.kron(A, B, K)
        wc, ws, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W).to(dev), xf, fmt="mxfp4", with_wbar=False)
        L1d, L2d = torch.from_numpy(L1).to(dev), torch.from_numpy(L2).to(dev)
        wsp = torch.empty((max(kq.lowrank_down_workspace_bytes(M, K, r), 16),), dtype=torch.uint8, device=dev)
        # one set of activation codes and T per rotated input, for the GEMM pass
        acts = []
        for s in range(R):
            c, sc, _, T = kq.transform_quantize_lowrank(Xs[s][K], xf, L1d, workspace=wsp)
            acts.append((c, sc, T))
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        c0, s0 = acts[0][0], acts[0][1]
        T0 = torch.empty_like(acts[0][2])
        t_tq = timer(lambda i: kq.transform_quantize(Xs[i % R][K], xf, codes=c0, scales=s0))
        t_fu = timer(lambda i: kq.transform_quantize_lowrank(Xs[i % R][K], xf, L1d, codes=c0, scales=s0, T=T0,
                                                             workspace=wsp))
        t_gm = timer(lambda i: kq.w4a4_linear_t(acts[i % R][0], acts[i % R][1], wc, ws, T=acts[i % R][2], L2=L2d,
                                                Y=Y))
        tb = transform_bytes(M, K, False)
        gfl = gemm_flops(M, K, N, r, False)
        lin = layer_flops(M, K, N, r, False)
        out.append({"layer": name, "M": M, "K": K, "N": N,
                    "transform_quant_us": round(t_tq * 1e3, 2), "transform_quant_GBps": round(tb / t_tq / 1e6, 1),
                    "transform_quant_frac_hbm": round(tb / t_tq / 1e6 / PEAK_HBM_GBS, 4),
                    "transform_lowrank_fused_us": round(t_fu * 1e3, 2),
                    "w4a4_gemm_us": round(t_gm * 1e3, 2), "w4a4_gemm_TFLOPs": round(gfl / t_gm / 1e9, 1),
                    "w4a4_gemm_frac_fp4": round(gfl / t_gm / 1e9 / PEAK_FP4_TFLOPS, 4),
                    "layer_us": round((t_fu + t_gm) * 1e3, 2), "layer_TFLOPs": round(lin / (t_fu + t_gm) / 1e9, 1)})
        log(f"cfg {cfg_idx} {name}: kron transform {t_tq*1e3:7.2f} us {tb/t_tq/1e6:7.1f} GB/s | fused with "
            f"lowrank {t_fu*1e3:7.2f} us | W4A4 {t_gm*1e3:8.2f} us {gfl/t_gm/1e9:7.1f} TFLOP/s")
        del acts
    del Xs
    torch.cuda.empty_cache()
    return {"workload": cfg["name"], "M": M, "rotated_input_sets": R, "layers": out}


def vendor_gemm(torch, kq, timer, layers, Xsets, R, center, M):
    """Per layer: the vendor MXFP4 GEMM (torch._scaled_mm over hipBLASLt, bf16 output) and this
    library's GEMM without the low-rank and rank-1 terms, on the same packed activations and
    weights, with their relative Frobenius difference.  None where torch has no such path."""
    rows = []
    for L in layers:
        K, N = L["K"], L["N"]
        sets = [kq.transform_quantize(Xsets[s][K], L["xf"], center=center)[:2] for s in range(R)]
        Yv = torch.empty((M, N), dtype=torch.float16, device=Xsets[0][K].device)
        a = [c.view(torch.float4_e2m1fn_x2) for c, _ in sets]
        sa = [sc.view(torch.float8_e8m0fnu) for _, sc in sets]
        b = L["wc"].view(torch.float4_e2m1fn_x2).t()
        sb = L["ws"].view(torch.float8_e8m0fnu)
        try:
            ref = torch._scaled_mm(a[0], b, sa[0], sb, out_dtype=torch.bfloat16)
        except (RuntimeError, TypeError, ValueError) as e:
            log(f"vendor MXFP4 GEMM unavailable: {str(e)[:200]}")
            return None
        kq.w4a4_linear_t(sets[0][0], sets[0][1], L["wc"], L["ws"], Y=Yv)
        torch.cuda.synchronize()
        rel = float(torch.linalg.norm(ref.float() - Yv.float()) / torch.linalg.norm(Yv.float()))
        t_v = timer(lambda i: torch._scaled_mm(a[i % R], b, sa[i % R], sb, out_dtype=torch.bfloat16))
        t_o = timer(lambda i: kq.w4a4_linear_t(sets[i % R][0], sets[i % R][1], L["wc"], L["ws"], Y=Yv))
        fl = 2 * M * N * K
        rows.append({"layer": L["name"], "M": M, "K": K, "N": N,
                     "vendor_us": round(t_v * 1e3, 2), "vendor_TFLOPs": round(fl / t_v / 1e9, 1),
                     "library_us": round(t_o * 1e3, 2), "library_TFLOPs": round(fl / t_o / 1e9, 1),
                     "speedup": round(t_v / t_o, 3), "rel_fro_diff_bf16_vs_fp16": round(rel, 5)})
        log(f"vendor MXFP4 GEMM {L['name']}: {t_v*1e3:7.2f} us vs library {t_o*1e3:7.2f} us "
            f"(x{t_v/t_o:.2f}); rel diff {rel:.2e}")
        del sets, a, sa, ref
    return {"api": "torch._scaled_mm (hipBLASLt), MXFP4 x MXFP4 with E8M0 block scales, bf16 output",
            "layers": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=0, help="activation buffer sets (0: enough for >= 1 GiB)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="tokens per linear in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other configurations and the transform variants")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the vendor-library MXFP4 GEMM timed beside the library's")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import w4a4_post_quantization_amd as kq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    timer = Timer(torch)
    CFG = 3
    cfg = synth.CONFIGS[CFG]
    M, r, center = cfg["M"], cfg["rank"], cfg["center"]

    # ---- inputs and offline preparation (untimed)
    widths = sorted({K for _, K, _ in cfg["layers"]})
    X0 = {K: torch.from_numpy(synth.activations(M, K, CFG, cfg["sigma_mu"], cfg["frames"])).to(dev) for K in widths}
    R = args.rotate or rotation_count(sum(x.numel() * 2 for x in X0.values()))
    Xsets = [X0] + [{K: x.clone() for K, x in X0.items()} for _ in range(R - 1)]
    layers = []
    for li, (name, K, N) in enumerate(cfg["layers"]):
        W, L1, L2 = synth.weights(K, N, CFG, li, r)
        perm, sign = synth.rpbh_params(K, CFG, li)
        xf = kq.Xform.rpbh(torch.from_numpy(perm).to(dev), torch.from_numpy(sign).to(dev))
        wc, ws, wbar = kq.fold_inverse_into_weights_nk(torch.from_numpy(W).to(dev), xf, fmt="mxfp4")
        layers.append(dict(
            name=name, K=K, N=N, xf=xf, wc=wc, ws=ws, wbar=wbar,
            L1=torch.from_numpy(L1).to(dev), L2=torch.from_numpy(L2).to(dev),
            codes=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
            mu=torch.empty((M,), dtype=torch.float16, device=dev),
            T=torch.empty((M, r), dtype=torch.float16, device=dev),
            lrws=torch.empty((max(kq.lowrank_down_workspace_bytes(M, K, r), 16),), dtype=torch.uint8, device=dev),
            Y=torch.empty((M, N), dtype=torch.float16, device=dev)))
    torch.cuda.synchronize()
    nl = len(layers)

    def act_pass(li, s):
        L, X = layers[li], Xsets[s % R][layers[li]["K"]]
        kq.transform_quantize_lowrank(X, L["xf"], L["L1"], center=center, codes=L["codes"], scales=L["scales"],
                                      mu=L["mu"], T=L["T"], workspace=L["lrws"])

    def gemm(li):
        L = layers[li]
        kq.w4a4_linear_t(L["codes"], L["scales"], L["wc"], L["ws"], T=L["T"], L2=L["L2"], mu=L["mu"],
                         wbar=L["wbar"], Y=L["Y"])

    def step(s):
        for li in range(nl):
            act_pass(li, s)
            gemm(li)

    # every rotated input set goes through the step once before the warm-up steps, so that
    # none is first touched (address translation, caches) inside the timed region
    for s in range(R):
        step(s)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps between two events on the stream the kernels run on
    t0 = time.perf_counter()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_start.record()
    for s in range(args.steps):
        step(args.warmup + s)
    e_end.record()
    host_submit = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e_start.elapsed_time(e_end) / args.steps
    log(f"{args.steps} steps: {ms_per_step * 1e3:.1f} us per step")

    # ---- per-launch durations, each call of the step on its own.  The GEMM reads packed
    # activations, T and mu rotated like the inputs (one set per input copy, made here)
    per_layer = []
    dur = []
    for li, L in enumerate(layers):
        K = L["K"]
        sets = []
        for s in range(R):
            c, sc, mu_s, T_s = kq.transform_quantize_lowrank(Xsets[s][K], L["xf"], L["L1"], center=center,
                                                              workspace=L["lrws"])
            sets.append((c, sc, mu_s, T_s))
        t_tq = timer(lambda i: kq.transform_quantize(Xsets[i % R][K], L["xf"], center=center, codes=L["codes"],
                                                     scales=L["scales"], mu=L["mu"]))
        t_lr = timer(lambda i: kq.lowrank_down(Xsets[i % R][K], L["L1"], T=L["T"], workspace=L["lrws"]))
        t_fu = timer(lambda i: act_pass(li, i))
        t_gm = timer(lambda i: kq.w4a4_linear_t(sets[i % R][0], sets[i % R][1], L["wc"], L["ws"], T=sets[i % R][3],
                                                L2=L["L2"], mu=sets[i % R][2], wbar=L["wbar"], Y=L["Y"]))
        dur.append((t_tq, t_lr, t_fu, t_gm))
        log(f"per-launch {L['name']}: {t_tq * 1e3:.2f} / {t_lr * 1e3:.2f} / {t_fu * 1e3:.2f} / {t_gm * 1e3:.2f} us")
        del sets

    # ---- the GPU clock while the GEMMs run
    def gemm_round():
        for li in range(nl):
            gemm(li)
    clock_mhz = probe_clock(torch, kq, gemm_round)
    clock_idle = probe_clock(torch, kq)
    log(f"shader clock: {clock_mhz} MHz while the GEMMs run, {clock_idle} MHz idle")

    # ---- what the FP4 matrix cores sustain alone, for the GEMM's standing against it
    probe = mfma_probe(torch, kq, layers[0]["codes"].view(-1))
    log(f"FP4 matrix-core probe: {probe['TFLOPs']} TFLOP/s at {probe['shader_mhz']} MHz")

    # ---- the vendor library's MXFP4 GEMM (hipBLASLt through torch._scaled_mm) on the step's
    # packed operands, beside this library's GEMM with no epilogue terms (the same product):
    # a comparison only, nothing of the step goes through it
    vendor = None
    if not args.no_vendor:
        vendor = vendor_gemm(torch, kq, timer, layers, Xsets, R, center, M)

    # ---- the other configurations, per launch
    others = {}
    variants, sana = [], []
    if not args.no_variants:
        for ci, key in ((4, "cogvideox_like_cfg4"), (1, "pixart_block_cfg1"), (0, "pixart_single_cfg0")):
            others[key] = kron_config(torch, kq, synth, timer, ci, dev)

        # transform variants beside the path (not part of the step), at the step's widths:
        # the Kronecker factors and a dense 32x32 P on the streaming matrix-core kernel,
        # per-block factors on theirs, MXFP4 without centring, each also behind
        # power-of-two channel scaling (exponent 6 on the planted outlier channels)
        for K in widths:
            A, B = synth.kron_factors(CFG, 0)
            P = torch.from_numpy(synth.dense_block(CFG, 0)).to(dev)
            codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
            pts = torch.from_numpy(synth.pts_exponents(K, synth.outlier_channels(M, K, CFG, cfg["sigma_mu"]))).to(dev)
            Ab, Bb = synth.kron_block_factors(CFG, 0, K // 32)
            AB = torch.from_numpy(kq.Xform.pack_block_factors(Ab, Bb)).to(dev)
            kx, dx, bx = kq.Xform.kron(A, B, K), kq.Xform.dense(P, K), kq.Xform.kron_blocks(AB, K)
            L = next(L for L in layers if L["K"] == K)
            for name, xf, c in (("rpbh_32 (no centring)", L["xf"], False), ("rpbh_32 centred", L["xf"], True),
                                ("kron_4x8", kx, False), ("dense_32", dx, False), ("kron_blocks", bx, False),
                                ("kron_4x8+pts", kx.with_pts(pts), False), ("dense_32+pts", dx.with_pts(pts), False),
                                ("kron_blocks+pts", bx.with_pts(pts), False)):
                ms = timer(lambda i, xf=xf, c=c: kq.transform_quantize(Xsets[i % R][K], xf, fmt="mxfp4", center=c,
                                                                       codes=codes, scales=scales, mu=L["mu"]))
                tb = transform_bytes(M, K, c)
                variants.append({"transform": name, "M": M, "K": K, "us": round(ms * 1e3, 2),
                                 "GBps": round(tb / ms / 1e6, 1), "frac": round(tb / ms / 1e6 / PEAK_HBM_GBS, 4)})
                log(f"variant {name:>22} K={K:5d}: {ms*1e3:7.2f} us {tb/ms/1e6:8.1f} GB/s")

        # the SANA-like workload's Lloyd-Max path: per layer the RPBH + per-token Lloyd-Max
        # transform (4-bit sign-magnitude codes, one fp32 scale per token) and the W2A4 linear
        # (2-bit weights with fp16 group scales, dequantized through LDS tables to fp16 for
        # the matrix cores: its roofline is the fp16 peak)
        c2 = synth.CONFIGS[2]
        M2 = c2["M"]
        for li, (name, K, N) in enumerate(c2["layers"]):
            X2 = torch.from_numpy(synth.activations(M2, K, 2, c2["sigma_mu"], c2["frames"])).to(dev)
            nrot = rotation_count(X2.numel() * 2)
            X2s = [X2] + [X2.clone() for _ in range(nrot - 1)]
            W2, _, _ = synth.weights(K, N, 2, li, 0)
            perm, sign = synth.rpbh_params(K, 2, li)
            xf2 = kq.Xform.rpbh(torch.from_numpy(perm).to(dev), torch.from_numpy(sign).to(dev))
            wc2, ws2, _ = kq.fold_inverse_into_weights_nk(torch.from_numpy(W2).to(dev), xf2, fmt="lm2")
            sets2 = [kq.transform_quantize(X2s[s], xf2, fmt="lm4")[:2] for s in range(nrot)]
            codes2 = torch.empty((M2, K // 2), dtype=torch.uint8, device=dev)
            scales2 = torch.empty((M2,), dtype=torch.float32, device=dev)
            Y2 = torch.empty((M2, N), dtype=torch.float16, device=dev)
            ms_tq = timer(lambda i: kq.transform_quantize(X2s[i % nrot], xf2, fmt="lm4", codes=codes2, scales=scales2))
            ms_mm = timer(lambda i: kq.w4a4_linear_t(sets2[i % nrot][0], sets2[i % nrot][1], wc2, ws2, fmt="lm2",
                                                     Y=Y2))
            tb = M2 * K * 2 + M2 * K // 2 + M2 * 4
            fl = 2 * M2 * N * K
            sana.append({"layer": name, "M": M2, "K": K, "N": N,
                         "transform_lm4_us": round(ms_tq * 1e3, 2), "transform_GBps": round(tb / ms_tq / 1e6, 1),
                         "transform_frac_hbm": round(tb / ms_tq / 1e6 / PEAK_HBM_GBS, 4),
                         "w2a4_gemm_us": round(ms_mm * 1e3, 2), "w2a4_TFLOPs": round(fl / ms_mm / 1e9, 1),
                         "w2a4_frac_fp16_peak": round(fl / ms_mm / 1e9 / PEAK_FP16_TFLOPS, 4)})
            log(f"sana-like {name}: RPBH+LM4 {ms_tq*1e3:7.2f} us {tb/ms_tq/1e6:8.1f} GB/s | "
                f"W2A4 {ms_mm*1e3:7.2f} us {fl/ms_mm/1e9:8.1f} TFLOP/s")
            del X2s, sets2

    if args.copy_calibration:
        # a plain elementwise pass over 256 MiB (read 256 MiB, write 256 MiB): the reference
        # dispatch for scaling the HBM byte counters
        src = torch.empty((1 << 27,), dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    traffic_gemm = recorded_traffic("w4a4_gemm")
    traffic_tq = recorded_traffic("transform")
    tot_flops = tot_gemm_flops = tot_tq_bytes = 0
    tot_tq_ms = tot_lr_ms = tot_fu_ms = tot_gemm_ms = 0.0
    floor_s = 0.0
    for L, (tq_ms, lr_ms, fu_ms, gm_ms) in zip(layers, dur):
        K, N = L["K"], L["N"]
        fl = layer_flops(M, K, N, r, center)
        gfl = gemm_flops(M, K, N, r, center)
        tb = transform_bytes(M, K, center)
        tot_flops += fl
        tot_gemm_flops += gfl
        tot_tq_bytes += tb
        tot_tq_ms += tq_ms
        tot_lr_ms += lr_ms
        tot_fu_ms += fu_ms
        tot_gemm_ms += gm_ms
        floor_s += composite_floor_s(M, K, N, r)
        per_layer.append({
            "layer": L["name"], "M": M, "K": K, "N": N,
            "transform_quant_us": round(tq_ms * 1e3, 2),
            "transform_quant_GBps": round(tb / tq_ms / 1e6, 1),
            "transform_quant_frac_hbm": round(tb / tq_ms / 1e6 / PEAK_HBM_GBS, 4),
            "lowrank_down_us": round(lr_ms * 1e3, 2),
            "transform_lowrank_call_us": round(fu_ms * 1e3, 2),
            "w4a4_gemm_us": round(gm_ms * 1e3, 2),
            "w4a4_gemm_TFLOPs": round(gfl / gm_ms / 1e9, 1),
            "w4a4_gemm_frac_fp4": round(gfl / gm_ms / 1e9 / PEAK_FP4_TFLOPS, 4),
            "w4a4_gemm_algorithmic_bytes": gemm_bytes(M, K, N, r, center),
            "w4a4_gemm_traffic_bytes": traffic_gemm.get(L["name"]) if traffic_gemm else None,
            "transform_quant_traffic_bytes": traffic_tq.get(L["name"]) if traffic_tq else None,
            "linear_TFLOPs": round(fl / (lr_ms + gm_ms) / 1e9, 1),
            "composite_g2g3_frac": round(composite_floor_s(M, K, N, r) / ((lr_ms + gm_ms) * 1e-3), 4),
        })
        log(f"{L['name']:>4}: transform+quant {tq_ms*1e3:8.2f} us {tb/tq_ms/1e6:8.1f} GB/s | lowrank-down "
            f"{lr_ms*1e3:7.2f} us | both in one call {fu_ms*1e3:7.2f} us | W4A4 GEMM {gm_ms*1e3:8.2f} us "
            f"{gfl/gm_ms/1e9:8.1f} TFLOP/s")

    value = tot_flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = tot_gemm_flops / (tot_gemm_ms * 1e-3) / 1e12
    tq_gbs = tot_tq_bytes / (tot_tq_ms * 1e-3) / 1e9
    composite = floor_s / ((tot_lr_ms + tot_gemm_ms) * 1e-3)
    peak_at_clock = PEAK_FP4_TFLOPS * clock_mhz / PEAK_CLOCK_MHZ if clock_mhz else None
    log(f"step {ms_per_step*1e3:.1f} us; whole-step linear throughput {value:.1f} TFLOP/s; "
        f"GEMM {gemm_tflops:.1f} TFLOP/s ({gemm_tflops/PEAK_FP4_TFLOPS:.1%} of MXFP4 peak); composite "
        f"G2+G3 {composite:.1%}; transform+quant {tq_gbs:.1f} GB/s ({tq_gbs/PEAK_HBM_GBS:.1%} of HBM peak); "
        f"clock {clock_mhz} MHz; wall {wall:.2f} s; host submission {host_submit / args.steps * 1e6:.1f} us per step")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": "FLUX.1-like joint block linears, M=4608 tokens (4096 image + 512 text): "
                               "qkv 3072->9216, fc1 3072->12288, fc2 12288->3072; centred RPBH-32 + MXFP4 "
                               "activations and weights, rank-32 fp16 branch, rank-1 mean restore",
                   "tokens": M, "rotated_input_sets": R},
        "roofline": {"bound": "mfma", "kernel": "kq_w4a4_linear_t (W4A4 GEMM + fused low-rank/rank-1 epilogue), "
                                                "the three launches of one step",
                     "achieved": round(gemm_tflops, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": (round(sum(traffic_gemm.get(L["name"], 0.0) for L in layers))
                                 if traffic_gemm else None),
                     "algorithmic_bytes": sum(gemm_bytes(M, L["K"], L["N"], r, center) for L in layers),
                     "peak_at_measured_clock": round(peak_at_clock, 1) if peak_at_clock else None,
                     "frac_at_measured_clock": round(gemm_tflops / peak_at_clock, 4) if peak_at_clock else None,
                     "frac_of_mfma_probe": round(gemm_tflops / probe["TFLOPs"], 4)},
        "roofline_composite_g2g3": {"bound": "mfma", "definition": "(2MNK / MXFP4 peak + 2Mr(K+N) / fp16 peak) / "
                                                                  "(down-projection + GEMM time), the three layers",
                                    "frac": round(composite, 4),
                                    "floor_us": round(floor_s * 1e6, 2),
                                    "time_us": round((tot_lr_ms + tot_gemm_ms) * 1e3, 2)},
        "roofline_transform": {"bound": "hbm", "kernel": "kq_transform_quantize (centre + RPBH-32 + MXFP4), "
                                                         "the three launches of one step",
                               "achieved": round(tq_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(tq_gbs / PEAK_HBM_GBS, 4),
                               "traffic": (round(sum(traffic_tq.get(L["name"], 0.0) for L in layers))
                                           if traffic_tq else None),
                               "algorithmic_bytes": tot_tq_bytes},
        "clock": {"shader_mhz_during_gemm": clock_mhz, "shader_mhz_idle": clock_idle,
                  "peak_engine_mhz": PEAK_CLOCK_MHZ,
                  "source": "kq_clock_probe (shader cycles over 300 us of the 100 MHz reference counter) on a "
                            "second stream while the step's three GEMMs run back to back; median of 5"},
        "transform_quant_GBps": round(tq_gbs, 1),
        "w4a4_gemm_TFLOPs": round(gemm_tflops, 1),
        "linear_TFLOPs": round(tot_flops / ((tot_lr_ms + tot_gemm_ms) * 1e-3) / 1e12, 1),
        "per_layer": per_layer,
        "timing": "per-launch: median of 5 group means, 50 launches after 10 warm-up, host queued ahead",
        "other_configs": others,
        "context": "KroQuant page: its quantization kernel up to 14% faster than SmoothQuant's on an MI350 "
                   "(relative only, other chip)",
        "transform_variants": variants,
        "sana_like_lloyd_max": sana,
        "vendor_mxfp4_gemm": vendor,
        "mfma_fp4_probe": probe,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(CFG, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

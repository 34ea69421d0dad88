#!/usr/bin/env python3
"""Throughput of the sparse MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ``moe_forward`` of the whole layer (router GEMM, top-k + softmax,
dispatch, activation quantisation, GEMM1 + SwiGLU + requantisation, GEMM2, combine)
over one batch of T synthetic tokens whose inputs are already resident in HBM.  The
default workload is the gpt-oss-120b-shaped prefill layer (T=8192, H=2880, E=128,
top-4, I=2880).  The timed region brackets the dominant GEMM of every step with HIP
events recorded between the library's kernels on the same stream
(``moe_forward_profiled``), which gives the roofline's live kernel time; the other stage
times come from a separate, untimed pass that records every stage boundary.  The same
run also times the two decode-sized layers (gpt-oss-20b and qwen3-235b shapes) with the
caches evicted before every step.  One JSON line.

The CPU baseline is the fp64 oracle (test infrastructure) on the whole layer, with the
BLAS threads on every core of the process's affinity mask.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE layer tokens/s + TFLOP/s & HBM GB/s vs MI355X peak (gpt-oss-120b shape)"


def kb(n):
    return (n + 127) // 128


def algorithmic(shape, counts, fmt="block"):
    """Algorithmic flops and compulsory HBM bytes of the layer and of its two GEMMs.

    Compulsory bytes: x and out (bf16), the router, and the weights of every *active*
    expert (codes, scales, biases; an expert with no routed token is never read).  The
    intermediates (x codes, h, y) are implementation traffic and are not counted.  Per
    GEMM: its own weights.  Scales: fp32 per 128x128 weight block, or (MXFP8, MXFP4) one
    E8M0 byte per 32 elements along K.  MXFP4 weight elements are half a byte."""
    T, H, E, k, I = shape.T, shape.H, shape.E, shape.top_k, shape.I
    rows = T * k
    active = int((counts > 0).sum())
    wb = 0.5 if fmt == "mxfp4" else 1
    if fmt in ("mxfp8", "mxfp4"):
        sw13, sw2 = 2 * I * H // 32, H * I // 32
    else:
        sw13, sw2 = kb(2 * I) * kb(H) * 4, kb(H) * kb(I) * 4
    w13 = active * int(2 * I * H * wb + sw13 + (2 * I * 2 if shape.expert_bias else 0))
    w2 = active * int(H * I * wb + sw2 + (H * 2 if shape.expert_bias else 0))
    layer_bytes = T * H * 2 + E * H * 4 + E * 4 + w13 + w2 + T * H * 2
    g1_flops = 2 * rows * H * 2 * I
    g2_flops = 2 * rows * I * H
    return dict(
        active_experts=active,
        layer_flops=g1_flops + g2_flops, layer_bytes=layer_bytes,
        gemm1=dict(flops=g1_flops, bytes=w13),
        gemm2=dict(flops=g2_flops, bytes=w2))


def pmc_record(workload, kernel):
    """The committed rocprofv3 counter summary of one GEMM launch on this workload, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if sources_sha256(rec.get("sources", ["gemm.hip"])) == rec.get("source_sha256") else None


def sources_sha256(names):
    """sha256 of the named kernel sources (csrc/), concatenated in the given order."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_moe_ffn_gemm_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gpu_sysfs(torch, index=0):
    """sysfs directory of the torch device, matched by PCI address (None if not found)."""
    p = torch.cuda.get_device_properties(index)
    try:
        addr = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}."
    except AttributeError:
        return None
    for d in glob.glob("/sys/class/drm/card*/device"):
        if (os.path.basename(os.path.realpath(d)).startswith(addr)
                and os.path.exists(os.path.join(d, "pp_dpm_sclk"))):
            return d
    return None


def current_mhz(sysdir, name):
    """The level a pp_dpm_* file marks as current ('*'), in MHz (None if unreadable)."""
    if sysdir is None:
        return None
    try:
        with open(os.path.join(sysdir, name)) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*mhz", line, re.I)
                    return int(m.group(1)) if m else None
    except OSError:
        pass
    return None


def device_copy_gbs(torch, dev, mib=1024, reps=5):
    """Bytes read + written per second by a plain 1 GiB device-to-device copy (context for
    the vendor HBM peak)."""
    a = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * a.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def blas_vendor():
    import numpy as np
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:
        return "unknown"


def cpu_baseline(shape, li, fmt="block"):
    """The oracle's forward on the whole layer (every token, every expert), float64 NumPy,
    BLAS threads on every core of the affinity mask.  The weight conversion (the oracle's
    own quantiser, from the generator's fp32 weights) is offline work and is not timed."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import moe_ref as R
    from synth import expert_weights
    from synth.cases import _base_shape

    cores = len(os.sched_getaffinity(0))
    vendor = blas_vendor()
    print(f"[bench] cpu baseline: oracle on the whole layer, {cores} cores, BLAS {vendor}",
          file=sys.stderr, flush=True)
    base = _base_shape(shape)
    dev = "cuda" if base.weights_on_device else "cpu"
    quant = {"block": R.quantize_blocks, "mxfp8": R.quantize_mx, "mxfp4": R.quantize_mxfp4}[fmt]

    def by_rows(w):   # 128-row slices (whole scale blocks): the same codes, cache-sized
        parts = [quant(w[i:i + 128]) for i in range(0, w.shape[0], 128)]
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])

    t_conv = time.perf_counter()
    c13, s13, c2, s2 = {}, {}, {}, {}
    with ThreadPoolExecutor(max_workers=cores) as ex:
        for e0 in range(0, shape.E, 32):     # draw 32 experts at a time, convert in parallel
            host = {e: (expert_weights(shape, "w13", e, dev).cpu().numpy(),
                        expert_weights(shape, "w2", e, dev).cpu().numpy())
                    for e in range(e0, min(shape.E, e0 + 32))}
            conv = dict(zip(host, ex.map(lambda ws: (by_rows(ws[0]), by_rows(ws[1])), host.values())))
            del host
            for e, ((q13, t13), (q2, t2)) in conv.items():
                c13[e], s13[e], c2[e], s2[e] = q13, t13, q2, t2
    t_conv = time.perf_counter() - t_conv
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        R.forward(li.x, li.router_w, li.router_b, shape.top_k, shape.I, c13, s13, li.b13, c2, s2,
                  li.b2, fmt=fmt)
        dt = time.perf_counter() - t0
    return {"value": round(shape.T / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas": vendor, "seconds": round(dt, 2),
            "sample": f"the whole layer: all {shape.T} tokens, all {shape.E} experts; fp64 NumPy "
                      f"forward incl. per-expert weight dequantisation, {dt:.1f} s (weight "
                      f"conversion {t_conv:.1f} s, untimed)"}


def roofline(k_alg, k_s, shape, fmt, kernel):
    """Roofline of the dominant kernel, both fractions: algorithmic FP8 flops against the
    5.0 PFLOP/s FP8 peak and algorithmic (compulsory) bytes against 8 TB/s, over the
    kernel's live launch time.  The line leads with the one the layer's target is stated
    on: the matrix cores when the kernel's intensity is within 4x of the ridge (625 flop/B)
    or above it (prefill-sized groups), HBM for weight-streaming (decode-sized) layers.
    ``traffic`` is the kernel's measured HBM bytes per launch from the committed rocprofv3
    counter summary, when it was taken on the current kernel source (else null)."""
    flops, nbytes = k_alg["flops"], k_alg["bytes"]
    mfma = flops / k_s / 1e12
    hbm = nbytes / k_s / 1e9
    ridge = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / nbytes >= ridge / 4:
        roof = {"bound": "mfma", "achieved": round(mfma, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(mfma / PEAK_FP8_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(hbm / PEAK_HBM_GBS, 4)}
    prof_name = shape.name if fmt == "block" else f"{shape.name}-{fmt}"
    rec = pmc_record(prof_name, kernel)
    roof["traffic"] = rec.get("hbm_bytes_per_launch") if rec else None
    roof["traffic_source"] = (f"profiles/pmc_{kernel}_{prof_name}.json: rocprofv3 --pmc FETCH_SIZE, "
                              f"WRITE_SIZE, scaled by a 1 GiB copy" if rec else None)
    roof.update({
        "kernel": kernel, "kernel_us": round(k_s * 1e6, 2),
        "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
        "intensity_flop_per_byte": round(flops / nbytes, 1),
        "mfma_tflops": round(mfma, 2), "mfma_frac": round(mfma / PEAK_FP8_TFLOPS, 4),
        "hbm_gbs": round(hbm, 1), "hbm_frac": round(hbm / PEAK_HBM_GBS, 4)})
    return roof


def decode_layer(shape, fmt, dev, steps=40, warmup=5, fused_only=False):
    """A decode-sized (weight-streaming) layer timed in the same run: per-step times with
    the caches evicted before every step by reading a 1 GiB buffer (outside the events),
    and warm; the compulsory bytes (bench.algorithmic) over the cold median against 8 TB/s.
    Also the cold median of the one-kernel path; with fused_only, that path alone."""
    import numpy as np
    import torch

    import sparse_moe_ffn_gemm_amd as moe
    from synth import expert_weights, make_inputs

    li = make_inputs(shape)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    layer = moe.MoELayer.from_expert_weights(
        torch.from_numpy(li.router_w), torch.from_numpy(li.router_b), shape.top_k,
        bf(li.b13) if shape.expert_bias else None, bf(li.b2) if shape.expert_bias else None,
        lambda e: expert_weights(shape, "w13", e, "cuda"),
        lambda e: expert_weights(shape, "w2", e, "cuda"), device=dev, fmt=fmt)
    x = bf(li.x)
    out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=dev)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k, dev)
    ws = layer.workspace(shape.T)
    fa = (x, layer.router_w, layer.router_b, layer.w13, layer.w13_scales, layer.b13, layer.w2,
          layer.w2_scales, layer.b2, shape.top_k)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    if not fused_only:
        for _ in range(warmup):
            moe.forward(*fa, out=out, routing=routing, workspace=ws)

    def run(cold):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            if cold:
                torch.sum(flush, dim=0, out=sink)
            a.record()
            moe.forward(*fa, out=out, routing=routing, workspace=ws)
            b.record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    cold, warm = (run(True), run(False)) if not fused_only else (None, None)
    # the same layer through the one-kernel decode path (moe_forward_fused)
    fused = None
    try:
        for _ in range(warmup):
            moe.forward_fused(*fa, out=out, routing=routing, workspace=ws)
        evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evf:
            torch.sum(flush, dim=0, out=sink)
            a.record()
            moe.forward_fused(*fa, out=out, routing=routing, workspace=ws)
            b.record()
        torch.cuda.synchronize()
        st = moe.fused_status(ws, shape.T, shape.H, shape.E, shape.top_k, shape.I)
        tf = np.array([a.elapsed_time(b) for a, b in evf]) * 1e3
        fused = {"cold_us_p50": round(float(np.median(tf)), 1), "waits_ok": st == 0}
        print(f"[bench] {shape.name}: one-kernel decode path cold p50 {fused['cold_us_p50']:.1f} us",
              file=sys.stderr, flush=True)
    except moe.MoEError as e:             # outside the fused kernel's envelope
        fused = {"unsupported": str(e)}
    if fused_only:
        del layer, ws, flush
        torch.cuda.empty_cache()
        return fused
    counts = routing["expert_counts"].cpu().numpy()
    alg = algorithmic(shape, counts, fmt)
    p50 = float(np.median(cold))
    gbs = alg["layer_bytes"] / (p50 * 1e-6) / 1e9
    print(f"[bench] {shape.name}: cold p50 {p50:.1f} us, warm p50 {np.median(warm):.1f} us, "
          f"{gbs:.0f} GB/s of compulsory bytes ({gbs / PEAK_HBM_GBS:.1%} of 8 TB/s)",
          file=sys.stderr, flush=True)
    r = {"T": shape.T, "H": shape.H, "E": shape.E, "top_k": shape.top_k, "I": shape.I,
         "cold_us": {"p10": round(float(np.percentile(cold, 10)), 1), "p50": round(p50, 1),
                     "p90": round(float(np.percentile(cold, 90)), 1)},
         "warm_us_p50": round(float(np.median(warm)), 1),
         "tokens_per_s": round(shape.T / (p50 * 1e-6), 1),
         "compulsory_bytes": alg["layer_bytes"], "active_experts": alg["active_experts"],
         "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "steps": steps,
         "path": "multi-kernel (moe_forward)", "fused_kernel": fused}
    del layer, ws, flush
    torch.cuda.empty_cache()
    return r


def copy_calibration(gib=1.0, reps=5):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "reps": reps}))


def one_token_per_expert(args):
    """The pages' decode GEMM benchmark ("Hosting Qwen on Blackwell", section "MoE GEMM":
    every expert activated with a single token, over expert-parallel degrees): one GPU's
    share of the qwen3-235b layer (H 4096, I 1536, 128 experts) at EP degree d is 128/d
    experts, each routed exactly one token (T = 128/d, top_k = 1, a router with each
    token's own direction planted in its expert's row).  Prints a table on stderr and one
    JSON line with the GEMM and layer times per (d, weight format)."""
    import numpy as np
    import torch

    import sparse_moe_ffn_gemm_amd as moe
    from sparse_moe_ffn_gemm_amd._lib import PROFILE_STAGES
    from synth import expert_weights, make_inputs
    from synth.cases import LayerShape

    dev = torch.device("cuda:0")
    results = []
    for fmt in ("block", "mxfp8", "mxfp4"):
        for ep in (1, 2, 4, 8, 16, 32, 64):
            n = 128 // ep
            shape = LayerShape(f"qwen3-235b-one-token-per-expert-ep{ep}", T=n, H=4096, E=n,
                               top_k=1, I=1536, seed=3, expert_bias=False,
                               weights_on_device=True, router="one_per_expert")
            li = make_inputs(shape)
            bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
            layer = moe.MoELayer.from_expert_weights(
                torch.from_numpy(li.router_w), torch.from_numpy(li.router_b), 1, None, None,
                lambda e: expert_weights(shape, "w13", e, "cuda"),
                lambda e: expert_weights(shape, "w2", e, "cuda"), device=dev, fmt=fmt)
            x = bf(li.x)
            out = torch.empty((n, shape.H), dtype=torch.bfloat16, device=dev)
            routing = moe.new_routing(n, n, 1, dev)
            ws = layer.workspace(n)
            fa = (x, layer.router_w, layer.router_b, layer.w13, layer.w13_scales, None,
                  layer.w2, layer.w2_scales, None, 1)
            for _ in range(args.warmup):
                moe.forward(*fa, out=out, routing=routing, workspace=ws)
            torch.cuda.synchronize()
            counts = routing["expert_counts"].cpu().numpy()
            if not np.all(counts == 1):
                raise RuntimeError(f"ep {ep}: expert counts {counts} (expected one token each)")
            nprof = max(10, args.steps)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(PROFILE_STAGES) + 1)]
                  for _ in range(nprof)]
            for k in range(nprof):
                moe.forward_profiled(ev[k], *fa, out=out, routing=routing, workspace=ws)
            torch.cuda.synchronize()
            st = {name: float(np.median([ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(nprof)]))
                  for i, name in enumerate(PROFILE_STAGES)}
            steps = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(max(20, args.steps))]
            for a_, b_ in steps:
                a_.record()
                moe.forward(*fa, out=out, routing=routing, workspace=ws)
                b_.record()
            torch.cuda.synchronize()
            layer_ms = float(np.median([a_.elapsed_time(b_) for a_, b_ in steps]))
            wbytes = n * 3 * shape.H * shape.I * {"block": 1 + 1 / 4096, "mxfp8": 1 + 1 / 32,
                                                   "mxfp4": 0.5 + 1 / 32}[fmt]
            gemm_us = (st["gemm1"] + st["gemm2"]) * 1e3
            r = {"ep": ep, "experts": n, "format": fmt, "gemm1_us": round(st["gemm1"] * 1e3, 2),
                 "gemm2_us": round(st["gemm2"] * 1e3, 2), "gemm_us": round(gemm_us, 2),
                 "layer_us_p50": round(layer_ms * 1e3, 2),
                 "weight_gbs": round(wbytes / (gemm_us * 1e-6) / 1e9, 1)}
            results.append(r)
            print(f"[microbench] {fmt:6s} EP {ep:3d} ({n:3d} experts x 1 token): GEMM1 "
                  f"{r['gemm1_us']:7.1f} us  GEMM2 {r['gemm2_us']:7.1f} us  layer p50 "
                  f"{r['layer_us_p50']:7.1f} us  weights {r['weight_gbs']:7.1f} GB/s",
                  file=sys.stderr, flush=True)
            del layer, ws, x, out
            torch.cuda.empty_cache()
    print(json.dumps({"microbench": "one-token-per-expert",
                      "layer": "qwen3-235b MoE (H 4096, I 1536, 128 experts), one GPU's share at EP degree d",
                      "data": "synthetic", "results": results}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt-oss-120b-prefill")
    ap.add_argument("--no-decode-layers", action="store_true",
                    help="skip the two decode-sized layers timed after the workload")
    ap.add_argument("--format", choices=["block", "mxfp8", "mxfp4"], default="block",
                    help="expert weight format: 128x128 block scales (default), MXFP8, or MXFP4 "
                         "weights with MXFP8 activations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--microbench", choices=["one-token-per-expert"],
                    help="instead of the layer benchmark: the decode GEMM sweep over "
                         "expert-parallel degrees, every expert given one token")
    ap.add_argument("--fused-only", action="store_true",
                    help="only time the one-kernel decode path (moe_forward_fused) on --workload "
                         "(decode-sized), caches evicted before every step; prints one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the layer runs on one GPU; multi-GPU runs (--gpus > 1) are not "
              "supported (expert-parallel sharding is a design, not an implementation)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    if args.fused_only:
        from synth import SHAPES
        import torch
        r = decode_layer(SHAPES[args.workload], args.format, torch.device("cuda:0"),
                         steps=args.steps, warmup=args.warmup, fused_only=True)
        print(json.dumps({"fused_only": args.workload, "format": args.format, **r}), flush=True)
        return
    if args.microbench:
        one_token_per_expert(args)
        return

    import sparse_moe_ffn_gemm_amd as moe
    from sparse_moe_ffn_gemm_amd._lib import PROFILE_STAGES
    from synth import SHAPES, expert_weights, make_inputs

    if args.workload not in SHAPES:
        sys.exit(f"unknown workload {args.workload}; one of {list(SHAPES)}")
    shape = SHAPES[args.workload]
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    li = make_inputs(shape)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    layer = moe.MoELayer.from_expert_weights(
        torch.from_numpy(li.router_w), torch.from_numpy(li.router_b), shape.top_k,
        bf(li.b13) if shape.expert_bias else None, bf(li.b2) if shape.expert_bias else None,
        lambda e: expert_weights(shape, "w13", e, "cuda"),
        lambda e: expert_weights(shape, "w2", e, "cuda"), device=dev, fmt=args.format)
    x = bf(li.x)
    out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=dev)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k, dev)
    ws = layer.workspace(shape.T)
    fwd_args = (x, layer.router_w, layer.router_b, layer.w13, layer.w13_scales, layer.b13,
                layer.w2, layer.w2_scales, layer.b2, shape.top_k)
    torch.cuda.synchronize()
    sysdir = gpu_sysfs(torch)
    clocks = {"sclk_mhz_before": current_mhz(sysdir, "pp_dpm_sclk"),
              "mclk_mhz_before": current_mhz(sysdir, "pp_dpm_mclk")}
    print(f"[bench] {shape.name}: setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr,
          flush=True)

    for _ in range(args.warmup):
        moe.forward(*fwd_args, out=out, routing=routing, workspace=ws)
    torch.cuda.synchronize()

    # per-stage breakdown, outside the timed region: every stage boundary recorded
    nprof = max(3, min(args.steps, 10))
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(PROFILE_STAGES) + 1)]
              for _ in range(nprof)]
    for s in range(nprof):
        moe.forward_profiled(events[s], *fwd_args, out=out, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                                     for s in range(nprof)]))
                for i, name in enumerate(PROFILE_STAGES)}
    # dominant kernel: the one with the most device time
    dom = max(("gemm1", "gemm2"), key=lambda k: stage_ms[k])
    i_dom = PROFILE_STAGES.index(dom)

    # timed region: K steps; only the dominant kernel is bracketed by events (each recorded
    # event adds a small gap between kernels), so its launch time is measured live
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for s in range(args.steps):
        evs = [None] * (len(PROFILE_STAGES) + 1)
        evs[i_dom], evs[i_dom + 1] = dom_ev[s]
        moe.forward_profiled(evs, *fwd_args, out=out, routing=routing, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in dom_ev]))
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall:.3f} s), {dom} "
          f"{dom_ms * 1e3:.1f} us; stages (separate pass) "
          + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in stage_ms.items()), file=sys.stderr,
          flush=True)

    # Per-step distribution (after the timed region): each step bracketed by its own events;
    # for weight-streaming (HBM-bound) layers also with the caches evicted before every step
    # by reading a 1 GiB buffer (outside the events; a read sweep leaves no dirty lines to
    # write back during the step), so no weight bytes come from L2 or the 256 MB
    # last-level cache.
    def per_step(n, flush=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        sink = torch.empty((), dtype=torch.float32, device=dev)
        for a, b in ev:
            if flush is not None:
                torch.sum(flush, dim=0, out=sink)
            a.record()
            moe.forward(*fwd_args, out=out, routing=routing, workspace=ws)
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        return {"p10": round(float(np.percentile(t, 10)), 4), "p50": round(float(np.median(t)), 4),
                "p90": round(float(np.percentile(t, 90)), 4)}
    step_dist = {"warm_ms": per_step(max(args.steps, 20))}
    if shape.T * shape.top_k <= 4096:            # decode-sized: weight streaming
        scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        step_dist["cold_ms"] = per_step(max(args.steps, 20), flush=scratch)
        del scratch

    # Engine clock while the layer runs (clocks are not locked): enqueue about 0.3 s of
    # steps, then read the current sysfs level until they finish.
    n_busy = int(min(4000, max(20, 300.0 / ms_step)))
    done = torch.cuda.Event()
    for _ in range(n_busy):
        moe.forward(*fwd_args, out=out, routing=routing, workspace=ws)
    done.record()
    busy = []
    while not done.query():
        v = current_mhz(sysdir, "pp_dpm_sclk")
        if v is None:
            break
        busy.append(v)
        time.sleep(0.002)
    torch.cuda.synchronize()
    if busy:
        clocks["sclk_mhz_busy"] = {"p10": float(np.percentile(busy, 10)),
                                   "p50": float(np.median(busy)),
                                   "p90": float(np.percentile(busy, 90)), "samples": len(busy)}
    clocks["sclk_mhz_after"] = current_mhz(sysdir, "pp_dpm_sclk")
    clocks["mclk_mhz_after"] = current_mhz(sysdir, "pp_dpm_mclk")
    clocks["locked"] = False
    copy_gbs = device_copy_gbs(torch, dev)

    counts = routing["expert_counts"].cpu().numpy()
    alg = algorithmic(shape, counts, args.format)
    step_s = ms_step / 1e3
    tflops = alg["layer_flops"] / step_s / 1e12
    gbs = alg["layer_bytes"] / step_s / 1e9

    roof = roofline(alg[dom], dom_ms / 1e3, shape, args.format, dom)

    line = {
        "metric": METRIC, "value": round(shape.T / step_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"block": "fp8-e4m3", "mxfp8": "mxfp8-e4m3",
                  "mxfp4": "mxfp4-e2m1 x mxfp8-e4m3"}[args.format],
        "data": "synthetic",
        "config": {"workload": shape.name, "T": shape.T, "H": shape.H, "E": shape.E,
                   "top_k": shape.top_k, "I": shape.I, "parallelism": "single-gpu",
                   "weights": {"block": "fp8 128x128 block scales", "mxfp8": "mxfp8 1x32 E8M0 scales",
                               "mxfp4": "mxfp4 (e2m1) 1x32 E8M0 scales"}[args.format]},
        "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_FP8_TFLOPS, 4),
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "active_experts": alg["active_experts"],
        "expert_rows": {"min": int(counts.min()), "max": int(counts.max()),
                        "mean": round(float(counts.mean()), 2), "idle": int((counts == 0).sum())},
        "margin_redraws": int(li.redraws),
        "device_copy_gbs": round(copy_gbs, 1),
        "clocks": clocks,
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "step_ms_dist": step_dist,
        "roofline": roof,
        "decode_layers": None,
        "cpu_baseline": None,
    }
    if not args.no_decode_layers and shape.T * shape.top_k > 4096:
        del layer, ws, x, out
        torch.cuda.empty_cache()
        line["decode_layers"] = {n: decode_layer(SHAPES[n], args.format, dev)
                                 for n in ("gpt-oss-20b-decode", "qwen3-235b-decode")}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(shape, li, args.format)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

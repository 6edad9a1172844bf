#!/usr/bin/env python3
"""Benchmark of the DISCO sparse-contraction hot path on one MI355X.

One step = one pass of the whole hot path at 721x1440:
  * forward CSR contraction   x (1,64,721,1440) bf16 -> out (1,64,8,361,720) bf16  (K=8, 4 radial x 2 azimuthal, 3 deg)
  * backward (row-inverted)   gout (1,64,8,361,720) bf16 -> gx (1,64,721,1440) bf16 (same psi)
  * fused convolution         x (2,256,721,1440) bf16, W (256,256,16) -> y (2,256,721,1440) bf16 (K=16, 2 deg, p=1)
All three run on the bf16 matrix cores (fp32 accumulation).
Inputs are seeded synthetic tensors already resident in device memory; the psi
plans are built once before timing.  `value` is nnz-updates per second over the
whole step (one update = one fp32 multiply-add val*x for one (b, c, output
position)).  Per-op times come from HIP events recorded on the launch stream.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0


def op_bytes(op, w, nnz, Co=0):
    """Algorithmic bytes of one launch: inputs + outputs once, psi at 8 B/nnz plus row pointers."""
    esz = 2 if w.dtype == "bf16" else 4
    x = w.B * w.C * w.Hi * w.Wi * esz
    o = w.B * w.C * w.K * w.Ho * w.Wo * esz
    psi = 8 * nnz + 4 * (w.K * w.Ho + 1)
    if op in ("fwd", "bwd"):
        return x + o + psi
    y = w.B * Co * w.Ho * w.Wo * esz
    return x + Co * w.C * w.K * esz + y + psi


def op_updates(w, nnz):
    return w.B * w.C * w.Wo * nnz


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ops", default="fwd,bwd,fused", help="subset of ops in the step (profiling runs)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the separate timing of the fused-convolution backward")
    ap.add_argument("--no-einsum", action="store_true",
                    help="skip the timing of the fused op's einsum alone")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_gather_contraction_amd as sgc
    from disco_inputs import WORKLOADS, workload_gout, workload_psi, workload_weight, workload_x

    ops = [o for o in args.ops.split(",") if o]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wf = WORKLOADS["fwd_bf16_721x1440"]
    wb = WORKLOADS["bwd_bf16_721x1440"]
    wu = WORKLOADS["fused_bf16_721x1440"]
    t0 = time.time()
    psi_fb = workload_psi(wf)
    psi_u = workload_psi(wu)
    h_fb = sgc.disco_psi_create(psi_fb, 0)
    h_u = sgc.disco_psi_create(psi_u, 0)
    print(f"[bench] psi built and uploaded in {time.time() - t0:.1f}s (nnz {psi_fb.nnz}, {psi_u.nnz})",
          file=sys.stderr, flush=True)

    tensors = {}
    if "fwd" in ops:
        tensors["x3"] = workload_x(wf).to(dev)
        tensors["out3"] = torch.empty((wf.B, wf.C, wf.K, wf.Ho, wf.Wo), dtype=torch.bfloat16, device=dev)
    if "bwd" in ops:
        tensors["g4"] = workload_gout(wb).to(dev)
        tensors["gx4"] = torch.empty((wb.B, wb.C, wb.Hi, wb.Wi), dtype=torch.bfloat16, device=dev)
    if "fused" in ops:
        tensors["x5"] = workload_x(wu).to(dev)
        tensors["W5"] = workload_weight(wu).to(dev)
        tensors["y5"] = torch.empty((wu.B, wu.Co, wu.Ho, wu.Wo), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs resident after {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def run(op):
        if op == "fwd":
            sgc.disco_fwd(h_fb, tensors["x3"], tensors["out3"])
        elif op == "bwd":
            sgc.disco_bwd(h_fb, tensors["g4"], tensors["gx4"])
        else:
            sgc.disco_fused_conv(h_u, tensors["x5"], tensors["W5"], tensors["y5"])

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_calib_mib} MiB read + {args.copy_calib_mib} MiB written",
              file=sys.stderr, flush=True)
        del src, dst

    for i in range(args.warmup):
        for op in ops:
            run(op)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    ev = {op: [] for op in ops}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        for op in ops:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run(op)
            b.record(stream)
            ev[op].append((a, b))
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = 1e3 * t_total / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    per = {}
    cfg = {"fwd": (wf, psi_fb, 0), "bwd": (wb, psi_fb, 0), "fused": (wu, psi_u, wu.Co)}
    total_updates = 0
    total_bytes = 0
    for op in ops:
        w, psi, Co = cfg[op]
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[op]]))
        upd = op_updates(w, psi.nnz)
        byt = op_bytes(op, w, psi.nnz, Co)
        total_updates += upd
        total_bytes += byt
        d = {"ms": round(ms, 4), "GBps": round(byt / ms / 1e6, 2), "Gnnz_updates_per_s": round(upd / ms / 1e6, 2),
             "hbm_frac": round(byt / ms / 1e6 / PEAK_HBM_GBS, 5),
             "shape": {"B": w.B, "C": w.C, "K": w.K, "in": [w.Hi, w.Wi], "out": [w.Ho, w.Wo], "nnz": psi.nnz}}
        # every op of the step runs on bf16 matrix cores (psi packed into dense 16-offset blocks);
        # algorithmic flops: 2 per nnz-update, plus 2 per einsum MAC for the fused op
        alg = 2 * upd
        if op == "fused":
            macs = w.B * w.Ho * w.Wo * Co * w.C * w.K
            alg += 2 * macs
            d["einsum_macs"] = macs
            d["shape"]["Co"] = Co
        d["bound"] = "mfma"
        d["mfma_tflops_algorithmic"] = round(alg / ms / 1e9, 3)
        d["mfma_frac"] = round(alg / ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4)
        per[op] = d

    dom = max(per, key=lambda o: per[o]["ms"])
    traffic = counter_traffic(dom)
    dd = per[dom]
    roofline = {"bound": "mfma", "achieved": dd["mfma_tflops_algorithmic"], "peak": PEAK_BF16_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": dd["mfma_frac"], "traffic": traffic, "kernel": dom,
                "note": "algorithmic flops: 2 per nnz-update + 2 per einsum MAC; dense bf16 MFMA peak"}

    nxt = None
    if not args.no_next_rows and "fused" in ops:
        nxt = {"fused_bwd": time_fused_bwd(sgc, torch, np, h_u, tensors, wu, psi_u, dev, stream)}
        nxt["fused_saved"] = time_fused_saved(sgc, torch, np, h_u, tensors, wu, dev, stream)
        nxt["fused_saved"]["recompute_step_ms"] = round(per["fused"]["ms"] + nxt["fused_bwd"]["ms"], 4)
        nxt["f16"] = time_f16(sgc, torch, np, h_fb, h_u, wf, wb, wu, psi_fb, psi_u, dev, stream)
        nxt["page_shapes"] = time_page_shapes(sgc, torch, np, dev, stream)

    ein = None
    if not args.no_einsum and "fused" in ops:
        ein = time_einsum(sgc, torch, np, wu, tensors, dev, stream)
    ach = None if args.no_einsum else achievable_copy(torch, np, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wf, wb, wu, psi_fb, psi_u)

    line = {
        "metric": "DISCO fwd+bwd GB/s & Gnnz-updates/s at 721x1440; % HBM/MFMA roofline",
        "value": round(total_updates / (ms_step * 1e6), 3),
        "unit": "Gnnz-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in/out, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) tensors, equiangular-grid hat-basis psi)",
        "config": {"workload": "disco_721x1440: fwd (1,64,721x1440->361x720,K=8) + bwd (same) + "
                               "fused (2,256->256,721x1440,K=16)", "ops": ops,
                   "GBps_step": round(total_bytes / (ms_step * 1e6), 2)},
        "per_op": per,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "einsum_standalone": ein,
        "achievable": ach,
        "next_rows": nxt,
    }
    print(json.dumps(line), flush=True)


KERNEL_SOURCES = {"fused": "kernels_fused_mfma.hip", "einsum": "kernels_fused_mfma.hip"}


def counter_traffic(op):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the committed counter summary,
    or None when that summary was taken from a different kernel source than the one built here."""
    import hashlib
    import re

    name = KERNEL_SOURCES.get(op)
    summary = os.path.join(ROOT, "profiles", "disco_step_721x1440_hbm_counters.md")
    if name is None or not os.path.exists(summary):
        return None
    with open(os.path.join(ROOT, "sparse_gather_contraction_amd", "csrc", name), "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    with open(summary) as f:
        for line in f:
            m = re.match(r"traffic-record: (\{.*\})", line.strip())
            if m:
                rec = json.loads(m.group(1))
                if rec.get("kernel") == op and rec.get("source_sha256") == digest:
                    return int(rec["read_bytes"] + rec["write_bytes"])
    return None



def time_einsum(sgc, torch, np, w, tensors, dev, stream, warm=2, reps=10):
    """The fused op's einsum alone at its GEMM shape (M = Co = 256, K = C*K = 4096, N = B*Ho*Wo =
    2,076,480): disco_einsum on the fused kernel's matrix-core einsum tile, with the contraction
    t (B, C, K, Ho, Wo) staged in device memory as bf16 (a seeded device draw, 17 GB: far beyond
    the caches, so every tile comes from HBM).  Timed apart from the step (not part of `value`)."""
    from disco_inputs import randn_device

    t = randn_device((w.B, w.C, w.K, w.Ho, w.Wo), 3500, "bf16", dev)
    W = tensors["W5"]
    y = torch.empty((w.B, w.Co, w.Ho, w.Wo), dtype=torch.bfloat16, device=dev)
    for _ in range(warm):
        sgc.disco_einsum(W, t, y)
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sgc.disco_einsum(W, t, y)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    macs = w.B * w.Ho * w.Wo * w.Co * w.C * w.K
    byt = 2 * (t.numel() + W.numel() + y.numel())
    del t, y
    torch.cuda.empty_cache()
    res = {"ms": round(ms, 4), "macs": macs, "bound": "mfma",
           "mfma_tflops": round(2 * macs / ms / 1e9, 3),
           "mfma_frac": round(2 * macs / ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4),
           "bytes": byt, "GBps": round(byt / ms / 1e6, 2), "hbm_frac": round(byt / ms / 1e6 / PEAK_HBM_GBS, 4),
           "gemm_mkn": [w.Co, w.C * w.K, w.B * w.Ho * w.Wo], "traffic": counter_traffic("einsum"),
           "operand": "bf16 contraction (2,256,16,721,1440) in HBM, W (256,256,16), y (2,256,721,1440)"}
    print(f"[bench] einsum alone: {ms:.3f} ms ({res['mfma_tflops']} TFLOP/s, {res['GBps']} GB/s)",
          file=sys.stderr, flush=True)
    return res


def achievable_copy(torch, np, dev, stream, mib=1024, reps=5, read_gib=4):
    """What plain streaming reaches on this machine, beside the 8 TB/s spec peak: torch's device copy of
    `mib` MiB (read + write) and torch's sum over `read_gib` GiB of bf16 (read only), median of
    `reps` each, HIP events on the launch stream."""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_gbs = 2 * mib * (1 << 20) / timed(lambda: dst.copy_(src)) / 1e6
    del src, dst
    x = torch.ones(read_gib * (1 << 30) // 2, dtype=torch.bfloat16, device=dev)
    read_gbs = read_gib * (1 << 30) / timed(lambda: x.sum(dtype=torch.float32)) / 1e6
    del x
    torch.cuda.empty_cache()
    return {"copy_GBps": round(copy_gbs, 1), "copy_frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
            "read_GBps": round(read_gbs, 1), "read_frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4),
            "note": f"device copy of {mib} MiB (read + write) and a bf16 sum over {read_gib} GiB (read only), "
                    f"median of {reps} each"}

def time_fused_bwd(sgc, torch, np, h, tensors, w, psi, dev, stream, warm=2, reps=3):
    """Backward of the fused convolution on the fused workload (gradient gy ~ N(0,1), bf16), timed
    apart from the step (it is not part of `value`).  Algorithmic flops: the two dense products
    (W^T gy and the weight gradient, 2 per MAC each) plus the transpose contraction and the
    forward contraction it recomputes for the weight gradient (2 per nnz-update each)."""
    from disco_inputs import randn

    gy = randn((w.B, w.Co, w.Ho, w.Wo), 3100, "bf16").to(dev)
    gx = torch.empty_like(tensors["x5"])
    dW = torch.empty_like(tensors["W5"])
    ws = torch.empty(sgc.disco_fused_conv_bwd_workspace(h, w.B, w.C, w.Co), dtype=torch.uint8, device=dev)
    for _ in range(warm):
        sgc.disco_fused_conv_bwd(h, tensors["x5"], tensors["W5"], gy, gx, dW, workspace=ws)
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sgc.disco_fused_conv_bwd(h, tensors["x5"], tensors["W5"], gy, gx, dW, workspace=ws)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    macs = w.B * w.Ho * w.Wo * w.Co * w.C * w.K
    upd = op_updates(w, psi.nnz)
    alg = 4 * macs + 4 * upd
    print(f"[bench] fused backward: {ms:.3f} ms", file=sys.stderr, flush=True)
    return {"ms": round(ms, 4), "einsum_macs_x2": 2 * macs, "nnz_updates_x2": 2 * upd, "bound": "mfma",
            "mfma_tflops_algorithmic": round(alg / ms / 1e9, 3),
            "mfma_frac": round(alg / ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4),
            "workspace_bytes": int(ws.numel()),
            "shape": {"B": w.B, "C": w.C, "Co": w.Co, "K": w.K, "in": [w.Hi, w.Wi], "out": [w.Ho, w.Wo]}}



def time_fused_saved(sgc, torch, np, h, tensors, w, dev, stream, warm=2, reps=3):
    """A training step of the fused convolution that keeps its contraction: disco_fused_conv_save
    (y and out = F x, 17 GB of bf16 written) then disco_fused_conv_bwd_saved (no recompute of F x),
    timed apart from the step; compare `recompute_step_ms` (fused op + the recomputing backward)."""
    from disco_inputs import randn

    gy = randn((w.B, w.Co, w.Ho, w.Wo), 3100, "bf16").to(dev)
    x, W = tensors["x5"], tensors["W5"]
    y = torch.empty((w.B, w.Co, w.Ho, w.Wo), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w.B, w.C, w.K, w.Ho, w.Wo), dtype=torch.bfloat16, device=dev)
    gx = torch.empty_like(x)
    dW = torch.empty_like(W)
    ws = torch.empty(sgc.disco_fused_conv_bwd_workspace(h, w.B, w.C, w.Co), dtype=torch.uint8, device=dev)
    fns = {"fwd_save": lambda: sgc.disco_fused_conv_save(h, x, W, y, out),
           "bwd_saved": lambda: sgc.disco_fused_conv_bwd_saved(h, out, W, gy, gx, dW, workspace=ws)}
    res = {}
    for name, fn in fns.items():
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        res[name + "_ms"] = round(float(np.mean([a.elapsed_time(b) for a, b in ev])), 4)
    res["step_ms"] = round(res["fwd_save_ms"] + res["bwd_saved_ms"], 4)
    del out, ws
    torch.cuda.empty_cache()
    print(f"[bench] fused training step keeping the contraction: {res}", file=sys.stderr, flush=True)
    return res

def time_f16(sgc, torch, np, h_fb, h_u, wf, wb, wu, psi_fb, psi_u, dev, stream, warm=1, reps=3):
    """The three ops of the step with fp16 data (same shapes and psi), timed apart from the step;
    all three run on the fp16 matrix cores (psi as fp16 of psi * 2^e)."""
    from disco_inputs import randn

    x3 = randn((wf.B, wf.C, wf.Hi, wf.Wi), 3200, "f16").to(dev)
    g4 = randn((wb.B, wb.C, wb.K, wb.Ho, wb.Wo), 3201, "f16").to(dev)
    x5 = randn((wu.B, wu.C, wu.Hi, wu.Wi), 3202, "f16").to(dev)
    W5 = randn((wu.Co, wu.C, wu.K), 3203, "f16", std=1.0 / math.sqrt(wu.C * wu.K)).to(dev)
    calls = {"fwd": lambda: sgc.disco_fwd(h_fb, x3), "bwd": lambda: sgc.disco_bwd(h_fb, g4),
             "fused": lambda: sgc.disco_fused_conv(h_u, x5, W5)}
    res = {}
    for op, fn in calls.items():
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        w, psi = {"fwd": (wf, psi_fb), "bwd": (wb, psi_fb), "fused": (wu, psi_u)}[op]
        upd = op_updates(w, psi.nnz)
        res[op] = {"ms": round(ms, 4), "Gnnz_updates_per_s": round(upd / ms / 1e6, 2)}
    print(f"[bench] fp16: {res}", file=sys.stderr, flush=True)
    return res


def time_page_shapes(sgc, torch, np, dev, stream, reps=3):
    """The DISCO page's own benchmark shapes (section "Serial Benchmarks": Gauss-Legendre grids,
    theta_c = 0.017, K = 9 stand-in basis, batch 1), bf16: fused convolution and its backward."""
    from disco_inputs import WORKLOADS, randn, workload_psi, workload_weight, workload_x

    res = {}
    for name in ("page_self_256x360x720", "page_self_512x360x720", "page_down_80x721x1440"):
        w = WORKLOADS[name]
        psi = workload_psi(w)
        h = sgc.disco_psi_create(psi, 0)
        x = workload_x(w).to(dev)
        W = workload_weight(w).to(dev)
        gy = randn((w.B, w.Co, w.Ho, w.Wo), 3300 + w.index, "bf16").to(dev)
        y = torch.empty((w.B, w.Co, w.Ho, w.Wo), dtype=torch.bfloat16, device=dev)
        gx = torch.empty_like(x)
        dW = torch.empty_like(W)
        ws = torch.empty(max(1, sgc.disco_fused_conv_bwd_workspace(h, w.B, w.C, w.Co)), dtype=torch.uint8, device=dev)
        fns = {"fused": lambda: sgc.disco_fused_conv(h, x, W, y),
               "fused_bwd": lambda: sgc.disco_fused_conv_bwd(h, x, W, gy, gx, dW, workspace=ws)}
        upd = op_updates(w, psi.nnz)
        macs = w.B * w.Ho * w.Wo * w.Co * w.C * w.K
        r = {"shape": {"B": w.B, "C": w.C, "Co": w.Co, "K": w.K, "in": [w.Hi, w.Wi], "out": [w.Ho, w.Wo],
                       "nnz": psi.nnz, "grids": [w.grid_in, w.grid_out]}}
        for op, fn in fns.items():
            fn()
            torch.cuda.synchronize()
            ev = []
            for _ in range(reps):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                ev.append((a, b))
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            alg = (2 * upd + 2 * macs) * (2 if op == "fused_bwd" else 1)
            r[op] = {"ms": round(ms, 4), "mfma_tflops_algorithmic": round(alg / ms / 1e9, 3),
                     "mfma_frac": round(alg / ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4)}
        res[name] = r
        h.close()
        del x, W, gy, y, gx, dW, ws
    print(f"[bench] page shapes: { {k: (v['fused']['ms'], v['fused_bwd']['ms']) for k, v in res.items()} }",
          file=sys.stderr, flush=True)
    return res


def cpu_baseline(wf, wb, wu, psi_fb, psi_u):
    """The fp64 oracle on a bounded sample of the same workload (host cores)."""
    import oracle
    from disco_inputs import workload_gout, workload_weight, workload_x

    planes = 24
    x = workload_x(wf)[0, :planes]
    g = workload_gout(wb)[0, :planes]
    t = time.perf_counter()
    oracle.fwd(psi_fb, x)
    oracle.bwd(psi_fb, g)
    t_fb = time.perf_counter() - t
    upd = 2 * planes * wf.Wo * psi_fb.nnz
    x5 = workload_x(wu)[:1]
    W5 = workload_weight(wu)
    hos = [0, 45, 90, 180, 270, 360, 540, 700]  # pole to equator and on
    t = time.perf_counter()
    oracle.fused(psi_u, x5, W5, ho_list=hos)
    t_u = time.perf_counter() - t
    r0 = psi_u.row_ptr
    nnz_ho = sum(int(r0[k * wu.Ho + h + 1] - r0[k * wu.Ho + h]) for k in range(wu.K) for h in hos)
    upd_u = wu.C * wu.Wo * nnz_ho
    total = upd + upd_u
    return {"value": round(total / (t_fb + t_u) / 1e9, 4), "unit": "Gnnz-updates/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fwd+bwd on {planes}/64 channel planes of the 721x1440 K=8 workload "
                      f"({t_fb:.1f}s) + fused contraction and einsum for latitudes {hos} of batch 0 of the "
                      f"K=16 workload ({t_u:.1f}s); updates counted as in value",
            "seconds": round(t_fb + t_u, 2)}


if __name__ == "__main__":
    main()

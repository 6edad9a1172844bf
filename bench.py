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
CLOCK_HZ = 2.4e9  # peak engine clock (LDS bytes per clock are reported at it)
# Published vector fp32 figure: 256 CUs x 4 SIMDs x 32 fp32 FMA per clock x 2 flops x 2.4 GHz.  The
# library is built with packed fp32 ops disabled; the FMA-loop probe (plain v_fma_f32, no packed math)
# reaches 112.7 TFLOP/s on the box, above what 16 lanes per SIMD per clock could give (78.6), so the
# published figure is the vector-ALU roof of this code too.
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_FP32_FMA_TFLOPS = PEAK_FP32_VALU_TFLOPS
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_F16_MFMA_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3  # dense fp32 matrix peak (v_mfma_f32_16x16x4_f32)


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
    ap.add_argument("--no-fp32-configs", action="store_true",
                    help="skip the fp32 16x32 and 181x360 configurations")
    ap.add_argument("--fp32-only", action="store_true",
                    help="time only the fp32 configurations (profiling runs of their kernels)")
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
    if args.fp32_only:
        stream = torch.cuda.current_stream(dev)
        print(json.dumps({"fp32_configs": time_fp32_configs(sgc, torch, np, dev, stream)}), flush=True)
        return
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
        times = np.array([a.elapsed_time(b) for a, b in ev[op]])
        ms = float(np.mean(times))
        upd = op_updates(w, psi.nnz)
        byt = op_bytes(op, w, psi.nnz, Co)
        total_updates += upd
        total_bytes += byt
        d = {"ms": round(ms, 4), "ms_median": round(float(np.median(times)), 4),
             "ms_p10": round(float(np.percentile(times, 10)), 4), "ms_p90": round(float(np.percentile(times, 90)), 4),
             "GBps": round(byt / ms / 1e6, 2), "Gnnz_updates_per_s": round(upd / ms / 1e6, 2),
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
        nxt["fp32_fused"] = time_fp32_fused(sgc, torch, np, dev, stream)
        nxt["page_shapes"] = time_page_shapes(sgc, torch, np, dev, stream)
        nxt["valu_gathers_bf16"] = time_valu_gathers(sgc, torch, np, h_fb, tensors, wf, wb, psi_fb, dev, stream)

    ein = None
    if not args.no_einsum and "fused" in ops:
        ein = time_einsum(sgc, torch, np, wu, tensors, dev, stream)
    fp32 = None if args.no_fp32_configs else time_fp32_configs(sgc, torch, np, dev, stream)
    ach = None if args.no_einsum else achievable(torch, np, dev, stream)

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
        "fp32_configs": fp32,
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
    # the same GEMM through the ROCm BLAS library behind torch.matmul (a reference point for this
    # shape: bf16 in and out, one product per batch, contiguous operands)
    W2 = W.reshape(w.Co, w.C * w.K)
    tb = [t[b].reshape(w.C * w.K, w.Ho * w.Wo) for b in range(w.B)]
    yb = [y[b].reshape(w.Co, w.Ho * w.Wo) for b in range(w.B)]

    def lib_gemm():
        for b in range(w.B):
            torch.matmul(W2, tb[b], out=yb[b])

    lib_ms, lib_p10, lib_p90 = _timed(torch, np, stream, lib_gemm, 5)
    del tb, yb
    macs = w.B * w.Ho * w.Wo * w.Co * w.C * w.K
    byt = 2 * (t.numel() + W.numel() + y.numel())
    del t, y
    torch.cuda.empty_cache()
    res = {"ms": round(ms, 4), "macs": macs, "bound": "mfma",
           "mfma_tflops": round(2 * macs / ms / 1e9, 3),
           "mfma_frac": round(2 * macs / ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4),
           "bytes": byt, "GBps": round(byt / ms / 1e6, 2), "hbm_frac": round(byt / ms / 1e6 / PEAK_HBM_GBS, 4),
           "gemm_mkn": [w.Co, w.C * w.K, w.B * w.Ho * w.Wo], "traffic": counter_traffic("einsum"),
           "operand": "bf16 contraction (2,256,16,721,1440) in HBM, W (256,256,16), y (2,256,721,1440)",
           "library_gemm": {"ms_median": round(lib_ms, 4), "ms_p10_p90": [round(lib_p10, 4), round(lib_p90, 4)],
                            "mfma_frac": round(2 * macs / lib_ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4),
                            "what": "torch.matmul (ROCm BLAS) on the same GEMM, one product per batch, bf16 in/out"}}
    print(f"[bench] einsum alone: {ms:.3f} ms ({res['mfma_tflops']} TFLOP/s, {res['GBps']} GB/s); "
          f"library GEMM {lib_ms:.3f} ms",
          file=sys.stderr, flush=True)
    return res


def _timed(torch, np, stream, fn, reps):
    """Median and spread of `reps` calls of fn (one untimed call first), HIP events on `stream`."""
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
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def achievable(torch, np, dev, stream, read_gib=4, copy_mib=1024, reps=5):
    """What this machine reaches beside the published peaks, measured with microbenchmark kernels built
    here (sparse_gather_contraction_amd/csrc/probes.hip): a read-only stream over `read_gib` GiB with
    16-byte loads, a copy of `copy_mib` MiB (read + write), an fp32 FMA loop (no packed math, as in the
    library) and a bf16 MFMA loop (v_mfma_f32_32x32x16_bf16); medians of `reps` each."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_gather_contraction_amd", "libdisco_probes.so"))
    for f in ("disco_probe_read", "disco_probe_copy", "disco_probe_fma", "disco_probe_mfma", "disco_probe_lds",
              "disco_probe_lds_mfma", "disco_probe_dma_read"):
        getattr(lib, f).restype = ctypes.c_int
    P, S = ctypes.c_void_p, ctypes.c_size_t
    lib.disco_probe_dma_read.argtypes = [P, S, ctypes.c_int, ctypes.c_int, P]
    lib.disco_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P]
    lib.disco_probe_lds_mfma.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P]
    lib.disco_probe_read.argtypes = [P, S, P, ctypes.c_int, P]
    lib.disco_probe_copy.argtypes = [P, P, S, ctypes.c_int, P]
    lib.disco_probe_fma.argtypes = [ctypes.c_int, P, ctypes.c_int, P]
    lib.disco_probe_mfma.argtypes = [ctypes.c_int, P, ctypes.c_int, P]
    sp = stream.cuda_stream

    def ok(st):
        if st != 0:
            raise RuntimeError(f"probe launch failed with HIP status {st}")

    blocks = 256 * 8
    out = torch.zeros(blocks * 256, dtype=torch.float32, device=dev)
    buf = torch.ones(read_gib * (1 << 30) // 4, dtype=torch.float32, device=dev)
    nb = buf.numel() * 4
    ms_r = _timed(torch, np, stream, lambda: ok(lib.disco_probe_read(buf.data_ptr(), nb, out.data_ptr(), blocks, sp)),
                  reps)
    # the direct global -> LDS path (the library's stage loads): 3 GiB, one 4-wave workgroup per CU,
    # four 1 KiB loads in flight per wave
    nd = min(nb, 3 << 30)
    ms_d = _timed(torch, np, stream, lambda: ok(lib.disco_probe_dma_read(buf.data_ptr(), nd, 4, 256, sp)), reps)
    del buf
    src = torch.ones(copy_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms_c = _timed(torch, np, stream, lambda: ok(lib.disco_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel() * 4,
                                                                     blocks, sp)), reps)
    del src, dst
    iters = 4096
    ms_f = _timed(torch, np, stream, lambda: ok(lib.disco_probe_fma(iters, out.data_ptr(), blocks, sp)), reps)
    miters = 2048
    ms_m = _timed(torch, np, stream, lambda: ok(lib.disco_probe_mfma(miters, out.data_ptr(), blocks, sp)), reps)
    # LDS: 16- and 4-byte reads (512 threads, 8 reads per iteration), and the contraction's LDS-fed
    # MFMA pattern (two 16-byte x runs + four or five 4-byte psi words per two MFMAs)
    lblocks, liters = 1024, 4096
    lout = torch.zeros(lblocks * 512, dtype=torch.float32, device=dev)
    lds_ms = {w: _timed(torch, np, stream, lambda w=w: ok(lib.disco_probe_lds(liters, w, lout.data_ptr(), lblocks, sp)),
                        reps)[0] for w in (4, 16)}
    lm_iters = 8192
    lm_ms = {nb: _timed(torch, np, stream,
                        lambda nb=nb: ok(lib.disco_probe_lds_mfma(lm_iters, nb, lout.data_ptr(), lblocks, sp)), reps)[0]
             for nb in (4, 5)}
    del lout
    torch.cuda.empty_cache()
    read_gbs = nb / ms_r[0] / 1e6
    copy_gbs = 2 * copy_mib * (1 << 20) / ms_c[0] / 1e6
    fma_tf = blocks * 256 * iters * 8 * 2 / ms_f[0] / 1e9
    mfma_tf = blocks * 4 * miters * 4 * (32 * 32 * 16 * 2) / ms_m[0] / 1e9
    dma_gbs = nd / ms_d[0] / 1e6
    res = {"read_GBps": round(read_gbs, 1), "read_frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4),
           "lds_dma_read_GBps": round(dma_gbs, 1), "lds_dma_read_frac_of_peak": round(dma_gbs / PEAK_HBM_GBS, 4),
           "copy_GBps": round(copy_gbs, 1), "copy_frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
           "fp32_fma_TFLOPs": round(fma_tf, 2), "fp32_fma_frac_of_peak": round(fma_tf / PEAK_FP32_VALU_TFLOPS, 4),
           "bf16_mfma_TFLOPs": round(mfma_tf, 1), "bf16_mfma_frac_of_peak": round(mfma_tf / PEAK_BF16_MFMA_TFLOPS, 4),
           "lds_b128_bytes_per_clk_per_cu": round(lblocks * 512 * liters * 8 * 16 / lds_ms[16] / 1e-3 / 256 / CLOCK_HZ, 1),
           "lds_b32_bytes_per_clk_per_cu": round(lblocks * 512 * liters * 8 * 4 / lds_ms[4] / 1e-3 / 256 / CLOCK_HZ, 1),
           "lds_fed_mfma_TFLOPs": {f"{nb}_psi_words": round(lblocks * 8 * lm_iters * 2 * 32768 / lm_ms[nb] / 1e9, 1)
                                   for nb in (4, 5)},
           "note": f"HIP probes built here: read stream of {read_gib} GiB (16-byte loads), copy of {copy_mib} MiB "
                   f"(read + write), a 3 GiB stream of direct global-to-LDS loads, fp32 FMA loop, bf16 MFMA loop, LDS "
                   f"read loops (bytes per clock per CU at "
                   f"{CLOCK_HZ / 1e9} GHz), the contraction's LDS-fed MFMA loop; medians of {reps}"}
    print(f"[bench] achievable: {res}", file=sys.stderr, flush=True)
    return res


def time_fp32_configs(sgc, torch, np, dev, stream, warm=10, reps=60):
    """The two fp32 configurations: the tiny 16x32 forward (launch-latency bound) and the 181x360 ->
    91x180 forward and backward.  Each timed call reads and writes a different set of buffers, eight
    sets in rotation for 181x360 (8 x 67 MB > 512 MiB: beyond the 256 MiB last-level cache, so the
    bytes come from HBM); medians and spread of `reps` calls after `warm`.  Roofline: one fp32 FMA per
    nnz-update on the vector ALU (2 flops) against 16 flops per algorithmic byte: the ALU floor (6.8 us
    at 157.3 TFLOP/s) lies below the HBM floor (8.4 us at 8 TB/s), so the bound is HBM."""
    from disco_inputs import WORKLOADS, workload_gout, workload_psi, workload_x

    res = {}
    for name, nrot in (("tiny_fwd_f32_16x32", 1), ("fwdbwd_f32_181x360", 8)):
        w = WORKLOADS[name]
        psi = workload_psi(w)
        h = sgc.disco_psi_create(psi, 0)
        xs = [workload_x(w).to(dev) for _ in range(nrot)]
        outs = [torch.empty((w.B, w.C, w.K, w.Ho, w.Wo), dtype=torch.float32, device=dev) for _ in range(nrot)]
        calls = {"fwd": [lambda i=i: sgc.disco_fwd(h, xs[i], outs[i]) for i in range(nrot)]}
        if "bwd" in w.ops:
            gs = [workload_gout(w).to(dev) for _ in range(nrot)]
            gxs = [torch.empty((w.B, w.C, w.Hi, w.Wi), dtype=torch.float32, device=dev) for _ in range(nrot)]
            calls["bwd"] = [lambda i=i: sgc.disco_bwd(h, gs[i], gxs[i]) for i in range(nrot)]
        upd = op_updates(w, psi.nnz)
        for op, fns in calls.items():
            for i in range(warm):
                fns[i % nrot]()
            torch.cuda.synchronize()
            ev = []
            for i in range(reps):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fns[i % nrot]()
                b.record(stream)
                ev.append((a, b))
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) for a, b in ev])
            ms = float(np.median(t))
            byt = op_bytes(op, w, psi.nnz)
            tf = 2 * upd / ms / 1e9
            res[f"{name}:{op}"] = {
                "ms_median": round(ms, 5), "ms_p10": round(float(np.percentile(t, 10)), 5),
                "ms_p90": round(float(np.percentile(t, 90)), 5), "calls": reps, "buffer_sets": nrot,
                "bytes": byt, "updates": upd, "GBps": round(byt / ms / 1e6, 2),
                "Gnnz_updates_per_s": round(upd / ms / 1e6, 2), "hbm_frac": round(byt / ms / 1e6 / PEAK_HBM_GBS, 5),
                "bound": ("launch latency" if name == "tiny_fwd_f32_16x32" else
                          ("hbm" if byt / PEAK_HBM_GBS >= 2 * upd / PEAK_FP32_FMA_TFLOPS / 1e3 else "alu")),
                "valu_tflops": round(tf, 3), "valu_frac": round(tf / PEAK_FP32_FMA_TFLOPS, 4),
                "hbm_floor_us": round(byt / PEAK_HBM_GBS / 1e3, 2),
                "alu_floor_us": round(2 * upd / PEAK_FP32_FMA_TFLOPS / 1e6, 2),
                "shape": {"B": w.B, "C": w.C, "K": w.K, "in": [w.Hi, w.Wi], "out": [w.Ho, w.Wo], "nnz": psi.nnz}}
        h.close()
        del xs, outs
        torch.cuda.empty_cache()
    print(f"[bench] fp32 configs: { {k: v['ms_median'] for k, v in res.items()} }", file=sys.stderr, flush=True)
    return res

def time_fused_bwd(sgc, torch, np, h, tensors, w, psi, dev, stream, warm=2, reps=5):
    """Backward of the fused convolution on the fused workload (gradient gy ~ N(0,1), bf16), timed
    apart from the step (it is not part of `value`).  Algorithmic flops: the two dense products
    (W^T gy and the weight gradient, 2 per MAC each) plus the transpose contraction and the
    forward contraction it recomputes for the weight gradient (2 per nnz-update each)."""
    from disco_inputs import randn

    gy = randn((w.B, w.Co, w.Ho, w.Wo), 3100, "bf16").to(dev)
    gx = torch.empty_like(tensors["x5"])
    dW = torch.empty_like(tensors["W5"])
    ws = torch.empty(sgc.disco_fused_conv_bwd_workspace(h, w.B, w.C, w.Co), dtype=torch.uint8, device=dev)
    for _ in range(warm - 1):
        sgc.disco_fused_conv_bwd(h, tensors["x5"], tensors["W5"], gy, gx, dW, workspace=ws)
    ms, p10, p90 = _timed(torch, np, stream,
                          lambda: sgc.disco_fused_conv_bwd(h, tensors["x5"], tensors["W5"], gy, gx, dW, workspace=ws), reps)
    macs = w.B * w.Ho * w.Wo * w.Co * w.C * w.K
    upd = op_updates(w, psi.nnz)
    alg = 4 * macs + 4 * upd
    print(f"[bench] fused backward: {ms:.3f} ms", file=sys.stderr, flush=True)
    return {"ms": round(ms, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
            "einsum_macs_x2": 2 * macs, "nnz_updates_x2": 2 * upd, "bound": "mfma",
            "mfma_tflops_algorithmic": round(alg / ms / 1e9, 3),
            "mfma_frac": round(alg / ms / 1e9 / PEAK_BF16_MFMA_TFLOPS, 4),
            "workspace_bytes": int(ws.numel()),
            "shape": {"B": w.B, "C": w.C, "Co": w.Co, "K": w.K, "in": [w.Hi, w.Wi], "out": [w.Ho, w.Wo]}}



def time_fused_saved(sgc, torch, np, h, tensors, w, dev, stream, warm=2, reps=5):
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
        for _ in range(warm - 1):
            fn()
        med, p10, p90 = _timed(torch, np, stream, fn, reps)
        res[name + "_ms"] = round(med, 4)
        res[name + "_ms_p10_p90"] = [round(p10, 4), round(p90, 4)]
    res["step_ms"] = round(res["fwd_save_ms"] + res["bwd_saved_ms"], 4)
    del out, ws
    torch.cuda.empty_cache()
    print(f"[bench] fused training step keeping the contraction: {res}", file=sys.stderr, flush=True)
    return res

def time_f16(sgc, torch, np, h_fb, h_u, wf, wb, wu, psi_fb, psi_u, dev, stream, reps=5):
    """The three ops of the step and the fused op's backward with fp16 data (same shapes and psi),
    timed apart from the step; all run on the fp16 matrix cores (psi as fp16 of psi * 2^e)."""
    from disco_inputs import randn

    x3 = randn((wf.B, wf.C, wf.Hi, wf.Wi), 3200, "f16").to(dev)
    g4 = randn((wb.B, wb.C, wb.K, wb.Ho, wb.Wo), 3201, "f16").to(dev)
    x5 = randn((wu.B, wu.C, wu.Hi, wu.Wi), 3202, "f16").to(dev)
    W5 = randn((wu.Co, wu.C, wu.K), 3203, "f16", std=1.0 / math.sqrt(wu.C * wu.K)).to(dev)
    gy5 = randn((wu.B, wu.Co, wu.Ho, wu.Wo), 3204, "f16", std=0.1).to(dev)
    gx5 = torch.empty_like(x5)
    dW5 = torch.empty_like(W5)
    ws = torch.empty(sgc.disco_fused_conv_bwd_workspace(h_u, wu.B, wu.C, wu.Co), dtype=torch.uint8, device=dev)
    calls = {"fwd": lambda: sgc.disco_fwd(h_fb, x3), "bwd": lambda: sgc.disco_bwd(h_fb, g4),
             "fused": lambda: sgc.disco_fused_conv(h_u, x5, W5),
             "fused_bwd": lambda: sgc.disco_fused_conv_bwd(h_u, x5, W5, gy5, gx5, dW5, workspace=ws)}
    res = {}
    for op, fn in calls.items():
        med, p10, p90 = _timed(torch, np, stream, fn, reps)
        w, psi = {"fwd": (wf, psi_fb), "bwd": (wb, psi_fb), "fused": (wu, psi_u), "fused_bwd": (wu, psi_u)}[op]
        upd = op_updates(w, psi.nnz) * (2 if op == "fused_bwd" else 1)
        r = {"ms_median": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
             "Gnnz_updates_per_s": round(upd / med / 1e6, 2)}
        if op in ("fused", "fused_bwd"):
            macs = w.B * w.Ho * w.Wo * wu.Co * w.C * w.K * (2 if op == "fused_bwd" else 1)
            alg = 2 * upd + 2 * macs
            r["mfma_tflops_algorithmic"] = round(alg / med / 1e9, 3)
            r["mfma_frac"] = round(alg / med / 1e9 / PEAK_F16_MFMA_TFLOPS, 4)
        res[op] = r
    del x3, g4, x5, W5, gy5, gx5, dW5, ws
    torch.cuda.empty_cache()
    print(f"[bench] fp16: {res}", file=sys.stderr, flush=True)
    return res


def time_fp32_fused(sgc, torch, np, dev, stream, reps=5):
    """The fused convolution in fp32 (fp32 contraction on the vector ALUs, einsum on
    v_mfma_f32_16x16x4_f32) beside the same op in bf16, at the page's 256-channel self-convolution
    shape: the page's "every precision against its fp32 variant" comparison."""
    from disco_inputs import WORKLOADS, randn, workload_psi

    w = WORKLOADS["page_self_256x360x720"]
    psi = workload_psi(w)
    h = sgc.disco_psi_create(psi, 0)
    res = {"shape": {"B": w.B, "C": w.C, "Co": w.Co, "K": w.K, "in": [w.Hi, w.Wi], "out": [w.Ho, w.Wo],
                     "nnz": psi.nnz}}
    upd = op_updates(w, psi.nnz)
    macs = w.B * w.Ho * w.Wo * w.Co * w.C * w.K
    for dt, peak in (("f32", PEAK_FP32_MFMA_TFLOPS), ("bf16", PEAK_BF16_MFMA_TFLOPS)):
        x = randn((w.B, w.C, w.Hi, w.Wi), 3400, dt).to(dev)
        W = randn((w.Co, w.C, w.K), 3401, dt, std=1.0 / math.sqrt(w.C * w.K)).to(dev)
        y = torch.empty((w.B, w.Co, w.Ho, w.Wo), dtype=x.dtype, device=dev)
        med, p10, p90 = _timed(torch, np, stream, lambda: sgc.disco_fused_conv(h, x, W, y), reps)
        alg = 2 * upd + 2 * macs
        res[dt] = {"ms_median": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                   "tflops_algorithmic": round(alg / med / 1e9, 3), "peak_TFLOPs": peak,
                   "frac": round(alg / med / 1e9 / peak, 4)}
        del x, W, y
    h.close()
    torch.cuda.empty_cache()
    res["note"] = "f32 against the fp32 matrix peak (the einsum's instruction), bf16 against the bf16 peak"
    print(f"[bench] fp32 fused: {res}", file=sys.stderr, flush=True)
    return res


def time_valu_gathers(sgc, torch, np, h_fb, tensors, wf, wb, psi_fb, dev, stream, reps=5):
    """The bf16 forward and backward at 721x1440 on the vector-ALU gathers (the matrix-core kernels
    switched off with their knobs for these calls only): the LDS-staged gather path that 16-bit
    data took before the matrix-core kernels, HBM-bound in design."""
    res = {}
    x3 = tensors.get("x3")
    g4 = tensors.get("g4")
    calls = {}
    if x3 is not None:
        calls["fwd"] = ("DISCO_FWD_MFMA", lambda: sgc.disco_fwd(h_fb, x3, tensors["out3"]), wf)
    if g4 is not None:
        calls["bwd"] = ("DISCO_BWD_MFMA", lambda: sgc.disco_bwd(h_fb, g4, tensors["gx4"]), wb)
    for op, (knob, fn, w) in calls.items():
        old = os.environ.get(knob)
        os.environ[knob] = "0"
        try:
            med, p10, p90 = _timed(torch, np, stream, fn, reps)
        finally:
            if old is None:
                del os.environ[knob]
            else:
                os.environ[knob] = old
        byt = op_bytes(op, w, psi_fb.nnz)
        upd = op_updates(w, psi_fb.nnz)
        res[op] = {"ms_median": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                   "GBps": round(byt / med / 1e6, 2), "hbm_frac": round(byt / med / 1e6 / PEAK_HBM_GBS, 4),
                   "Gnnz_updates_per_s": round(upd / med / 1e6, 2),
                   "valu_frac": round(2 * upd / med / 1e9 / PEAK_FP32_VALU_TFLOPS, 4)}
    print(f"[bench] bf16 vector-ALU gathers: {res}", file=sys.stderr, flush=True)
    return res


def time_page_shapes(sgc, torch, np, dev, stream, reps=5):
    """The DISCO page's own benchmark shapes (section "Serial Benchmarks": Gauss-Legendre grids,
    theta_c = 0.017, K = 9 stand-in basis, batch 1), bf16: fused convolution and its backward
    (median of `reps`, p10 and p90)."""
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
            ms, p10, p90 = _timed(torch, np, stream, fn, reps)
            alg = (2 * upd + 2 * macs) * (2 if op == "fused_bwd" else 1)
            r[op] = {"ms": round(ms, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                     "mfma_tflops_algorithmic": round(alg / ms / 1e9, 3),
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
    return {"value": round(total / (t_fb + t_u) / 1e9, 4), "unit": "Gnnz-updates/s",
            "cores": len(os.sched_getaffinity(0)), "threads": oracle.num_threads(), "kind": "oracle",
            "legs_s": {"fwd_bwd": round(t_fb, 2), "fused": round(t_u, 2)},
            "sample": f"fwd+bwd on {planes}/64 channel planes of the 721x1440 K=8 workload "
                      f"({t_fb:.1f}s) + fused contraction and einsum for latitudes {hos} of batch 0 of the "
                      f"K=16 workload ({t_u:.1f}s); updates counted as in value",
            "seconds": round(t_fb + t_u, 2)}


if __name__ == "__main__":
    main()

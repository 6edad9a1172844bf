"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Error measure (per output element): |gpu - oracle| / N, with N the same
contraction taken over absolute values (sum |val * x|, and sum |W| * N_out for
the fused op).  Elements with N == 0 must be exactly 0.  Bars: 1e-5 for fp32
data, 2e-2 for bf16 data with fp32 accumulation.

Full-size workloads run on the GPU exactly as the benchmark launches them; the
oracle then checks whole (b, c) planes (every latitude, poles included) or
whole output latitudes of the fused op.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_gather_contraction_amd as sgc
from disco_inputs import WORKLOADS, randn, randn_device, workload_gout, workload_psi, workload_weight, workload_x
from disco_inputs.psi import PsiCSR, build_psi, random_psi

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = torch.device("cuda", 0)


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


def normalised_error(gpu, ref, nrm):
    g = gpu.detach().double().cpu().numpy() if hasattr(gpu, "detach") else np.asarray(gpu, np.float64)
    assert g.shape == ref.shape == nrm.shape
    assert np.all(np.isfinite(g)), "non-finite output (unwritten or NaN)"
    zero = nrm == 0
    assert np.all(g[zero] == 0.0), "elements with zero normaliser must be exactly 0"
    if np.all(zero):
        return 0.0
    return float(np.max(np.abs(g[~zero] - ref[~zero]) / nrm[~zero]))


F16_SUBNORMAL_HALF_SPACING = 2.0 ** -25  # rounding a result below fp16's normal range errs by up to this


def normalised_error_f16(gpu, ref, nrm):
    """normalised_error for fp16 results, with the absolute rounding error of fp16 subnormals taken off
    (a result below 2^-14 has an ulp of 2^-24, not a relative one)."""
    g = gpu.detach().double().cpu().numpy() if hasattr(gpu, "detach") else np.asarray(gpu, np.float64)
    assert g.shape == ref.shape == nrm.shape
    assert np.all(np.isfinite(g)), "non-finite output (unwritten or NaN)"
    zero = nrm == 0
    assert np.all(g[zero] == 0.0), "elements with zero normaliser must be exactly 0"
    if np.all(zero):
        return 0.0
    return float(np.max(np.maximum(np.abs(g[~zero] - ref[~zero]) - F16_SUBNORMAL_HALF_SPACING, 0.0) / nrm[~zero]))


_PSI = {}


def gpu_psi(psi):
    key = id(psi)
    if key not in _PSI:
        _PSI[key] = (psi, sgc.disco_psi_create(psi, 0))
    return _PSI[key][1]


def nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def tdtype(s):
    return torch.float32 if s == "f32" else torch.bfloat16


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["tiny_fwd_f32_16x32", "fwdbwd_f32_181x360"])
def test_fwd_full_parity_fp32(name):
    w = WORKLOADS[name]
    _log(f"fwd {name}")
    psi = workload_psi(w)
    x = workload_x(w)
    out = nan_like((w.B, w.C, w.K, w.Ho, w.Wo), torch.float32)
    sgc.disco_fwd(gpu_psi(psi), x.to(DEV), out)
    torch.cuda.synchronize()
    ref = oracle.fwd(psi, x)
    nrm = oracle.fwd(psi, x.abs(), abs_mode=True)
    assert normalised_error(out, ref, nrm) <= TOL["f32"]


def test_bwd_full_parity_fp32():
    w = WORKLOADS["fwdbwd_f32_181x360"]
    _log("bwd fwdbwd_f32_181x360")
    psi = workload_psi(w)
    g = workload_gout(w)
    gx = nan_like((w.B, w.C, w.Hi, w.Wi), torch.float32)
    sgc.disco_bwd(gpu_psi(psi), g.to(DEV), gx)
    torch.cuda.synchronize()
    ref = oracle.bwd(psi, g)
    nrm = oracle.bwd(psi, g.abs(), abs_mode=True)
    assert normalised_error(gx, ref, nrm) <= TOL["f32"]


@pytest.mark.parametrize("planes", [1, 3, 4, 6])
def test_fp32_181x360_few_planes(planes):
    """With few channel planes the tiled gather splits each task's records over more waves (2 or 4 waves
    share a workgroup's planes and add their partial sums in wave order); the 181x360 forward's tasks are
    large enough for that split.  Forward and backward against the oracle."""
    w = WORKLOADS["fwdbwd_f32_181x360"]
    _log(f"fp32 181x360 with {planes} planes")
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = randn((1, planes, w.Hi, w.Wi), 3900 + planes, "f32")
    out = nan_like((1, planes, w.K, w.Ho, w.Wo), torch.float32)
    sgc.disco_fwd(h, x.to(DEV), out)
    g = randn((1, planes, w.K, w.Ho, w.Wo), 3950 + planes, "f32")
    gx = nan_like((1, planes, w.Hi, w.Wi), torch.float32)
    sgc.disco_bwd(h, g.to(DEV), gx)
    torch.cuda.synchronize()
    assert normalised_error(out, oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL["f32"]
    assert normalised_error(gx, oracle.bwd(psi, g), oracle.bwd(psi, g.abs(), abs_mode=True)) <= TOL["f32"]


PLANES_721 = [0, 21, 42, 63]


def test_fwd_bf16_721x1440_full_size():
    w = WORKLOADS["fwd_bf16_721x1440"]
    _log("fwd_bf16_721x1440 (GPU full, oracle on 4 planes)")
    psi = workload_psi(w)
    x = workload_x(w)
    out = nan_like((w.B, w.C, w.K, w.Ho, w.Wo), torch.bfloat16)
    sgc.disco_fwd(gpu_psi(psi), x.to(DEV), out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    xs = x[0, PLANES_721]
    ref = oracle.fwd(psi, xs)
    nrm = oracle.fwd(psi, xs.abs(), abs_mode=True)
    assert normalised_error(out[0, PLANES_721], ref, nrm) <= TOL["bf16"]


def test_bwd_bf16_721x1440_full_size():
    w = WORKLOADS["bwd_bf16_721x1440"]
    _log("bwd_bf16_721x1440 (GPU full, oracle on 4 planes)")
    psi = workload_psi(w)
    g = workload_gout(w)
    gx = nan_like((w.B, w.C, w.Hi, w.Wi), torch.bfloat16)
    sgc.disco_bwd(gpu_psi(psi), g.to(DEV), gx)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(gx).all())
    gs = g[0, PLANES_721]
    ref = oracle.bwd(psi, gs)
    nrm = oracle.bwd(psi, gs.abs(), abs_mode=True)
    assert normalised_error(gx[0, PLANES_721], ref, nrm) <= TOL["bf16"]


def test_fused_721x1440_full_size():
    w = WORKLOADS["fused_bf16_721x1440"]
    _log("fused_bf16_721x1440 (GPU full, oracle on 5 latitudes)")
    psi = workload_psi(w)
    x = workload_x(w)
    W = workload_weight(w)
    y = nan_like((w.B, w.Co, w.Ho, w.Wo), torch.bfloat16)
    sgc.disco_fused_conv(gpu_psi(psi), x.to(DEV), W.to(DEV), y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    hos = [0, 3, 360, 601]
    ref = oracle.fused(psi, x, W, ho_list=hos)
    nrm = oracle.fused(psi, x.abs(), W.abs(), ho_list=hos, abs_mode=True)
    assert normalised_error(y[:, :, hos], ref, nrm) <= TOL["bf16"]


# ---------------------------------------------------------------- edge cases

def _fwd_bwd_check(psi, BC, dtype, seed):
    x = randn((1, BC, psi.Hi, psi.Wi), seed, dtype)
    g = randn((1, BC, psi.K, psi.Ho, psi.Wo), seed + 1, dtype)
    h = sgc.disco_psi_create(psi, 0)
    out = nan_like((1, BC, psi.K, psi.Ho, psi.Wo), tdtype(dtype))
    gx = nan_like((1, BC, psi.Hi, psi.Wi), tdtype(dtype))
    sgc.disco_fwd(h, x.to(DEV), out)
    sgc.disco_bwd(h, g.to(DEV), gx)
    torch.cuda.synchronize()
    e1 = normalised_error(out, oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True))
    e2 = normalised_error(gx, oracle.bwd(psi, g), oracle.bwd(psi, g.abs(), abs_mode=True))
    return e1, e2


@pytest.mark.parametrize("BC", [1, 3, 4, 7, 8, 9, 65])
def test_channel_counts(BC):
    psi = workload_psi(WORKLOADS["tiny_fwd_f32_16x32"])
    e1, e2 = _fwd_bwd_check(psi, BC, "f32", 100 + BC)
    assert e1 <= TOL["f32"] and e2 <= TOL["f32"]


@pytest.mark.parametrize("geom", [
    # Hi, Wi, Ho, Wo, theta_c, n_r, n_a: polar caps spanning whole rings, wrapped runs, pscale 2 and 3
    (31, 60, 16, 20, 0.5, 2, 2),
    (31, 60, 31, 20, 1.5, 3, 4),
    (37, 72, 19, 24, 0.9, 4, 2),
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_generated_psi_geometries(geom, dtype):
    psi = build_psi(*geom)
    e1, e2 = _fwd_bwd_check(psi, 6, dtype, 300)
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype]


def test_random_psi_with_empty_rows_and_long_rows():
    # Wo = 1100 > 1024 exercises the outer position loop; dense rows give runs longer than one segment
    psi = random_psi(3, 4, 1100, 5, 2200, 0.05, seed=11, empty_rows=(0, 5, 11))
    psi_dense = random_psi(2, 3, 40, 4, 80, 0.9, seed=12, empty_rows=(1,))
    for p, seed in ((psi, 400), (psi_dense, 410)):
        e1, e2 = _fwd_bwd_check(p, 5, "f32", seed)
        assert e1 <= TOL["f32"] and e2 <= TOL["f32"]


def test_empty_rows_write_exact_zero():
    psi = random_psi(2, 5, 16, 6, 32, 0.2, seed=13, empty_rows=(0, 3, 7))
    h = sgc.disco_psi_create(psi, 0)
    x = randn((2, 3, 6, 32), 500).to(DEV)
    out = nan_like((2, 3, 2, 5, 16), torch.float32)
    sgc.disco_fwd(h, x, out)
    torch.cuda.synchronize()
    flat = out.reshape(2, 3, 10, 16)
    for r in (0, 3, 7):
        assert bool((flat[:, :, r] == 0).all())
    # input rows no entry touches come back as exact zeros from the backward
    gx = nan_like((2, 3, 6, 32), torch.float32)
    sgc.disco_bwd(h, randn((2, 3, 2, 5, 16), 501).to(DEV), gx)
    torch.cuda.synchronize()
    used = np.zeros((6, 32), bool)
    used[psi.col_hi, :] = True  # every longitude of a touched row can be reached by some wo
    assert bool(torch.isfinite(gx).all())
    for hi in range(6):
        if not used[hi].any():
            assert bool((gx[:, :, hi] == 0).all())


def test_bitwise_deterministic():
    w = WORKLOADS["fwdbwd_f32_181x360"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = workload_x(w).to(DEV)
    g = workload_gout(w).to(DEV)
    o1, o2 = sgc.disco_fwd(h, x), sgc.disco_fwd(h, x)
    g1, g2 = sgc.disco_bwd(h, g), sgc.disco_bwd(h, g)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(g1, g2)


def test_bf16_against_fp32_variant():
    w = WORKLOADS["fwdbwd_f32_181x360"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    xb = randn((2, 8, w.Hi, w.Wi), 600, "bf16").to(DEV)
    ob = sgc.disco_fwd(h, xb)
    of = sgc.disco_fwd(h, xb.float())
    torch.cuda.synchronize()
    nrm = oracle.fwd(psi, xb.cpu().abs(), abs_mode=True)
    assert normalised_error(ob, of.double().cpu().numpy(), nrm) <= TOL["bf16"]


# ---------------------------------------------------------------- fused

@pytest.mark.parametrize("cfg", [
    # (Hi, Wi, Ho, Wo, theta_c, n_r, n_a, B, C, Co)
    (31, 60, 31, 60, 0.5, 4, 4, 2, 8, 32),      # K=16, p=1, Wo % 8 != 0 (VALU-contraction kernel)
    (31, 64, 31, 64, 0.5, 4, 4, 2, 8, 32),      # K=16, p=1, packed matrix-core kernel, ragged longitude tile
    (31, 64, 31, 64, 1.5, 4, 4, 1, 6, 33),      # caps spanning whole rings: several packed pieces per latitude
    (31, 60, 16, 30, 0.6, 3, 1, 1, 23, 20),     # K=3: chunk of 21 channels, Co not a multiple of 16
    (19, 144, 19, 72, 0.7, 4, 2, 2, 9, 300),    # K=8, p=2, Co > one block
    (13, 40, 13, 40, 0.9, 2, 2, 1, 1, 1),       # single channel in and out
])
def test_fused_small_ragged(cfg):
    Hi, Wi, Ho, Wo, tc, n_r, n_a, B, C, Co = cfg
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((B, C, Hi, Wi), 700, "bf16")
    W = randn((Co, C, psi.K), 701, "bf16", std=1.0 / np.sqrt(C * psi.K))
    y = nan_like((B, Co, Ho, Wo), torch.bfloat16)
    sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.fused(psi, x, W)
    nrm = oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)
    assert normalised_error(y, ref, nrm) <= TOL["bf16"]


def test_fused_equals_einsum_of_forward():
    psi = build_psi(31, 60, 31, 60, 0.5, 4, 4)
    h = sgc.disco_psi_create(psi, 0)
    B, C, Co = 2, 12, 24
    x = randn((B, C, 31, 60), 710, "bf16").to(DEV)
    W = randn((Co, C, psi.K), 711, "bf16", std=0.1).to(DEV)
    y = sgc.disco_fused_conv(h, x, W)
    out = sgc.disco_fwd(h, x.float())  # fp32 contraction
    yu = torch.matmul(W.float().reshape(Co, C * psi.K), out.reshape(B, C * psi.K, -1)).reshape(B, Co, 31, 60)
    torch.cuda.synchronize()
    nrm = oracle.fused(psi, x.cpu().abs(), W.cpu().abs(), abs_mode=True)
    assert normalised_error(y, yu.double().cpu().numpy(), nrm) <= TOL["bf16"]


# ---------------------------------------------------------------- error paths on the device

def _raw(fn, *descs):
    lib = sgc.load_library()
    st = getattr(lib, fn)(*descs)
    return sgc.STATUS_NAMES[st], lib.disco_last_error().decode()


def test_error_paths_leave_outputs_untouched():
    psi = workload_psi(WORKLOADS["tiny_fwd_f32_16x32"])
    h = gpu_psi(psi)
    x = randn((1, 2, psi.Hi, psi.Wi), 800).to(DEV)
    sentinel = 7.25
    out = torch.full((1, 2, psi.K, psi.Ho, psi.Wo + 1), sentinel, device=DEV)  # wrong Wo
    st, msg = _raw("disco_fwd", h.handle, ctypes.byref(sgc.tensor_desc(x)), ctypes.byref(sgc.tensor_desc(out)), None)
    assert st == "DISCO_ERR_SHAPE"
    out_bf = torch.full((1, 2, psi.K, psi.Ho, psi.Wo), sentinel, device=DEV, dtype=torch.bfloat16)
    st, msg = _raw("disco_fwd", h.handle, ctypes.byref(sgc.tensor_desc(x)), ctypes.byref(sgc.tensor_desc(out_bf)), None)
    assert st == "DISCO_ERR_DTYPE"
    x64 = x.double()  # fp64 data is not a supported dtype
    out16 = torch.full((1, 2, psi.K, psi.Ho, psi.Wo), sentinel, device=DEV, dtype=torch.float64)
    st, msg = _raw("disco_fwd", h.handle, ctypes.byref(sgc.tensor_desc(x64)), ctypes.byref(sgc.tensor_desc(out16)), None)
    assert st == "DISCO_ERR_DTYPE"
    host = torch.full((1, 2, psi.K, psi.Ho, psi.Wo), sentinel)
    st, msg = _raw("disco_fwd", h.handle, ctypes.byref(sgc.tensor_desc(x)), ctypes.byref(sgc.tensor_desc(host)), None)
    assert st == "DISCO_ERR_INVALID_ARGUMENT" and "device memory" in msg
    Wf = torch.zeros((3, 2, psi.K), device=DEV, dtype=torch.bfloat16)  # dtypes of one call differ
    yf = torch.full((1, 3, psi.Ho, psi.Wo), sentinel, device=DEV)
    st, msg = _raw("disco_fused_conv", h.handle, ctypes.byref(sgc.tensor_desc(x)), ctypes.byref(sgc.tensor_desc(Wf)),
                   ctypes.byref(sgc.tensor_desc(yf)), None)
    assert st == "DISCO_ERR_DTYPE"
    torch.cuda.synchronize()
    for t in (out, out_bf, out16, host, yf):
        assert bool((t == sentinel).all())
    # an empty batch is valid and writes nothing
    x0 = torch.empty((0, 2, psi.Hi, psi.Wi), device=DEV)
    assert sgc.disco_fwd(h, x0).shape == (0, 2, psi.K, psi.Ho, psi.Wo)


def test_architecture_refusal_knob(monkeypatch):
    psi = workload_psi(WORKLOADS["tiny_fwd_f32_16x32"])
    monkeypatch.setenv("DISCO_REQUIRE_ARCH", "gfx000")
    with pytest.raises(sgc.DiscoError) as ei:
        sgc.disco_psi_create(psi, 0)
    assert ei.value.status_name == "DISCO_ERR_UNSUPPORTED_DEVICE"
    monkeypatch.delenv("DISCO_REQUIRE_ARCH")
    sgc.disco_psi_create(psi, 0).close()


@pytest.mark.parametrize("path", ["tiled", "staged", "plain"])
def test_plain_staged_and_tiled_gather_agree_with_oracle(path, monkeypatch):
    """fp32 data runs the register-tiled gather where its plan covers the shape; DISCO_TILE=0 falls
    back to the LDS-staged gather and DISCO_TILE=0 DISCO_STAGED=0 to the plain one (bf16 data with
    DISCO_FWD_MFMA=0 / DISCO_BWD_MFMA=0 takes the same vector-ALU gathers)."""
    monkeypatch.setenv("DISCO_TILE", "1" if path == "tiled" else "0")
    monkeypatch.setenv("DISCO_STAGED", "0" if path == "plain" else "1")
    monkeypatch.setenv("DISCO_FWD_MFMA", "0")
    monkeypatch.setenv("DISCO_BWD_MFMA", "0")
    w = WORKLOADS["fwdbwd_f32_181x360"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    for dtype in ("f32", "bf16"):
        x = randn((1, 5, w.Hi, w.Wi), 900, dtype)
        g = randn((1, 5, w.K, w.Ho, w.Wo), 901, dtype)
        out = sgc.disco_fwd(h, x.to(DEV))
        gx = sgc.disco_bwd(h, g.to(DEV))
        torch.cuda.synchronize()
        assert normalised_error(out, oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL[dtype]
        assert normalised_error(gx, oracle.bwd(psi, g), oracle.bwd(psi, g.abs(), abs_mode=True)) <= TOL[dtype]


@pytest.mark.parametrize("mfma", ["0", "1"])
def test_fused_both_kernels_agree_with_oracle(mfma, monkeypatch):
    """DISCO_FUSED_MFMA=0 forces the VALU-contraction fused kernel on a shape the packed kernel covers."""
    monkeypatch.setenv("DISCO_FUSED_MFMA", mfma)
    psi = build_psi(19, 144, 19, 72, 0.7, 4, 2)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((2, 5, 19, 144), 950, "bf16")
    W = randn((40, 5, psi.K), 951, "bf16", std=0.2)
    y = sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.fused(psi, x, W)
    nrm = oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)
    assert normalised_error(y, ref, nrm) <= TOL["bf16"]


@pytest.mark.parametrize("mfma", ["0", "1"])
@pytest.mark.parametrize("geom", [(31, 64, 31, 64, 0.5, 4, 2, 9), (33, 128, 17, 64, 0.6, 4, 2, 8),
                                  (25, 48, 25, 48, 0.7, 4, 4, 5), (19, 144, 19, 72, 0.7, 4, 1, 3)])
def test_fwd_bf16_both_kernels_agree_with_oracle(geom, mfma, monkeypatch):
    """bf16 forward on the matrix cores (phase-split psi; K <= 8 and K = 16, s = 1 and 2, ragged
    channel counts and longitude spans) and, with DISCO_FWD_MFMA=0, on the vector-ALU gather."""
    monkeypatch.setenv("DISCO_FWD_MFMA", mfma)
    Hi, Wi, Ho, Wo, tc, nr, na, C = geom
    psi = build_psi(Hi, Wi, Ho, Wo, tc, nr, na)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((2, C, Hi, Wi), 960 + C, "bf16")
    out = sgc.disco_fwd(h, x.to(DEV))
    torch.cuda.synchronize()
    assert normalised_error(out, oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL["bf16"]


@pytest.mark.parametrize("mfma", ["0", "1"])
@pytest.mark.parametrize("geom", [(31, 64, 31, 64, 0.5, 4, 2, 9), (33, 128, 17, 64, 0.6, 4, 2, 8),
                                  (25, 48, 25, 48, 0.7, 4, 4, 5), (19, 144, 19, 72, 0.7, 4, 1, 3)])
def test_bwd_bf16_both_kernels_agree_with_oracle(geom, mfma, monkeypatch):
    """bf16 backward on the matrix cores (a forward over the inverse CSR: gradient rows grouped by
    eight, s = 1 and 2, K = 4..16, ragged channel counts) and, with DISCO_BWD_MFMA=0, on the
    vector-ALU gather."""
    monkeypatch.setenv("DISCO_BWD_MFMA", mfma)
    Hi, Wi, Ho, Wo, tc, nr, na, C = geom
    psi = build_psi(Hi, Wi, Ho, Wo, tc, nr, na)
    h = sgc.disco_psi_create(psi, 0)
    g = randn((2, C, psi.K, Ho, Wo), 970 + C, "bf16")
    gx = sgc.disco_bwd(h, g.to(DEV))
    torch.cuda.synchronize()
    assert normalised_error(gx, oracle.bwd(psi, g), oracle.bwd(psi, g.abs(), abs_mode=True)) <= TOL["bf16"]


# ---------------------------------------------------------------- backward of the fused convolution

def _fused_bwd_check(psi, B, C, Co, seed, dtype="bf16"):
    h = gpu_psi(psi)
    x = randn((B, C, psi.Hi, psi.Wi), seed, dtype)
    W = randn((Co, C, psi.K), seed + 1, dtype, std=1.0 / np.sqrt(C * psi.K))
    gy = randn((B, Co, psi.Ho, psi.Wo), seed + 2, dtype)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    gx = nan_like((B, C, psi.Hi, psi.Wi), tdt)
    dW = nan_like((Co, C, psi.K), tdt)
    sgc.disco_fused_conv_bwd(h, x.to(DEV), W.to(DEV), gy.to(DEV), gx, dW)
    torch.cuda.synchronize()
    rgx, rdW = oracle.fused_bwd(psi, x, W, gy)
    ngx, ndW = oracle.fused_bwd(psi, x, W, gy, abs_mode=True)
    return normalised_error(gx, rgx, ngx), normalised_error(dW, rdW, ndW), (gx, dW)


@pytest.mark.parametrize("cfg", [
    (31, 64, 31, 64, 0.5, 4, 4, 2, 20, 24),     # K=16, s=1: one chunk of 20 channels, positions not a tile multiple
    (19, 144, 19, 72, 0.7, 4, 2, 2, 9, 40),     # K=8, s=2: one chunk of 9 channels
    (25, 48, 25, 48, 0.7, 4, 1, 1, 70, 8),      # K=4: 70 channels in one chunk (up to 256 at K=4), Co = 8
    (16, 32, 16, 32, 2 * np.pi / 16, 3, 1, 3, 5, 136),  # K=3, B=3, Co above one tile
])
def test_fused_bwd_small_ragged(cfg):
    """Input and weight gradients of the fused convolution against the fp64 oracle (bf16 data)."""
    Hi, Wi, Ho, Wo, tc, nr, na, B, C, Co = cfg
    psi = build_psi(Hi, Wi, Ho, Wo, tc, nr, na)
    _log(f"fused bwd {cfg}")
    egx, edW, _ = _fused_bwd_check(psi, B, C, Co, 1100 + C)
    assert egx <= TOL["bf16"], egx
    assert edW <= TOL["bf16"], edW


@pytest.mark.parametrize("cfg", [
    (31, 64, 31, 64, 0.5, 4, 4, 2, 20, 24, "bf16"),   # K=16, s=1, Hi = Ho
    (21, 48, 17, 48, 0.6, 3, 3, 1, 9, 264, "f16"),    # K=9 (W' in rows of 16), Hi != Ho, Co over one tile
    (25, 48, 25, 48, 0.7, 4, 1, 2, 70, 8, "bf16"),    # K=4, B=2, 70 channels in one chunk
])
def test_fused_bwd_gx_through_the_transposed_psi(cfg, monkeypatch):
    """With Wi = Wo the fused backward computes gx as a fused convolution over the per-basis transpose of
    psi; DISCO_BWD_FUSED=0 keeps the W^T gy products and the transpose contraction.  Both against the
    oracle; dW does not depend on the gx path (bitwise equal)."""
    Hi, Wi, Ho, Wo, tc, nr, na, B, C, Co, dt = cfg
    psi = build_psi(Hi, Wi, Ho, Wo, tc, nr, na)
    _log(f"fused bwd gx paths {cfg}")
    tol = TOL_F16 if dt == "f16" else TOL["bf16"]
    egx, edW, (gx_t, dW_t) = _fused_bwd_check(psi, B, C, Co, 1500 + C, dt)
    assert egx <= tol and edW <= tol, (egx, edW)
    monkeypatch.setenv("DISCO_BWD_FUSED", "0")
    egx0, edW0, (gx_0, dW_0) = _fused_bwd_check(psi, B, C, Co, 1500 + C, dt)
    monkeypatch.delenv("DISCO_BWD_FUSED")
    assert egx0 <= tol and edW0 <= tol, (egx0, edW0)
    assert torch.equal(dW_t, dW_0)
    assert not torch.equal(gx_t, gx_0)  # the two paths round differently: both really ran


def test_fused_bwd_deterministic_and_workspace_reuse():
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    h = gpu_psi(psi)
    B, C, Co = 2, 18, 16
    x = randn((B, C, 31, 64), 1200, "bf16").to(DEV)
    W = randn((Co, C, psi.K), 1201, "bf16", std=0.05).to(DEV)
    gy = randn((B, Co, 31, 64), 1202, "bf16").to(DEV)
    ws = torch.full((sgc.disco_fused_conv_bwd_workspace(h, B, C, Co),), 0x7f, dtype=torch.uint8, device=DEV)
    a = sgc.disco_fused_conv_bwd(h, x, W, gy, workspace=ws)
    b = sgc.disco_fused_conv_bwd(h, x, W, gy, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fused_bwd_rejects_bad_arguments():
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    h = gpu_psi(psi)
    x = randn((1, 4, 31, 64), 1210, "bf16").to(DEV)
    W = randn((12, 4, psi.K), 1211, "bf16").to(DEV)   # Co = 12: not a multiple of 8
    gy = randn((1, 12, 31, 64), 1212, "bf16").to(DEV)
    gx = nan_like((1, 4, 31, 64), torch.bfloat16)
    dW = nan_like((12, 4, psi.K), torch.bfloat16)
    with pytest.raises(sgc.DiscoError, match="multiples of 8"):
        sgc.disco_fused_conv_bwd(h, x, W, gy, gx, dW)
    W8 = randn((8, 4, psi.K), 1213, "bf16").to(DEV)
    gy8 = randn((1, 8, 31, 64), 1214, "bf16").to(DEV)
    dW8 = nan_like((8, 4, psi.K), torch.bfloat16)
    small = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(sgc.DiscoError, match="workspace"):
        sgc.disco_fused_conv_bwd(h, x, W8, gy8, gx, dW8, workspace=small)
    with pytest.raises(sgc.DiscoError, match="bf16"):
        sgc.disco_fused_conv_bwd(h, x.float(), W8.float(), gy8.float(), gx.float(), dW8.float())
    torch.cuda.synchronize()
    assert torch.isnan(gx).all() and torch.isnan(dW8).all()


def test_fused_bwd_721x1440_full_size_sampled():
    """The 721x1440 K=16 workload (B=2, C=Co=256) as the benchmark runs it; input-gradient planes
    and weight-gradient columns of two channels checked against the oracle's transpose and
    forward contractions (each pinned) composed with exact fp64 products."""
    w = WORKLOADS["fused_bf16_721x1440"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = workload_x(w)
    W = workload_weight(w)
    gy = randn((w.B, w.Co, psi.Ho, psi.Wo), 1300, "bf16")
    _log("fused bwd 721x1440: GPU")
    gx, dW = sgc.disco_fused_conv_bwd(h, x.to(DEV), W.to(DEV), gy.to(DEV))
    torch.cuda.synchronize()
    gx, dW = gx.cpu(), dW.cpu()
    gy64 = gy.double().numpy().reshape(w.B, w.Co, -1)
    W64 = W.double().numpy()
    for c in (131,):
        _log(f"fused bwd 721x1440: oracle channel {c}")
        for b in range(w.B):
            g = (W64[:, c, :].T @ gy64[b]).reshape(1, psi.K, psi.Ho, psi.Wo)
            ga = (np.abs(W64[:, c, :]).T @ np.abs(gy64[b])).reshape(1, psi.K, psi.Ho, psi.Wo)
            ref = oracle.bwd(psi, g.astype(np.float32))
            nrm = oracle.bwd(psi, ga.astype(np.float32), abs_mode=True)
            # g is rounded to fp32 for the oracle call; the bound below covers that (2^-24 relative)
            assert normalised_error(gx[b, c][None], ref, nrm) <= TOL["bf16"]
        out = np.stack([oracle.fwd(psi, x[b, c][None])[0].reshape(psi.K, -1) for b in range(w.B)])
        outa = np.stack([oracle.fwd(psi, x[b, c][None].abs(), abs_mode=True)[0].reshape(psi.K, -1) for b in range(w.B)])
        ref = sum(gy64[b] @ out[b].T for b in range(w.B))
        nrm = sum(np.abs(gy64[b]) @ outa[b].T for b in range(w.B))
        assert normalised_error(dW[:, c, :], ref, nrm) <= TOL["bf16"]


# ---------------------------------------------------------------- fp16 data
# fp16 tensors (round to nearest even from the N(0,1) draw) and fp32 accumulation; every 16-bit
# result is rounded once.  The matrix-core paths take psi as fp16 of psi * 2^e (e puts the largest
# |psi| near 2^14; the power of two is undone exactly in fp32), the vector-ALU paths fp32 psi.
# Bar: 2e-3 of the normaliser, above the worst case 3 u (u = 2^-11, the fp16 unit roundoff: psi,
# the contraction chunk of the fused op, and the output).
TOL_F16 = 2e-3


@pytest.mark.parametrize("mfma", ["0", "1"])
@pytest.mark.parametrize("geom", [(31, 64, 31, 64, 0.5, 4, 2, 9), (33, 128, 17, 64, 0.6, 4, 2, 8),
                                  (19, 144, 19, 72, 0.7, 4, 1, 3), (16, 32, 16, 32, 2 * np.pi / 16, 3, 1, 4)])
def test_fwd_bwd_f16_agree_with_oracle(geom, mfma, monkeypatch):
    monkeypatch.setenv("DISCO_FWD_MFMA", mfma)
    monkeypatch.setenv("DISCO_BWD_MFMA", mfma)
    Hi, Wi, Ho, Wo, tc, nr, na, C = geom
    psi = build_psi(Hi, Wi, Ho, Wo, tc, nr, na)
    h = gpu_psi(psi)
    x = randn((2, C, Hi, Wi), 1400 + C, "f16")
    g = randn((2, C, psi.K, Ho, Wo), 1450 + C, "f16")
    out = sgc.disco_fwd(h, x.to(DEV))
    gx = sgc.disco_bwd(h, g.to(DEV))
    torch.cuda.synchronize()
    assert out.dtype == torch.float16 and gx.dtype == torch.float16
    assert normalised_error(out, oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL_F16
    assert normalised_error(gx, oracle.bwd(psi, g), oracle.bwd(psi, g.abs(), abs_mode=True)) <= TOL_F16


@pytest.mark.parametrize("mfma", ["0", "1"])
@pytest.mark.parametrize("cfg", [
    (31, 64, 31, 64, 0.5, 4, 4, 2, 8, 32),
    (31, 64, 31, 64, 1.5, 4, 4, 1, 6, 33),
    (19, 144, 19, 72, 0.7, 4, 2, 2, 9, 300),
    (31, 60, 16, 30, 0.6, 3, 1, 1, 23, 20),
])
def test_fused_f16_agrees_with_oracle(cfg, mfma, monkeypatch):
    monkeypatch.setenv("DISCO_FUSED_MFMA", mfma)
    Hi, Wi, Ho, Wo, tc, n_r, n_a, B, C, Co = cfg
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    h = gpu_psi(psi)
    x = randn((B, C, Hi, Wi), 1500 + C, "f16")
    W = randn((Co, C, psi.K), 1501 + C, "f16", std=1.0 / np.sqrt(C * psi.K))
    y = nan_like((B, Co, Ho, Wo), torch.float16)
    sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.fused(psi, x, W)
    nrm = oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)
    assert normalised_error(y, ref, nrm) <= TOL_F16


def test_f16_721x1440_forward_sampled():
    """The 721x1440 K=8 forward with fp16 data at its benchmark size (matrix cores); two whole
    channel planes."""
    w = WORKLOADS["fwd_bf16_721x1440"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = randn((w.B, w.C, w.Hi, w.Wi), 1600, "f16")
    out = sgc.disco_fwd(h, x.to(DEV))
    torch.cuda.synchronize()
    for c in (0, 37):
        xs = x[:, c:c + 1]
        assert normalised_error(out[:, c:c + 1].cpu(), oracle.fwd(psi, xs),
                                oracle.fwd(psi, xs.abs(), abs_mode=True)) <= TOL_F16


def test_f16_fused_721x1440_sampled():
    """The 721x1440 K=16 fused op with fp16 data at its benchmark size (matrix cores); whole output
    latitudes from pole to equator."""
    w = WORKLOADS["fused_bf16_721x1440"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = randn((w.B, w.C, w.Hi, w.Wi), 1700, "f16")
    W = randn((w.Co, w.C, w.K), 1701, "f16", std=1.0 / np.sqrt(w.C * w.K))
    y = sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    hos = [0, 3, 200, 360]
    ref = oracle.fused(psi, x[:1], W, ho_list=hos)
    nrm = oracle.fused(psi, x[:1].abs(), W.abs(), ho_list=hos, abs_mode=True)
    assert normalised_error(y[:1, :, hos].cpu(), ref, nrm) <= TOL_F16


# ---------------------------------------------------------------- the page's benchmark shapes

@pytest.mark.parametrize("name", ["page_self_256x360x720", "page_self_512x360x720", "page_down_80x721x1440"])
def test_page_shapes_fused_sampled(name):
    """Fused convolution at the DISCO page's benchmark shapes (Gauss-Legendre grids, K = 9): whole
    output latitudes from pole to equator against the oracle."""
    w = WORKLOADS[name]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = workload_x(w)
    W = workload_weight(w)
    _log(f"{name}: GPU")
    y = sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    hos = [0, 1, 90, 179, 359]
    ref = oracle.fused(psi, x, W, ho_list=hos)
    nrm = oracle.fused(psi, x.abs(), W.abs(), ho_list=hos, abs_mode=True)
    assert normalised_error(y[:, :, hos].cpu(), ref, nrm) <= TOL["bf16"]


def test_page_shape_fused_bwd_sampled():
    """Fused backward at the page's down-sampling shape (721x1440 equiangular -> 360x720
    Gauss-Legendre, s = 2, 80 -> 512 channels); one input channel's gradients checked."""
    w = WORKLOADS["page_down_80x721x1440"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = workload_x(w)
    W = workload_weight(w)
    gy = randn((w.B, w.Co, psi.Ho, psi.Wo), 1800, "bf16")
    gx, dW = sgc.disco_fused_conv_bwd(h, x.to(DEV), W.to(DEV), gy.to(DEV))
    torch.cuda.synchronize()
    gx, dW = gx.cpu(), dW.cpu()
    gy64 = gy.double().numpy().reshape(w.B, w.Co, -1)
    W64 = W.double().numpy()
    c = 37
    g = (W64[:, c, :].T @ gy64[0]).reshape(1, psi.K, psi.Ho, psi.Wo)
    ga = (np.abs(W64[:, c, :]).T @ np.abs(gy64[0])).reshape(1, psi.K, psi.Ho, psi.Wo)
    assert normalised_error(gx[0, c][None], oracle.bwd(psi, g.astype(np.float32)),
                            oracle.bwd(psi, ga.astype(np.float32), abs_mode=True)) <= TOL["bf16"]
    out = oracle.fwd(psi, x[0, c][None])[0].reshape(psi.K, -1)
    outa = oracle.fwd(psi, x[0, c][None].abs(), abs_mode=True)[0].reshape(psi.K, -1)
    assert normalised_error(dW[:, c, :], gy64[0] @ out.T, np.abs(gy64[0]) @ outa.T) <= TOL["bf16"]


# ---------------------------------------------------------------- the einsum alone

TOL_EIN = {"bf16": 2e-2, "f16": 2e-3}


@pytest.mark.parametrize("cfg", [
    # (B, C, Co, K, Ho, Wo, dtype)
    (2, 5, 40, 3, 7, 37, "bf16"),      # ragged channel chunk, K < 16, 259 positions (element loads, ragged tile)
    (1, 8, 256, 16, 16, 64, "bf16"),   # direct loads of t and W, one full output-channel block
    (2, 9, 300, 8, 5, 48, "bf16"),     # two output-channel blocks (the second ragged), K = 8
    (1, 12, 64, 16, 3, 100, "f16"),    # fp16, 300 positions (ragged last tile)
    (1, 4, 33, 16, 1, 8, "f16"),       # one partial tile
])
def test_einsum_small_ragged(cfg):
    B, C, Co, K, Ho, Wo, dt = cfg
    _log(f"einsum {cfg}")
    t = randn((B, C, K, Ho, Wo), 3100 + C, dt)
    W = randn((Co, C, K), 3200 + C, dt, std=1.0 / np.sqrt(C * K))
    y = nan_like((B, Co, Ho, Wo), t.dtype)
    sgc.disco_einsum(W.to(DEV), t.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.einsum(W, t)
    nrm = oracle.einsum(W.abs(), t.abs(), abs_mode=True)
    assert normalised_error(y.cpu(), ref, nrm) <= TOL_EIN[dt]


def test_einsum_edge_cases_and_errors():
    _log("einsum edge cases")
    # no input channels: y is exactly zero; no positions: nothing to do
    W0 = torch.empty((8, 0, 16), dtype=torch.bfloat16, device=DEV)
    t0 = torch.empty((1, 0, 16, 4, 8), dtype=torch.bfloat16, device=DEV)
    y0 = sgc.disco_einsum(W0, t0, nan_like((1, 8, 4, 8), torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.all(y0 == 0)
    sgc.disco_einsum(torch.zeros((8, 3, 4), dtype=torch.bfloat16, device=DEV),
                     torch.zeros((2, 3, 4, 0, 8), dtype=torch.bfloat16, device=DEV))
    # rejected calls leave the output untouched
    t = randn((1, 3, 4, 2, 8), 3300, "bf16").to(DEV)
    W = randn((5, 3, 4), 3301, "bf16").to(DEV)
    y = nan_like((1, 5, 2, 8), torch.bfloat16)
    bad = [
        (W, randn((1, 3, 17, 2, 8), 3302, "bf16").to(DEV), y, "DISCO_ERR_SHAPE"),  # K > 16
        (W.float(), t.float(), y.float(), "DISCO_ERR_DTYPE"),                        # fp32
        (W, t, nan_like((1, 5, 2, 8), torch.float16), "DISCO_ERR_DTYPE"),            # dtypes differ
        (W, t, nan_like((1, 4, 2, 8), torch.bfloat16), "DISCO_ERR_SHAPE"),           # y channels
        (randn((5, 2, 4), 3303, "bf16").to(DEV), t, y, "DISCO_ERR_SHAPE"),            # W channels
    ]
    for Wb, tb, yb, code in bad:
        with pytest.raises(sgc.DiscoError) as e:
            sgc.disco_einsum(Wb, tb, yb)
        assert e.value.status_name == code
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(y))


def test_einsum_721x1440_full_size_sampled():
    """The einsum at the fused workload's GEMM shape (B=2, C=Co=256, K=16, 721x1440), launched as the
    bench times it; whole output latitudes from pole to equator against the oracle, and bitwise
    run-to-run determinism."""
    w = WORKLOADS["fused_bf16_721x1440"]
    _log("einsum 721x1440")
    t = randn_device((w.B, w.C, w.K, w.Ho, w.Wo), 3400, "bf16", DEV)
    W = workload_weight(w)
    y = sgc.disco_einsum(W.to(DEV), t)
    y2 = sgc.disco_einsum(W.to(DEV), t)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    hos = [0, 360, 720]
    ts = t[:, :, :, hos].cpu()
    ref = oracle.einsum(W, ts)
    nrm = oracle.einsum(W.abs(), ts.abs(), abs_mode=True)
    assert normalised_error(y[:, :, hos].cpu(), ref, nrm) <= TOL_EIN["bf16"]


def test_one_handle_from_two_streams():
    """A psi handle is read-only after creation and may be used from several streams at once: the
    forward and backward on one side stream, the fused op and the einsum on another, and both fused
    backwards (which fork onto the library's own second stream) on both, concurrently, each equal
    bitwise to the same call on the default stream."""
    _log("two streams")
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((2, 8, 31, 64), 3600, "bf16").to(DEV)
    g = randn((2, 8, psi.K, 31, 64), 3601, "bf16").to(DEV)
    W = randn((16, 8, psi.K), 3602, "bf16", std=0.1).to(DEV)
    gy = randn((2, 16, 31, 64), 3603, "bf16").to(DEV)
    _, kept = sgc.disco_fused_conv_save(h, x, W)
    ref = (sgc.disco_fwd(h, x), sgc.disco_bwd(h, g), sgc.disco_fused_conv(h, x, W), sgc.disco_einsum(W, g),
           *sgc.disco_fused_conv_bwd_saved(h, kept, W, gy), *sgc.disco_fused_conv_bwd(h, x, W, gy))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)  # default priority
    outs = []
    for _ in range(3):
        # both backwards fork onto the library's side stream, from both caller streams at once
        with torch.cuda.stream(sa):
            o, gx = sgc.disco_fwd(h, x), sgc.disco_bwd(h, g)
            sgx_a, sdw_a = sgc.disco_fused_conv_bwd_saved(h, kept, W, gy)
            rgx_a, rdw_a = sgc.disco_fused_conv_bwd(h, x, W, gy)
        with torch.cuda.stream(sb):
            y, ye = sgc.disco_fused_conv(h, x, W), sgc.disco_einsum(W, g)
            sgx_b, sdw_b = sgc.disco_fused_conv_bwd_saved(h, kept, W, gy)
            rgx_b, rdw_b = sgc.disco_fused_conv_bwd(h, x, W, gy)
        outs.append((o, gx, y, ye, sgx_a, sdw_a, rgx_a, rdw_a))
        outs.append((o, gx, y, ye, sgx_b, sdw_b, rgx_b, rdw_b))
    torch.cuda.synchronize()
    for got in outs:
        for a, b in zip(got, ref):
            assert torch.equal(a, b)


# ---------------------------------------------------------------- fused op that keeps its contraction

@pytest.mark.parametrize("geom,B,C,Co", [
    ((31, 64, 31, 64, 0.5, 4, 4), 2, 12, 24),   # three 4-channel chunks, Co below one 32-row tile
    ((33, 128, 17, 64, 0.6, 4, 4), 1, 7, 40),   # s = 2, ragged channel chunk and output tiles
])
def test_fused_save_and_saved_backward(geom, B, C, Co):
    """disco_fused_conv_save: y equal bitwise to disco_fused_conv, the kept contraction within the bar of
    the oracle's forward; disco_fused_conv_bwd_saved on it equal bitwise to disco_fused_conv_bwd."""
    _log(f"fused save {geom} B={B} C={C} Co={Co}")
    psi = build_psi(*geom)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((B, C, psi.Hi, psi.Wi), 3700 + C, "bf16").to(DEV)
    W = randn((Co, C, psi.K), 3701 + C, "bf16", std=0.1).to(DEV)
    gy = randn((B, Co, psi.Ho, psi.Wo), 3702 + C, "bf16").to(DEV)
    y0 = sgc.disco_fused_conv(h, x, W)
    y, out = sgc.disco_fused_conv_save(h, x, W)
    gx0, dW0 = sgc.disco_fused_conv_bwd(h, x, W, gy)
    gx, dW = sgc.disco_fused_conv_bwd_saved(h, out, W, gy)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    xc = x.cpu()
    assert normalised_error(out.cpu(), oracle.fwd(psi, xc), oracle.fwd(psi, xc.abs(), abs_mode=True)) <= TOL["bf16"]
    assert torch.equal(gx, gx0) and torch.equal(dW, dW0)


def test_fused_save_fallback_path(monkeypatch):
    """Without the matrix-core fused kernel the contraction is kept by the forward kernel; both
    results within the bar of the oracle."""
    monkeypatch.setenv("DISCO_FUSED_MFMA", "0")
    psi = build_psi(31, 60, 31, 60, 0.5, 4, 4)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((1, 6, 31, 60), 3710, "bf16")
    W = randn((16, 6, psi.K), 3711, "bf16", std=0.1)
    y, out = sgc.disco_fused_conv_save(h, x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    assert normalised_error(out.cpu(), oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL["bf16"]
    assert normalised_error(y.cpu(), oracle.fused(psi, x, W), oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)) <= TOL["bf16"]


def test_fused_save_721x1440_full_size():
    """The fused workload (B=2, C=Co=256, K=16, 721x1440) as the bench times it: y of the saving
    forward equal bitwise to the fused op's, and the saved backward equal bitwise to the recomputing
    one (which the oracle checks at this size in test_fused_bwd_721x1440_full_size_sampled)."""
    w = WORKLOADS["fused_bf16_721x1440"]
    _log("fused save 721x1440")
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = workload_x(w).to(DEV)
    W = workload_weight(w).to(DEV)
    gy = randn((w.B, w.Co, w.Ho, w.Wo), 3720, "bf16").to(DEV)
    y0 = sgc.disco_fused_conv(h, x, W)
    y, out = sgc.disco_fused_conv_save(h, x, W)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    del y0
    ws = torch.empty(sgc.disco_fused_conv_bwd_workspace(h, w.B, w.C, w.Co), dtype=torch.uint8, device=DEV)
    gx0, dW0 = sgc.disco_fused_conv_bwd(h, x, W, gy, workspace=ws)
    gx, dW = sgc.disco_fused_conv_bwd_saved(h, out, W, gy, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(gx, gx0) and torch.equal(dW, dW0)


def test_fused_save_rejects_bad_arguments():
    """The saving forward and the saved backward validate `out` before anything is enqueued; rejected
    calls leave every output untouched."""
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((1, 4, 31, 64), 3730, "bf16").to(DEV)
    W = randn((8, 4, psi.K), 3731, "bf16").to(DEV)
    gy = randn((1, 8, 31, 64), 3732, "bf16").to(DEV)
    y = nan_like((1, 8, 31, 64), torch.bfloat16)
    out_bad = nan_like((1, 4, psi.K - 1, 31, 64), torch.bfloat16)
    for out, name in ((out_bad, "DISCO_ERR_SHAPE"), (nan_like((1, 4, psi.K, 31, 64), torch.float16), "DISCO_ERR_DTYPE")):
        with pytest.raises(sgc.DiscoError) as e:
            sgc.disco_fused_conv_save(h, x, W, y, out)
        assert e.value.status_name == name
    lib = sgc.load_library()
    descs = [sgc.tensor_desc(t) for t in (x, W, y)]
    st = lib.disco_fused_conv_save(h.handle, *[ctypes.byref(d) for d in descs], None, sgc._stream(DEV))
    assert sgc.STATUS_NAMES[st] == "DISCO_ERR_INVALID_ARGUMENT"
    gx = nan_like((1, 4, 31, 64), torch.bfloat16)
    dW = nan_like((8, 4, psi.K), torch.bfloat16)
    with pytest.raises(sgc.DiscoError) as e:
        sgc.disco_fused_conv_bwd_saved(h, out_bad, W, gy, gx, dW)
    assert e.value.status_name == "DISCO_ERR_SHAPE"
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(y)) and torch.all(torch.isnan(gx)) and torch.all(torch.isnan(dW))


def test_fused_save_f16():
    """fp16 data: the saving fused op's y equals the fused op's bitwise; the kept contraction (fp16 of the
    unscaled accumulator) within the fp16 bar of the oracle's forward."""
    _log("fused save fp16")
    psi = build_psi(33, 128, 17, 64, 0.6, 4, 4)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((1, 6, psi.Hi, psi.Wi), 3740, "f16")
    W = randn((24, 6, psi.K), 3741, "f16", std=0.1)
    y0 = sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV))
    y, out = sgc.disco_fused_conv_save(h, x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert normalised_error(out.cpu(), oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL_F16


# ---------------------------------------------------------------- fp32 fused convolution, fp16 fused backward
# The fp32 fused convolution keeps every step in fp32 (fp32 psi, fp32 contraction chunk, fp32
# matrix-core einsum): the fp32 variant each precision is compared with (bar 1e-5).  The fused
# backward with fp16 data: g = W^T gy, the transpose contraction, the recomputed contraction and dW
# all in fp16 data with fp32 accumulation (bar: the fp16 one).

FUSED_F32_CFGS = [
    # (Hi, Wi, Ho, Wo, theta_c, n_r, n_a, B, C, Co)
    (31, 64, 31, 64, 0.5, 4, 4, 2, 8, 32),      # K=16, p=1, two channel chunks of 4
    (31, 60, 16, 30, 0.6, 3, 1, 1, 23, 20),     # K=3: chunks of 21 + 2 channels, ragged longitude tile
    (19, 144, 19, 72, 0.7, 4, 2, 2, 9, 300),    # K=8, p=2, Co above one block of 256
    (31, 64, 31, 64, 1.5, 4, 4, 1, 6, 33),      # caps spanning whole rings
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("cfg", FUSED_F32_CFGS)
def test_fused_f32_windows_equal_global_reads(cfg, dtype, monkeypatch):
    """The vector-ALU fused kernels (fp32 data; 16-bit data with DISCO_FUSED_MFMA=0) read their sources from
    windows staged in LDS where a latitude's windows fit, and the latitude's psi from an LDS copy where it
    fits (DISCO_FUSED_PSI_LDS=0: psi from memory; DISCO_FUSED_WIN=0: everything from memory); all multiply
    the same values in the same order, so y must be bitwise equal (the configurations include caps
    spanning whole rings)."""
    Hi, Wi, Ho, Wo, tc, n_r, n_a, B, C, Co = cfg
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    h = gpu_psi(psi)
    if dtype != "f32":
        monkeypatch.setenv("DISCO_FUSED_MFMA", "0")
    x = randn((B, C, Hi, Wi), 4200 + C, dtype).to(DEV)
    W = randn((Co, C, psi.K), 4201 + C, dtype, std=1.0 / np.sqrt(C * psi.K)).to(DEV)
    y_lds = sgc.disco_fused_conv(h, x, W)
    monkeypatch.setenv("DISCO_FUSED_PSI_LDS", "0")
    y_win = sgc.disco_fused_conv(h, x, W)
    monkeypatch.setenv("DISCO_FUSED_WIN", "0")
    y_glob = sgc.disco_fused_conv(h, x, W)
    torch.cuda.synchronize()
    assert torch.equal(y_lds, y_glob) and torch.equal(y_win, y_glob)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_with_no_input_channels_writes_zeros(dtype):
    """C = 0: y is an empty sum, so every output is written as zero (fp32 allocates no packed W then)."""
    psi = build_psi(19, 144, 19, 72, 0.7, 4, 2)
    h = gpu_psi(psi)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    x = torch.empty((2, 0, psi.Hi, psi.Wi), dtype=tdt, device=DEV)
    W = torch.empty((40, 0, psi.K), dtype=tdt, device=DEV)
    y = nan_like((2, 40, psi.Ho, psi.Wo), tdt)
    sgc.disco_fused_conv(h, x, W, y)
    torch.cuda.synchronize()
    assert bool((y == 0).all())


@pytest.mark.parametrize("cfg", FUSED_F32_CFGS)
def test_fused_f32_agrees_with_oracle(cfg):
    Hi, Wi, Ho, Wo, tc, n_r, n_a, B, C, Co = cfg
    _log(f"fused fp32 {cfg}")
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    h = gpu_psi(psi)
    x = randn((B, C, Hi, Wi), 4100 + C)
    W = randn((Co, C, psi.K), 4101 + C, std=1.0 / np.sqrt(C * psi.K))
    y = nan_like((B, Co, Ho, Wo), torch.float32)
    sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.fused(psi, x, W)
    nrm = oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)
    assert normalised_error(y, ref, nrm) <= TOL["f32"]


def test_fused_f32_721x1440_sampled():
    """The 721x1440 K=16 filter of the fused workload with fp32 data (4 input, 8 output channels):
    latitudes from pole to pole checked against the oracle."""
    w = WORKLOADS["fused_bf16_721x1440"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = randn((1, 4, psi.Hi, psi.Wi), 4200)
    W = randn((8, 4, psi.K), 4201, std=1.0 / np.sqrt(4 * psi.K))
    _log("fused fp32 721x1440: GPU")
    y = nan_like((1, 8, psi.Ho, psi.Wo), torch.float32)
    sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV), y)
    torch.cuda.synchronize()
    hos = [0, 1, 2, 180, 360, 540, 718, 719, 720]
    _log("fused fp32 721x1440: oracle")
    ref = oracle.fused(psi, x, W, ho_list=hos)
    nrm = oracle.fused(psi, x.abs(), W.abs(), ho_list=hos, abs_mode=True)
    assert normalised_error(y[:, :, hos], ref, nrm) <= TOL["f32"]


def test_fused_f32_save():
    """fp32 data: the saving fused op's y equals the fused op's bitwise, and its kept contraction is
    the fp32 forward (the fused kernel's contraction and the forward sum in different orders)."""
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    h = gpu_psi(psi)
    x = randn((1, 5, psi.Hi, psi.Wi), 4300)
    W = randn((7, 5, psi.K), 4301, std=0.1)
    y0 = sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV))
    y, out = sgc.disco_fused_conv_save(h, x.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert normalised_error(out, oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL["f32"]


@pytest.mark.parametrize("cfg", [
    (31, 64, 31, 64, 0.5, 4, 4, 2, 20, 24),     # K=16, s=1: two channel chunks (16 + 4)
    (19, 144, 19, 72, 0.7, 4, 2, 2, 9, 40),     # K=8, s=2
    (16, 32, 16, 32, 2 * np.pi / 16, 3, 1, 3, 5, 136),  # K=3, B=3, Co above one tile
])
def test_fused_bwd_f16_small_ragged(cfg):
    Hi, Wi, Ho, Wo, tc, nr, na, B, C, Co = cfg
    psi = build_psi(Hi, Wi, Ho, Wo, tc, nr, na)
    _log(f"fused bwd fp16 {cfg}")
    egx, edW, (gx, dW) = _fused_bwd_check(psi, B, C, Co, 4400 + C, "f16")
    assert egx <= TOL_F16, egx
    assert edW <= TOL_F16, edW
    # the training path that keeps the contraction reproduces it bitwise
    x = randn((B, C, psi.Hi, psi.Wi), 4400 + C, "f16").to(DEV)
    W = randn((Co, C, psi.K), 4401 + C, "f16", std=1.0 / np.sqrt(C * psi.K)).to(DEV)
    gy = randn((B, Co, psi.Ho, psi.Wo), 4402 + C, "f16").to(DEV)
    h = gpu_psi(psi)
    _, out = sgc.disco_fused_conv_save(h, x, W)
    gxs, dWs = sgc.disco_fused_conv_bwd_saved(h, out, W, gy)
    torch.cuda.synchronize()
    assert torch.equal(gxs, gx) and torch.equal(dWs, dW)


def test_fused_bwd_f16_721x1440_sampled():
    """The fused workload's backward with fp16 data (B=2, C=Co=256 at 721x1440, K=16): one channel's
    input-gradient planes and weight-gradient column against the oracle."""
    w = WORKLOADS["fused_bf16_721x1440"]
    psi = workload_psi(w)
    h = gpu_psi(psi)
    x = randn((w.B, w.C, w.Hi, w.Wi), 4500, "f16")
    W = randn((w.Co, w.C, w.K), 4501, "f16", std=1.0 / np.sqrt(w.C * w.K))
    gy = randn((w.B, w.Co, psi.Ho, psi.Wo), 4502, "f16")
    _log("fused bwd fp16 721x1440: GPU")
    gx, dW = sgc.disco_fused_conv_bwd(h, x.to(DEV), W.to(DEV), gy.to(DEV))
    torch.cuda.synchronize()
    gx, dW = gx.cpu(), dW.cpu()
    gy64 = gy.double().numpy().reshape(w.B, w.Co, -1)
    W64 = W.double().numpy()
    c = 77
    _log(f"fused bwd fp16 721x1440: oracle channel {c}")
    for b in range(w.B):
        g = (W64[:, c, :].T @ gy64[b]).reshape(1, psi.K, psi.Ho, psi.Wo)
        ga = (np.abs(W64[:, c, :]).T @ np.abs(gy64[b])).reshape(1, psi.K, psi.Ho, psi.Wo)
        ref = oracle.bwd(psi, g.astype(np.float32))
        nrm = oracle.bwd(psi, ga.astype(np.float32), abs_mode=True)
        assert normalised_error(gx[b, c][None], ref, nrm) <= TOL_F16
    out = np.stack([oracle.fwd(psi, x[b, c][None])[0].reshape(psi.K, -1) for b in range(w.B)])
    outa = np.stack([oracle.fwd(psi, x[b, c][None].abs(), abs_mode=True)[0].reshape(psi.K, -1) for b in range(w.B)])
    ref = sum(gy64[b] @ out[b].T for b in range(w.B))
    nrm = sum(np.abs(gy64[b]) @ outa[b].T for b in range(w.B))
    assert normalised_error(dW[:, c, :], ref, nrm) <= TOL_F16


def test_fused_save_more_than_256_output_channels():
    """Co = 512 (two output-channel blocks per latitude span, one of which writes the kept
    contraction): y and the saved backward equal the plain and recomputing calls bitwise."""
    psi = build_psi(24, 64, 24, 64, 0.4, 3, 3)  # K = 9, the page's stand-in basis shape
    h = gpu_psi(psi)
    x = randn((1, 16, psi.Hi, psi.Wi), 4600, "bf16").to(DEV)
    W = randn((512, 16, psi.K), 4601, "bf16", std=1.0 / np.sqrt(16 * psi.K)).to(DEV)
    gy = randn((1, 512, psi.Ho, psi.Wo), 4602, "bf16").to(DEV)
    y0 = sgc.disco_fused_conv(h, x, W)
    y, out = sgc.disco_fused_conv_save(h, x, W)
    gx0, dW0 = sgc.disco_fused_conv_bwd(h, x, W, gy)
    gx, dW = sgc.disco_fused_conv_bwd_saved(h, out, W, gy)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(gx, gx0) and torch.equal(dW, dW0)


def test_outputs_overlapping_inputs_are_refused():
    """Outputs that share bytes with an input are refused (DISCO_ERR_INVALID_ARGUMENT) before
    anything is enqueued, and nothing is written."""
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    h = gpu_psi(psi)
    nx = 2 * 4 * 31 * 64
    buf = torch.full((4 * nx,), 5.0, dtype=torch.bfloat16, device=DEV)
    x = buf[:nx].view(2, 4, 31, 64)
    W = randn((8, 4, psi.K), 4700, "bf16", std=0.1).to(DEV)
    big = torch.full((2 * 4 * psi.K * 31 * 64 + nx,), 5.0, dtype=torch.bfloat16, device=DEV)
    xb = big[:nx].view(2, 4, 31, 64)
    xb.copy_(x)
    out_over_x = big[nx // 2: nx // 2 + 2 * 4 * psi.K * 31 * 64].view(2, 4, psi.K, 31, 64)
    st, msg = _raw("disco_fwd", h.handle, ctypes.byref(sgc.tensor_desc(xb)), ctypes.byref(sgc.tensor_desc(out_over_x)),
                   None)
    assert st == "DISCO_ERR_INVALID_ARGUMENT" and "overlaps" in msg
    # the saving fused op: out overlapping y
    ybuf = torch.full((2 * 8 * 31 * 64 + 2 * 4 * psi.K * 31 * 64,), 5.0, dtype=torch.bfloat16, device=DEV)
    y = ybuf[: 2 * 8 * 31 * 64].view(2, 8, 31, 64)
    out_over_y = ybuf[8: 8 + 2 * 4 * psi.K * 31 * 64].view(2, 4, psi.K, 31, 64)
    st, msg = _raw("disco_fused_conv_save", h.handle, ctypes.byref(sgc.tensor_desc(x)),
                   ctypes.byref(sgc.tensor_desc(W)), ctypes.byref(sgc.tensor_desc(y)),
                   ctypes.byref(sgc.tensor_desc(out_over_y)), None)
    assert st == "DISCO_ERR_INVALID_ARGUMENT" and "overlaps" in msg
    # the fused backward: gx overlapping gy
    gbuf = torch.full((2 * 8 * 31 * 64 + nx,), 5.0, dtype=torch.bfloat16, device=DEV)
    gy = gbuf[: 2 * 8 * 31 * 64].view(2, 8, 31, 64)
    gx_over_gy = gbuf[64: 64 + nx].view(2, 4, 31, 64)
    dW = torch.full((8, 4, psi.K), 5.0, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(sgc.disco_fused_conv_bwd_workspace(h, 2, 4, 8), dtype=torch.uint8, device=DEV)
    lib = sgc.load_library()
    stc = lib.disco_fused_conv_bwd(h.handle, *[ctypes.byref(sgc.tensor_desc(t)) for t in (x, W, gy, gx_over_gy, dW)],
                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert sgc.STATUS_NAMES[stc] == "DISCO_ERR_INVALID_ARGUMENT" and "overlaps" in lib.disco_last_error().decode()
    torch.cuda.synchronize()
    assert bool((big[nx:] == 5.0).all()) and bool((ybuf == 5.0).all()) and bool((gbuf == 5.0).all())
    assert bool((dW == 5.0).all())


def test_oversized_launch_is_refused_and_writes_nothing(monkeypatch):
    """A launch whose LDS request exceeds the device's per-workgroup LDS is refused on the host
    (DISCO_ERR_HIP) before anything is dispatched, and its output is untouched; the next call with a
    fitting request runs normally.  DISCO_TEST_LDS_EXTRA inflates the request of every kernel that asks
    for dynamic LDS (the matrix-core kernels, the fp32 tiled gather and the fp32 fused kernel) by 1 MiB."""
    psi = build_psi(19, 144, 19, 72, 0.7, 4, 2)  # a shape the matrix-core kernels and the fp32 kernels cover
    h = gpu_psi(psi)
    x = randn((2, 5, 19, 144), 4800, "bf16").to(DEV)
    x32 = randn((2, 5, 19, 144), 4802, "f32").to(DEV)
    W = randn((40, 5, psi.K), 4801, "bf16", std=0.2).to(DEV)
    W32 = randn((40, 5, psi.K), 4803, "f32", std=0.2).to(DEV)
    ref_y = sgc.disco_fused_conv(h, x, W)
    ref_o = sgc.disco_fwd(h, x)
    ref_o32 = sgc.disco_fwd(h, x32)
    ref_y32 = sgc.disco_fused_conv(h, x32, W32)
    torch.cuda.synchronize()
    monkeypatch.setenv("DISCO_TEST_LDS_EXTRA", str(1 << 20))
    y = nan_like((2, 40, 19, 72), torch.bfloat16)
    o = nan_like((2, 5, psi.K, 19, 72), torch.bfloat16)
    o32 = nan_like((2, 5, psi.K, 19, 72), torch.float32)
    y32 = nan_like((2, 40, 19, 72), torch.float32)
    for call in (lambda: sgc.disco_fused_conv(h, x, W, y), lambda: sgc.disco_fwd(h, x, o),
                 lambda: sgc.disco_fwd(h, x32, o32), lambda: sgc.disco_fused_conv(h, x32, W32, y32)):
        with pytest.raises(sgc.DiscoError) as ei:
            call()
        assert ei.value.status_name == "DISCO_ERR_HIP"
    torch.cuda.synchronize()
    for t in (y, o, o32, y32):
        assert bool(torch.isnan(t).all())
    monkeypatch.delenv("DISCO_TEST_LDS_EXTRA")
    sgc.disco_fused_conv(h, x, W, y)
    sgc.disco_fwd(h, x, o)
    sgc.disco_fwd(h, x32, o32)
    sgc.disco_fused_conv(h, x32, W32, y32)
    torch.cuda.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(o, ref_o) and torch.equal(o32, ref_o32) and torch.equal(y32, ref_y32)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_with_packed_w_equals_elementwise_w_staging(dtype, monkeypatch):
    """K < 16: the fused op packs W into 16-element rows in a stream-ordered temporary and loads its W
    slices as 16-byte runs; DISCO_PACK_W=0 keeps the element-wise staging.  Both multiply the same values
    in the same order, so y (and the kept contraction) must be bitwise equal, and match the oracle; two
    output-channel blocks (Co = 300) and a ragged channel count."""
    psi = build_psi(19, 144, 19, 72, 0.7, 3, 3)  # K = 9
    assert psi.K == 9
    h = gpu_psi(psi)
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    x = randn((2, 7, 19, 144), 4900, dtype).to(DEV)
    W = randn((300, 7, 9), 4901, dtype, std=0.2).to(DEV)
    y_pack, o_pack = sgc.disco_fused_conv_save(h, x, W)
    torch.cuda.synchronize()
    monkeypatch.setenv("DISCO_PACK_W", "0")
    y_elem, o_elem = sgc.disco_fused_conv_save(h, x, W)
    torch.cuda.synchronize()
    monkeypatch.delenv("DISCO_PACK_W")
    assert y_pack.dtype == td
    assert torch.equal(y_pack, y_elem) and torch.equal(o_pack, o_elem)
    xc, Wc = x.cpu(), W.cpu()
    ref = oracle.fused(psi, xc, Wc)
    nrm = oracle.fused(psi, xc.abs(), Wc.abs(), abs_mode=True)
    assert normalised_error(y_pack, ref, nrm) <= (2e-3 if dtype == "f16" else TOL["bf16"])
    y2 = sgc.disco_fused_conv(h, x, W)  # the plain op takes the same path
    torch.cuda.synchronize()
    assert torch.equal(y2, y_pack)


@pytest.mark.parametrize("cfg", [(2, 5, 40, 3, 7, 37, "bf16"), (2, 9, 300, 8, 5, 48, "bf16"), (1, 12, 256, 9, 4, 96, "f16")])
def test_einsum_with_packed_w_equals_elementwise_w_staging(cfg, monkeypatch):
    """K < 16: disco_einsum packs W into 16-element rows (stream-ordered temporary) and takes the direct
    W-slice loads; DISCO_PACK_W=0 keeps the element-wise staging.  Same values, same order: bitwise equal."""
    B, C, Co, K, Ho, Wo, dt = cfg
    t = randn((B, C, K, Ho, Wo), 3300 + C, dt).to(DEV)
    W = randn((Co, C, K), 3400 + C, dt, std=1.0 / np.sqrt(C * K)).to(DEV)
    y_pack = sgc.disco_einsum(W, t)
    torch.cuda.synchronize()
    monkeypatch.setenv("DISCO_PACK_W", "0")
    y_elem = sgc.disco_einsum(W, t)
    torch.cuda.synchronize()
    monkeypatch.delenv("DISCO_PACK_W")
    assert torch.equal(y_pack, y_elem)
    ref = oracle.einsum(W.cpu(), t.cpu())
    nrm = oracle.einsum(W.cpu().abs(), t.cpu().abs(), abs_mode=True)
    assert normalised_error(y_pack.cpu(), ref, nrm) <= TOL_EIN[dt]


@pytest.mark.parametrize("mfma", ["1", "0"])
def test_latitudes_without_psi_entries_get_zero_contractions(mfma, monkeypatch):
    """An output latitude whose psi rows are all empty has no plan pieces: the fused op's saved contraction
    and the fused backward's recomputed contraction are still written there (zeros), whatever the outputs
    and the workspace held before (NaN fills); on the matrix-core kernels and with DISCO_FUSED_MFMA=0."""
    monkeypatch.setenv("DISCO_FUSED_MFMA", mfma)
    K, Ho, Wo = 4, 12, 64
    empty = [k * Ho + 5 for k in range(K)]  # latitude 5: no entries in any basis row
    psi = random_psi(K, Ho, Wo, Ho, Wo, 0.004, seed=77, empty_rows=empty)
    h = gpu_psi(psi)
    B, C, Co = 1, 6, 16
    x = randn((B, C, Ho, Wo), 1900, "bf16")
    W = randn((Co, C, K), 1901, "bf16", std=0.3)
    gy = randn((B, Co, Ho, Wo), 1902, "bf16")
    y = nan_like((B, Co, Ho, Wo), torch.bfloat16)
    out = nan_like((B, C, K, Ho, Wo), torch.bfloat16)
    sgc.disco_fused_conv_save(h, x.to(DEV), W.to(DEV), y, out)
    ws = torch.full((sgc.disco_fused_conv_bwd_workspace(h, B, C, Co),), 0xFF, dtype=torch.uint8, device=DEV)
    gx, dW = sgc.disco_fused_conv_bwd(h, x.to(DEV), W.to(DEV), gy.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    assert bool((out[:, :, :, 5] == 0).all()) and bool((y[:, :, 5] == 0).all())
    assert normalised_error(out.cpu(), oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= TOL["bf16"]
    assert normalised_error(y.cpu(), oracle.fused(psi, x, W), oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)) <= TOL["bf16"]
    rgx, rdW = oracle.fused_bwd(psi, x, W, gy)
    ngx, ndW = oracle.fused_bwd(psi, x, W, gy, abs_mode=True)
    assert normalised_error(gx.cpu(), rgx, ngx) <= TOL["bf16"]
    assert normalised_error(dW.cpu(), rdW, ndW) <= TOL["bf16"]


def _random_case(seed, k_range=None):
    """A random small problem: sparse random psi (some rows empty), s in {1, 2}, ragged sizes."""
    rng = np.random.default_rng(seed)
    K = int(rng.integers(*(k_range or (1, 21))))  # K > 16: the vector-ALU fused kernel
    s = int(rng.integers(1, 3))
    Ho = int(rng.integers(1, 10))
    Wo = int(rng.choice([8, 16, 24, 40, 64, 72, 96, 264]))
    Hi = int(rng.integers(1, 12))
    Wi = s * Wo
    empty = tuple(int(r) for r in rng.choice(K * Ho, size=min(K * Ho, int(rng.integers(0, 4))), replace=False))
    psi = random_psi(K, Ho, Wo, Hi, Wi, float(rng.uniform(0.002, 0.05)), seed=seed, empty_rows=empty)
    B = int(rng.integers(1, 3))
    C = int(rng.integers(1, 11))
    Co = 8 * int(rng.integers(1, 6))
    dt = str(rng.choice(["bf16", "bf16", "f16", "f32"]))
    return psi, B, C, Co, dt


def test_fused_bwd_overlap_equals_one_stream(monkeypatch):
    """The recomputing backward runs its contraction and dW products on a second stream beside the gx
    launch; DISCO_BWD_OVERLAP=0 keeps them on the caller's stream.  Two channel chunks (K = 16, 70
    channels), the workspace reused across calls: both orders give the same bits, and against the oracle."""
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)
    assert psi.K == 16
    _log("fused bwd overlap vs one stream")
    egx, edW, (gx_a, dW_a) = _fused_bwd_check(psi, 2, 70, 24, 1700)
    assert egx <= TOL["bf16"] and edW <= TOL["bf16"], (egx, edW)
    monkeypatch.setenv("DISCO_BWD_OVERLAP", "0")
    _, _, (gx_b, dW_b) = _fused_bwd_check(psi, 2, 70, 24, 1700)
    monkeypatch.delenv("DISCO_BWD_OVERLAP")
    assert torch.equal(gx_a, gx_b) and torch.equal(dW_a, dW_b)
    h = gpu_psi(psi)
    x = randn((2, 70, 31, 64), 1701, "bf16").to(DEV)
    W = randn((24, 70, psi.K), 1702, "bf16", std=0.05).to(DEV)
    gy = randn((2, 24, 31, 64), 1703, "bf16").to(DEV)
    ws = torch.full((sgc.disco_fused_conv_bwd_workspace(h, 2, 70, 24),), 0x7f, dtype=torch.uint8, device=DEV)
    runs = [sgc.disco_fused_conv_bwd(h, x, W, gy, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r[0], runs[0][0]) and torch.equal(r[1], runs[0][1])


@pytest.mark.parametrize("seed", list(range(5000, 5100)))
def test_random_problems_every_op_against_the_oracle(seed):
    """Seeded random problems through fwd, bwd, the fused op (plain and saving), its backward (recomputing
    and saved) and the einsum, each against the fp64 oracle, outputs NaN-filled beforehand (fp32 data: the
    ops that take it)."""
    _random_problem(seed)


RANDOM_PATH_KNOBS = {
    "vector-ALU fused": {"DISCO_FUSED_MFMA": "0"},
    "vector-ALU fwd and bwd": {"DISCO_FWD_MFMA": "0", "DISCO_BWD_MFMA": "0"},
    "staged fp32 gathers": {"DISCO_TILE": "0"},
    "plain gathers": {"DISCO_TILE": "0", "DISCO_STAGED": "0", "DISCO_FWD_MFMA": "0", "DISCO_BWD_MFMA": "0"},
    "gx through W^T gy": {"DISCO_BWD_FUSED": "0"},
    "fused backward on one stream": {"DISCO_BWD_OVERLAP": "0"},
    "element-wise W staging": {"DISCO_PACK_W": "0"},
    "one realigned psi copy": {"DISCO_PSI_COPIES": "1"},
    "two psi copies": {"DISCO_PSI_COPIES": "2"},
}


@pytest.mark.parametrize("path", sorted(RANDOM_PATH_KNOBS))
@pytest.mark.parametrize("seed", list(range(5100, 5125)))
def test_random_problems_on_every_kernel_path(seed, path, monkeypatch):
    """The random problems again with each kernel-path knob (a fresh psi handle, so that the knobs read
    when the plans are built apply too)."""
    for k, v in RANDOM_PATH_KNOBS[path].items():
        monkeypatch.setenv(k, v)
    _random_problem(seed, fresh=True)


@pytest.mark.parametrize("seed", list(range(5200, 5208)))
def test_random_problems_with_many_channels(seed):
    """The random problems with 60-200 input channels and K = 8..16: several channel chunks in the fused
    kernel and in the fused backward's recomputed contraction (64-128 channels per chunk at these K)."""
    rng = np.random.default_rng(seed)
    _random_problem(seed, channels=int(rng.integers(60, 201)), k_range=(8, 17))


def _random_problem(seed, fresh=False, channels=None, k_range=None):
    psi, B, C, Co, dt = _random_case(seed, k_range)
    if channels is not None:
        C = channels
    _log(f"random problem seed={seed} K={psi.K} {psi.Ho}x{psi.Wo} <- {psi.Hi}x{psi.Wi} B={B} C={C} Co={Co} {dt}")
    tol = {"f16": TOL_F16, "bf16": TOL["bf16"], "f32": TOL["f32"]}[dt]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]
    f32 = dt == "f32"
    err = normalised_error_f16 if dt == "f16" else normalised_error  # random psi reaches fp16 subnormals
    h = sgc.disco_psi_create(psi, 0) if fresh else gpu_psi(psi)
    x = randn((B, C, psi.Hi, psi.Wi), seed + 1, dt)
    g = randn((B, C, psi.K, psi.Ho, psi.Wo), seed + 2, dt)
    W = randn((Co, C, psi.K), seed + 3, dt, std=1.0 / np.sqrt(C * psi.K))
    gy = randn((B, Co, psi.Ho, psi.Wo), seed + 4, dt)
    out = nan_like((B, C, psi.K, psi.Ho, psi.Wo), tdt)
    gx = nan_like((B, C, psi.Hi, psi.Wi), tdt)
    y = nan_like((B, Co, psi.Ho, psi.Wo), tdt)
    ys = nan_like((B, Co, psi.Ho, psi.Wo), tdt)
    kept = nan_like((B, C, psi.K, psi.Ho, psi.Wo), tdt)
    sgc.disco_fwd(h, x.to(DEV), out)
    sgc.disco_bwd(h, g.to(DEV), gx)
    sgc.disco_fused_conv(h, x.to(DEV), W.to(DEV), y)
    sgc.disco_fused_conv_save(h, x.to(DEV), W.to(DEV), ys, kept)
    if not f32:
        fgx, fdW = sgc.disco_fused_conv_bwd(h, x.to(DEV), W.to(DEV), gy.to(DEV))
        sgx, sdW = sgc.disco_fused_conv_bwd_saved(h, kept, W.to(DEV), gy.to(DEV))
    ye = sgc.disco_einsum(W.to(DEV), g.to(DEV)) if psi.K <= 16 and not f32 else None
    torch.cuda.synchronize()
    assert err(out.cpu(), oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= tol
    assert err(gx.cpu(), oracle.bwd(psi, g), oracle.bwd(psi, g.abs(), abs_mode=True)) <= tol
    ry, ny = oracle.fused(psi, x, W), oracle.fused(psi, x.abs(), W.abs(), abs_mode=True)
    assert err(y.cpu(), ry, ny) <= tol
    assert torch.equal(ys, y)
    assert err(kept.cpu(), oracle.fwd(psi, x), oracle.fwd(psi, x.abs(), abs_mode=True)) <= tol
    if not f32:
        rgx, rdW = oracle.fused_bwd(psi, x, W, gy)
        ngx, ndW = oracle.fused_bwd(psi, x, W, gy, abs_mode=True)
        for gxx, dww in ((fgx, fdW), (sgx, sdW)):
            assert err(gxx.cpu(), rgx, ngx) <= tol
            assert err(dww.cpu(), rdW, ndW) <= tol
    if ye is not None:
        assert err(ye.cpu(), oracle.einsum(W, g), oracle.einsum(W.abs(), g.abs(), abs_mode=True)) <= tol
    if fresh:
        h.close()

"""The backward of the fused convolution through disco_fused_conv_bwd_noalloc, the entry point that
allocates nothing (its workspace is the library's per-device scratch array), called through the C
ABI and checked against disco_fused_conv_bwd (bitwise) and the fp64 oracle (bf16 bar, 2e-2 of the
normaliser), on two calls in a row, the second with a smaller input; and its refusal of a shape
whose workspace does not fit the array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_gather_contraction_amd as sgc
from disco_inputs import randn
from disco_inputs.psi import build_psi, random_psi

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
BAR = 2e-2


def _err(gpu, ref, nrm):
    g = gpu.double().cpu().numpy()
    zero = nrm == 0
    assert np.all(g[zero] == 0)
    return float(np.max(np.abs(g - ref)[~zero] / nrm[~zero])) if np.any(~zero) else 0.0


def _noalloc(h, x, W, gy, gx, dW):
    lib = sgc.load_library()
    d = [sgc.tensor_desc(t) for t in (x, W, gy, gx, dW)]
    st = lib.disco_fused_conv_bwd_noalloc(h.handle, *[ctypes.byref(v) for v in d],
                                          ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    return sgc.STATUS_NAMES[st], lib.disco_last_error().decode()


def test_noalloc_backward_matches_the_workspace_entry_point_twice():
    psi = build_psi(31, 64, 31, 64, 0.5, 4, 4)  # K = 16, s = 1
    h = sgc.disco_psi_create(psi, 0)
    for call, (B, C, Co, seed) in enumerate([(2, 20, 24, 7100), (1, 6, 8, 7200)]):  # second call smaller
        print(f"[no-alloc] call {call}: B={B} C={C} Co={Co}", flush=True)
        x = randn((B, C, psi.Hi, psi.Wi), seed, "bf16")
        W = randn((Co, C, psi.K), seed + 1, "bf16", std=1 / np.sqrt(C * psi.K))
        gy = randn((B, Co, psi.Ho, psi.Wo), seed + 2, "bf16")
        xd, Wd, gyd = x.to(DEV), W.to(DEV), gy.to(DEV)
        gx = torch.full_like(xd, float("nan"))
        dW = torch.full_like(Wd, float("nan"))
        st, msg = _noalloc(h, xd, Wd, gyd, gx, dW)
        assert st == "DISCO_OK", msg
        gx_ref, dW_ref = sgc.disco_fused_conv_bwd(h, xd, Wd, gyd)
        torch.cuda.synchronize()
        assert torch.equal(gx, gx_ref) and torch.equal(dW, dW_ref)
        rgx, rdW = oracle.fused_bwd(psi, x, W, gy)
        ngx, ndW = oracle.fused_bwd(psi, x, W, gy, abs_mode=True)
        assert _err(gx, rgx, ngx) <= BAR and _err(dW, rdW, ndW) <= BAR
    h.close()


def test_noalloc_backward_refuses_a_workspace_beyond_its_array():
    # 256 x 512 output positions, 256 output channels, Wi = 2 Wo (gx through W^T gy): gy^T alone is
    # 64 MiB, beyond the 64 MiB array
    psi = random_psi(1, 256, 512, 256, 1024, 2e-6, seed=31)
    h = sgc.disco_psi_create(psi, 0)
    x = torch.zeros((1, 2, psi.Hi, psi.Wi), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((256, 2, psi.K), dtype=torch.bfloat16, device=DEV)
    gy = torch.zeros((1, 256, psi.Ho, psi.Wo), dtype=torch.bfloat16, device=DEV)
    gx = torch.full_like(x, 3.0)
    dW = torch.full_like(W, 3.0)
    st, msg = _noalloc(h, x, W, gy, gx, dW)
    torch.cuda.synchronize()
    assert st == "DISCO_ERR_SHAPE" and "scratch" in msg, (st, msg)
    assert bool((gx == 3.0).all()) and bool((dW == 3.0).all())
    h.close()


def test_noalloc_backward_fits_where_gx_takes_the_transposed_psi():
    # the same positions with Wi = Wo: gx is one fused launch over the transposed psi, no gy^T is kept,
    # and the shape fits the array
    psi = random_psi(1, 256, 512, 256, 512, 2e-6, seed=31)
    h = sgc.disco_psi_create(psi, 0)
    x = randn((1, 2, psi.Hi, psi.Wi), 3901, "bf16").to(DEV)
    W = randn((256, 2, psi.K), 3902, "bf16", std=0.5).to(DEV)
    gy = randn((1, 256, psi.Ho, psi.Wo), 3903, "bf16").to(DEV)
    gx = torch.full_like(x, 3.0)
    dW = torch.full_like(W, 3.0)
    st, msg = _noalloc(h, x, W, gy, gx, dW)
    assert st == "DISCO_OK", (st, msg)
    rgx, rdW = sgc.disco_fused_conv_bwd(h, x, W, gy)
    torch.cuda.synchronize()
    assert torch.equal(gx, rgx) and torch.equal(dW, rdW)
    h.close()

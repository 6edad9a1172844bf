"""Pins of the fp64 oracle against facts fixed independently of it.

The DISCO page (torch-harmonics "disco-kernel-dev", section "Architecture
snapshot") names the three operations — CSR contraction to the K-expanded
output, its transpose, and contraction + channel/basis einsum — but prints no
values.  Each pin below is chosen so that a plausible slip in the oracle (a
wrong shift sign, a dropped subsampling factor, a transposed operand, a
missing term) fails at least one of them:

* hand-worked fixture (tests/golden/hand_tiny.json);
* dense brute force: the basis evaluated directly at every output longitude,
  contracted with numpy einsum (pins the shift direction and the s*wo stride);
* constant field -> psi row sums;
* longitude equivariance: rolling x by s columns rolls the output by one;
* adjoint identity <F x, g> = <x, F^T g> (pins the backward against the forward);
* same-latitude psi -> numpy FFT circular cross-correlation, subsampled by s;
* one-entry identity psi -> strided subsample, and fused -> numpy matmul;
* linearity in x and in the values;
* einsum alone: einsum of the forward oracle reproduces the fused oracle
  bitwise, the hand-worked fixture's fused values, and K = 1 -> numpy matmul;
* fused backward: unit directional derivatives of the fused oracle, the dense
  basis, and <gy, y> = <x, gx> = <W, dW>.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from disco_inputs import WORKLOADS, randn, workload_psi
from disco_inputs.psi import (PsiCSR, basis_values, build_psi, equiangular_colatitudes, grid_colatitudes,
                              grid_quadrature, quadrature_weights,
                              random_psi)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _psi_from_dict(d):
    return PsiCSR(d["K"], d["Ho"], d["Wo"], d["Hi"], d["Wi"], np.array(d["row_ptr"], np.int64),
                  np.array(d["col_hi"], np.int32), np.array(d["col_wi"], np.int32), np.array(d["val"], np.float32))


def test_hand_worked_fixture():
    d = json.load(open(os.path.join(GOLDEN, "hand_tiny.json")))
    psi = _psi_from_dict(d)
    x = np.array(d["x"], np.float32)[None, None]
    np.testing.assert_array_equal(oracle.fwd(psi, x)[0, 0], np.array(d["out"]))
    gout = np.array(d["gout"], np.float32)[None, None]
    np.testing.assert_array_equal(oracle.bwd(psi, gout)[0, 0], np.array(d["gx"]))
    W = np.array(d["W"], np.float32)
    np.testing.assert_array_equal(oracle.fused(psi, x, W)[0], np.array(d["y"]))


def _dense_operator(Hi, Wi, Ho, Wo, theta_c, n_r, n_a, grid_in="equiangular", grid_out="equiangular"):
    """D[k, ho, wo, hi, wi]: basis evaluated at the true output longitude 2*pi*wo/Wo.

    The longitude difference is taken from the integer (wi - s*wo) mod Wi, so
    membership is decided exactly as in the CSR built for output longitude 0.
    """
    s = Wi // Wo
    ti, to = grid_colatitudes(grid_in, Hi), grid_colatitudes(grid_out, Ho)
    q = grid_quadrature(grid_in, Hi, Wi)
    K = n_r * n_a
    D = np.zeros((K, Ho, Wo, Hi, Wi))
    wi = np.arange(Wi)
    for ho in range(Ho):
        for wo in range(Wo):
            dphi = 2 * np.pi * ((wi[None, :] - s * wo) % Wi) / Wi
            vals, hats = basis_values(to[ho], ti[:, None], dphi, theta_c, n_r, n_a, q[:, None])
            for m in range(n_r):
                keep = (hats[m] > 0) & (q[:, None] > 0)
                for a in range(n_a):
                    k = m * n_a + a
                    D[k, ho, wo] = np.where(keep, vals[k].astype(np.float32).astype(np.float64), 0.0)
    return D


@pytest.mark.parametrize("geom", [
    (16, 32, 16, 32, 2 * math.pi / 16, 3, 1),
    (13, 24, 7, 12, 0.6, 2, 2),
    (9, 16, 9, 8, 0.9, 2, 4),
])
def test_dense_brute_force(geom):
    Hi, Wi, Ho, Wo, tc, n_r, n_a = geom
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    D = _dense_operator(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    x = randn((2, 3, Hi, Wi), 7).numpy()
    g = randn((2, 3, psi.K, Ho, Wo), 8).numpy()
    ref_out = np.einsum("kowhv,bchv->bckow", D, x.astype(np.float64))
    ref_gx = np.einsum("kowhv,bckow->bchv", D, g.astype(np.float64))
    out = oracle.fwd(psi, x)
    gx = oracle.bwd(psi, g)
    assert np.abs(out - ref_out).max() <= 1e-12 * max(1.0, np.abs(ref_out).max())
    assert np.abs(gx - ref_gx).max() <= 1e-12 * max(1.0, np.abs(ref_gx).max())
    W = randn((5, 3, psi.K), 9).numpy()
    ref_y = np.einsum("ock,bckhw->bohw", W.astype(np.float64), ref_out)
    y = oracle.fused(psi, x, W)
    assert np.abs(y - ref_y).max() <= 1e-12 * max(1.0, np.abs(ref_y).max())


def test_constant_field_gives_row_sums():
    psi = workload_psi(WORKLOADS["fwdbwd_f32_181x360"])
    x = np.ones((1, 1, psi.Hi, psi.Wi), np.float32)
    out = oracle.fwd(psi, x)[0, 0]
    rs = np.add.reduceat(psi.val.astype(np.float64), psi.row_ptr[:-1]) if psi.nnz else None
    rs = np.where(np.diff(psi.row_ptr) > 0, rs, 0.0).reshape(psi.K, psi.Ho)
    np.testing.assert_allclose(out, np.broadcast_to(rs[:, :, None], out.shape), rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("name", ["tiny_fwd_f32_16x32", "fwdbwd_f32_181x360"])
def test_longitude_equivariance_bitwise(name):
    w = WORKLOADS[name]
    psi = workload_psi(w)
    s = psi.pscale
    x = randn((1, 2, psi.Hi, psi.Wi), 11).numpy()
    out = oracle.fwd(psi, x)
    out_r = oracle.fwd(psi, np.roll(x, s, axis=-1))
    np.testing.assert_array_equal(out_r, np.roll(out, 1, axis=-1))


@pytest.mark.parametrize("name", ["tiny_fwd_f32_16x32", "fwdbwd_f32_181x360"])
def test_adjoint_identity(name):
    psi = workload_psi(WORKLOADS[name])
    x = randn((2, 3, psi.Hi, psi.Wi), 12).numpy()
    g = randn((2, 3, psi.K, psi.Ho, psi.Wo), 13).numpy()
    lhs = float(np.sum(oracle.fwd(psi, x) * g))
    rhs = float(np.sum(x.astype(np.float64) * oracle.bwd(psi, g)))
    scale = float(np.sum(oracle.fwd(psi, np.abs(x), abs_mode=True) * np.abs(g)))
    assert abs(lhs - rhs) <= 1e-13 * scale


def test_adjoint_identity_random_psi():
    psi = random_psi(3, 5, 6, 7, 18, 0.2, seed=3, empty_rows=(2, 7))
    x = randn((1, 2, 7, 18), 14).numpy()
    g = randn((1, 2, 3, 5, 6), 15).numpy()
    lhs = float(np.sum(oracle.fwd(psi, x) * g))
    rhs = float(np.sum(x.astype(np.float64) * oracle.bwd(psi, g)))
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1.0)


@pytest.mark.parametrize("s", [1, 2, 3])
def test_same_latitude_psi_is_fft_correlation(s):
    H, Wi = 6, 24
    Wo = Wi // s
    rng = np.random.default_rng(s)
    filt = np.zeros((H, Wi), np.float32)
    hs, ws, vs = [], [], []
    for h in range(H):
        cols = np.sort(rng.choice(Wi, size=5, replace=False))
        v = rng.standard_normal(5).astype(np.float32)
        filt[h, cols] = v
        hs += [h] * 5
        ws += list(cols)
        vs += list(v)
    psi = PsiCSR(1, H, Wo, H, Wi, np.arange(0, 5 * H + 1, 5, dtype=np.int64), np.array(hs, np.int32),
                 np.array(ws, np.int32), np.array(vs, np.float32))
    x = randn((1, 1, H, Wi), 16).numpy()
    out = oracle.fwd(psi, x)[0, 0, 0]
    # out[h, wo] = sum_j f[h, j] * x[h, j + s*wo]  ==  cross-correlation at lag s*wo
    corr = np.fft.irfft(np.conj(np.fft.rfft(filt.astype(np.float64), axis=-1)) *
                        np.fft.rfft(x[0, 0].astype(np.float64), axis=-1), n=Wi, axis=-1)
    np.testing.assert_allclose(out, corr[:, ::s], rtol=0, atol=1e-12)


def test_identity_psi_subsample_and_fused_matmul():
    Hi, Wi, Ho, Wo = 9, 20, 5, 10  # latitude stride 2, longitude stride 2
    rows = np.arange(Ho + 1, dtype=np.int64)
    psi = PsiCSR(1, Ho, Wo, Hi, Wi, rows, (2 * np.arange(Ho)).astype(np.int32), np.zeros(Ho, np.int32),
                 np.ones(Ho, np.float32))
    x = randn((2, 4, Hi, Wi), 17).numpy()
    out = oracle.fwd(psi, x)
    np.testing.assert_array_equal(out[:, :, 0], x[:, :, ::2, ::2].astype(np.float64))
    W = randn((3, 4, 1), 18).numpy()
    y = oracle.fused(psi, x, W)
    ref = np.stack([W[:, :, 0].astype(np.float64) @ x[b, :, ::2, ::2].reshape(4, -1) for b in range(2)])
    np.testing.assert_allclose(y.reshape(2, 3, -1), ref, rtol=1e-13, atol=1e-13)


def test_linearity():
    psi = random_psi(2, 4, 8, 6, 16, 0.3, seed=5)
    rng = np.random.default_rng(19)
    # small integers: the combination 0.5*x1 + 0.25*x2 is exact in fp32
    x1 = rng.integers(-8, 9, (1, 1, 6, 16)).astype(np.float64)
    x2 = rng.integers(-8, 9, (1, 1, 6, 16)).astype(np.float64)
    a = oracle.fwd(psi, (0.5 * x1 + 0.25 * x2).astype(np.float32))
    b = 0.5 * oracle.fwd(psi, x1.astype(np.float32)) + 0.25 * oracle.fwd(psi, x2.astype(np.float32))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    psi2 = PsiCSR(psi.K, psi.Ho, psi.Wo, psi.Hi, psi.Wi, psi.row_ptr, psi.col_hi, psi.col_wi, psi.val * 2)
    np.testing.assert_array_equal(oracle.fwd(psi2, x1.astype(np.float32)), 2 * oracle.fwd(psi, x1.astype(np.float32)))


def test_empty_rows_are_zero_and_normaliser_nonnegative():
    psi = random_psi(2, 3, 4, 5, 8, 0.3, seed=6, empty_rows=(0, 4))
    x = randn((1, 2, 5, 8), 21).numpy()
    out = oracle.fwd(psi, x)
    assert np.all(out[:, :, 0, 0] == 0.0) and np.all(out[:, :, 1, 1] == 0.0)
    n = oracle.fwd(psi, x, abs_mode=True)
    assert np.all(n >= np.abs(out))


def test_fused_matches_einsum_of_forward():
    psi = random_psi(3, 4, 6, 5, 12, 0.25, seed=7)
    x = randn((2, 3, 5, 12), 22).numpy()
    W = randn((4, 3, 3), 23).numpy()
    out = oracle.fwd(psi, x)
    ref = np.einsum("ock,bckhw->bohw", W.astype(np.float64), out)
    np.testing.assert_allclose(oracle.fused(psi, x, W), ref, rtol=1e-13, atol=1e-13)
    # ho subset
    np.testing.assert_allclose(oracle.fused(psi, x, W, ho_list=[3, 1]), ref[:, :, [3, 1]], rtol=1e-13, atol=1e-13)



def test_einsum_of_forward_is_fused_bitwise():
    # the fused oracle is pinned on its own (dense brute force, fixture, matmul special case)
    psi = random_psi(3, 4, 6, 5, 12, 0.25, seed=7)
    x = randn((2, 3, 5, 12), 22).numpy()
    W = randn((4, 3, 3), 23).numpy()
    np.testing.assert_array_equal(oracle.einsum(W, oracle.fwd(psi, x)), oracle.fused(psi, x, W))
    n = oracle.einsum(W, oracle.fwd(psi, x, abs_mode=True), abs_mode=True)
    np.testing.assert_array_equal(n, oracle.fused(psi, x, W, abs_mode=True))


def test_einsum_hand_worked_fixture():
    d = json.load(open(os.path.join(GOLDEN, "hand_tiny.json")))
    out = np.array(d["out"], np.float64)[None, None]
    y = oracle.einsum(np.array(d["W"], np.float32), out)
    np.testing.assert_array_equal(y[0], np.array(d["y"]))


def test_einsum_single_basis_is_matmul():
    t = randn((2, 5, 1, 3, 7), 24).numpy()
    W = randn((6, 5, 1), 25).numpy()
    ref = np.stack([W[:, :, 0].astype(np.float64) @ t[b, :, 0].reshape(5, -1).astype(np.float64) for b in range(2)])
    np.testing.assert_allclose(oracle.einsum(W, t).reshape(2, 6, -1), ref, rtol=1e-13, atol=1e-13)
    # a transposed W (o and c swapped) would not even have this shape; check a non-symmetric square case too
    W2 = randn((5, 5, 1), 26).numpy()
    ref2 = np.stack([W2[:, :, 0].astype(np.float64) @ t[b, :, 0].reshape(5, -1).astype(np.float64) for b in range(2)])
    np.testing.assert_allclose(oracle.einsum(W2, t).reshape(2, 5, -1), ref2, rtol=1e-13, atol=1e-13)

# ---- backward of the fused convolution -------------------------------------------------------
# y = einsum(W, F x) is linear in x and in W, so <gy, y> has gradients
# gx = F^T (W^T gy) and dW = sum gy * (F x); each is fixed by evaluating the (separately pinned)
# fused oracle along unit directions, by the dense basis, and by the adjoint identities.

def test_fused_bwd_unit_directions():
    psi = random_psi(3, 4, 6, 5, 12, 0.25, seed=17, empty_rows=(1,))
    B, C, Co = 2, 3, 4
    x = randn((B, C, 5, 12), 41).numpy()
    W = randn((Co, C, 3), 42).numpy()
    gy = randn((B, Co, 4, 6), 43).numpy()
    gx, dW = oracle.fused_bwd(psi, x, W, gy)
    g64 = gy.astype(np.float64)
    ref_gx = np.zeros_like(gx)
    for b in range(B):
        for c in range(C):
            for hi in range(5):
                for wi in range(12):
                    e = np.zeros_like(x)
                    e[b, c, hi, wi] = 1.0
                    ref_gx[b, c, hi, wi] = np.sum(oracle.fused(psi, e, W) * g64)
    ref_dW = np.zeros_like(dW)
    for o in range(Co):
        for c in range(C):
            for k in range(3):
                e = np.zeros_like(W)
                e[o, c, k] = 1.0
                ref_dW[o, c, k] = np.sum(oracle.fused(psi, x, e) * g64)
    np.testing.assert_allclose(gx, ref_gx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW, ref_dW, rtol=1e-12, atol=1e-12)


def test_fused_bwd_dense_brute_force():
    Hi, Wi, Ho, Wo, tc, n_r, n_a = 9, 16, 9, 8, 0.9, 2, 4
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    D = _dense_operator(Hi, Wi, Ho, Wo, tc, n_r, n_a)
    x = randn((2, 3, Hi, Wi), 44).numpy().astype(np.float64)
    W = randn((5, 3, psi.K), 45).numpy().astype(np.float64)
    gy = randn((2, 5, Ho, Wo), 46).numpy().astype(np.float64)
    g = np.einsum("ock,bohw->bckhw", W, gy)
    ref_gx = np.einsum("kowhv,bckow->bchv", D, g)
    ref_dW = np.einsum("bohw,bckhw->ock", gy, np.einsum("kowhv,bchv->bckow", D, x))
    gx, dW = oracle.fused_bwd(psi, x, W, gy)
    assert np.abs(gx - ref_gx).max() <= 1e-12 * max(1.0, np.abs(ref_gx).max())
    assert np.abs(dW - ref_dW).max() <= 1e-12 * max(1.0, np.abs(ref_dW).max())


@pytest.mark.parametrize("name", ["tiny_fwd_f32_16x32", "fwdbwd_f32_181x360"])
def test_fused_bwd_adjoint_identities(name):
    psi = workload_psi(WORKLOADS[name])
    B, C, Co = 1, 3, 5
    x = randn((B, C, psi.Hi, psi.Wi), 47).numpy()
    W = randn((Co, C, psi.K), 48).numpy()
    gy = randn((B, Co, psi.Ho, psi.Wo), 49).numpy()
    lhs = float(np.sum(oracle.fused(psi, x, W) * gy))
    gx, dW = oracle.fused_bwd(psi, x, W, gy)
    scale = float(np.sum(oracle.fused(psi, np.abs(x), np.abs(W), abs_mode=True) * np.abs(gy)))
    assert abs(lhs - float(np.sum(x.astype(np.float64) * gx))) <= 1e-13 * scale
    assert abs(lhs - float(np.sum(W.astype(np.float64) * dW))) <= 1e-13 * scale
    ngx, ndW = oracle.fused_bwd(psi, x, W, gy, abs_mode=True)
    assert np.all(ngx >= np.abs(gx)) and np.all(ndW >= np.abs(dW))



@pytest.mark.parametrize("geom", [
    (12, 24, 12, 24, 0.5, 3, 3, "legendre-gauss", "legendre-gauss"),
    (13, 32, 8, 16, 0.6, 3, 3, "equiangular", "legendre-gauss"),
])
def test_dense_brute_force_legendre_gauss(geom):
    """The page's benchmark grids: Gauss-Legendre latitudes (and equiangular -> Gauss-Legendre with
    s = 2), three azimuthal factors; fwd, bwd and fused against the dense basis."""
    Hi, Wi, Ho, Wo, tc, n_r, n_a, gi, go = geom
    psi = build_psi(Hi, Wi, Ho, Wo, tc, n_r, n_a, gi, go)
    D = _dense_operator(Hi, Wi, Ho, Wo, tc, n_r, n_a, gi, go)
    x = randn((2, 3, Hi, Wi), 61).numpy()
    g = randn((2, 3, psi.K, Ho, Wo), 62).numpy()
    W = randn((4, 3, psi.K), 63).numpy()
    ref_out = np.einsum("kowhv,bchv->bckow", D, x.astype(np.float64))
    ref_gx = np.einsum("kowhv,bckow->bchv", D, g.astype(np.float64))
    ref_y = np.einsum("ock,bckhw->bohw", W.astype(np.float64), ref_out)
    assert np.abs(oracle.fwd(psi, x) - ref_out).max() <= 1e-12 * max(1.0, np.abs(ref_out).max())
    assert np.abs(oracle.bwd(psi, g) - ref_gx).max() <= 1e-12 * max(1.0, np.abs(ref_gx).max())
    assert np.abs(oracle.fused(psi, x, W) - ref_y).max() <= 1e-12 * max(1.0, np.abs(ref_y).max())

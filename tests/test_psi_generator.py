"""Sanity of the synthetic psi (pins the input, not the kernels).

* the quadrature sums to the sphere's area up to the equiangular rule's error;
* the hat partition of unity integrates to the tapered-cap area
  2*pi*(1 - (sin(theta_c) - sin(a)) / dr), a = (n_r - 1)*dr, on rows away from
  the poles;
* CSR invariants (monotone row pointer, columns in range, ascending (hi, wi));
* recorded nnz of each workload's psi.
"""
import math

import numpy as np
import pytest

from disco_inputs import WORKLOADS, workload_psi
from disco_inputs.psi import build_psi, equiangular_colatitudes, quadrature_weights

# nnz of each workload's psi as built by disco_inputs.psi.  At 721 rows the hat
# spacing theta_c/4 = 0.75 deg is exactly three grid rows, so ~38k candidate
# entries sit within 1e-12 of a hat edge and their membership is decided by
# fp64 rounding; the count below is this generator's outcome.
EXPECTED_NNZ = {
    "tiny_fwd_f32_16x32": 522,
    "fwdbwd_f32_181x360": 23309,
    "fwd_bf16_721x1440": 1829860,
    "fused_bf16_721x1440": 3417372,
}


@pytest.mark.parametrize("H,W,frac", [(16, 32, 0.99634), (181, 360, 0.99997), (721, 1440, 0.9999984)])
def test_quadrature_sums_to_sphere(H, W, frac):
    q = quadrature_weights(H, W)
    total = q.sum() * W
    # closed form: sum_j sin(pi j/(H-1)) = cot(pi/(2(H-1))); times dtheta*dphi*W
    dth = math.pi / (H - 1)
    closed = (1.0 / math.tan(dth / 2)) * dth * 2 * math.pi
    assert abs(total - closed) < 1e-10 * closed
    assert abs(total / (4 * math.pi) - frac) < 1e-5


def _cap_integral(theta_c, n_r):
    dr = theta_c / n_r
    a = (n_r - 1) * dr
    return 2 * math.pi * (1.0 - (math.sin(theta_c) - math.sin(a)) / dr)


@pytest.mark.parametrize("Hi,Wi,Ho,Wo,tc_deg,tol", [(181, 360, 91, 180, 4, 1e-2), (721, 1440, 361, 720, 3, 1e-3)])
def test_hat_partition_integrates_to_cap(Hi, Wi, Ho, Wo, tc_deg, tol):
    tc = tc_deg * math.pi / 180
    psi = build_psi(Hi, Wi, Ho, Wo, tc, 4, 1)
    to = equiangular_colatitudes(Ho)
    dth = math.pi / (Hi - 1)
    ref = _cap_integral(tc, 4)
    checked = 0
    for ho in range(Ho):
        if to[ho] < tc + dth or to[ho] > math.pi - tc - dth:
            continue
        tot = 0.0
        for k in range(4):
            _, _, v = psi.row(k, ho)
            tot += float(np.sum(v.astype(np.float64)))
        assert abs(tot / ref - 1.0) < tol, (ho, tot, ref)
        checked += 1
    assert checked > Ho // 2


@pytest.mark.parametrize("name", list(EXPECTED_NNZ))
def test_workload_psi_invariants_and_nnz(name):
    w = WORKLOADS[name]
    psi = workload_psi(w)
    assert psi.nnz == EXPECTED_NNZ[name]
    assert psi.row_ptr.shape == (w.K * w.Ho + 1,) and psi.row_ptr[0] == 0
    assert np.all(np.diff(psi.row_ptr) >= 0)
    assert psi.col_hi.min() >= 1 and psi.col_hi.max() <= w.Hi - 2  # poles carry zero weight
    assert psi.col_wi.min() >= 0 and psi.col_wi.max() < w.Wi
    for r in range(0, w.K * w.Ho, max(1, (w.K * w.Ho) // 37)):
        a, b = psi.row_ptr[r], psi.row_ptr[r + 1]
        key = psi.col_hi[a:b].astype(np.int64) * w.Wi + psi.col_wi[a:b]
        assert np.all(np.diff(key) > 0)
    # all azimuthal rows of one hat share their support
    if w.n_a > 1:
        for ho in (0, w.Ho // 3, w.Ho - 1):
            for m in range(w.n_r):
                base = psi.row(m * w.n_a, ho)
                for a in range(1, w.n_a):
                    other = psi.row(m * w.n_a + a, ho)
                    np.testing.assert_array_equal(base[0], other[0])
                    np.testing.assert_array_equal(base[1], other[1])



def test_legendre_gauss_grid_quadrature():
    """Gauss-Legendre latitudes: the weights integrate polynomials in cos(theta) of degree < 2H
    exactly; the sphere's area is 4 pi and the nodes are symmetric about the equator."""
    from disco_inputs.psi import grid_colatitudes, grid_quadrature
    for H, W in ((12, 24), (360, 720)):
        th = grid_colatitudes("legendre-gauss", H)
        q = grid_quadrature("legendre-gauss", H, W)
        assert np.all(np.diff(th) > 0) and th[0] > 0 and th[-1] < np.pi
        np.testing.assert_allclose(th + th[::-1], np.pi, atol=1e-12)
        np.testing.assert_allclose(W * q.sum(), 4 * np.pi, rtol=1e-13)
        # integral over the sphere of cos^2(theta) = 4 pi / 3
        np.testing.assert_allclose(W * np.sum(q * np.cos(th) ** 2), 4 * np.pi / 3, rtol=1e-12)


def test_page_benchmark_workloads():
    from disco_inputs import WORKLOADS, workload_psi
    for name in ("page_self_256x360x720", "page_down_80x721x1440"):
        w = WORKLOADS[name]
        p = workload_psi(w)
        assert p.K == 9 and (p.Ho, p.Wo, p.Hi, p.Wi) == (w.Ho, w.Wo, w.Hi, w.Wi)
        assert np.all(np.diff(p.row_ptr) > 0)  # every row sees some input at theta_c = 0.017
        assert p.col_hi.min() >= 0 and p.col_hi.max() < p.Hi and p.col_wi.max() < p.Wi

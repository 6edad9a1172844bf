"""Synthetic DISCO filter tensor ("psi") in CSR form.

This module builds the sparse filter that both the HIP path and the fp64 oracle
consume.  It holds no part of the contraction itself: only the geometry of the
sphere (grids, quadrature, geodesic distance, bearing) and the filter basis.

Source: torch-harmonics "disco-kernel-dev" skill page, section "Architecture
snapshot" — the forward op is a CSR sparse contraction from the input grid to a
K-expanded output (B, C, K, H, W), and the kpacked section stores psi values as
fp32.  The page does not define the basis, the grids or the quadrature; the
plain readings used here are:

* equiangular grid, poles included: colatitude theta_j = pi*j/(H-1), longitude
  phi_i = 2*pi*i/W (input and output grids alike);
* quadrature weight q_j = sin(theta_j) * dtheta * dphi, with sin set to exactly
  0 at both poles (so polar input rows carry no entries);
* the page's benchmark shapes also name a "legendre-gauss" grid (section
  "Serial Benchmarks"): colatitudes theta_j = arccos(x_j) for the H Gauss-Legendre
  nodes x_j in decreasing order (north to south), weights q_j = w_j * dphi with
  w_j the Gauss weights (they sum to 2, so the weights of the sphere sum to 4 pi);
* geodesic distance by the haversine formula in colatitude;
* isotropic piecewise-linear hats: dr = theta_c / n_r, centres r_m = m*dr,
  hat_m(d) = max(0, 1 - |d - r_m| / dr) for d < theta_c, else 0;
* azimuthal factors of the bearing alpha seen from the output point:
  n_a = 1 -> {1}; 2 -> {cos a, sin a}; 3 -> {1, cos a, sin a};
  4 -> {cos a, sin a, cos 2a, sin 2a} (the page's "harmonic" kernel_shape (3, 3)
  is read as 3 radial hats x these 3 azimuthal factors, K = 9);
* basis index k = m * n_a + a (radial outer, azimuthal inner);
* an entry (k, ho; hi, wi) is stored iff hat_m(d) > 0 and q_hi > 0 (the
  azimuthal factor never removes an entry, so all n_a rows of one hat share
  their support); value = hat * A_a(alpha) * q_hi in fp64, stored as fp32 (RNE);
* no normalisation of the basis.

The psi is shared by all output longitudes: column (hi, wi) of row (k, ho) is
the input pixel at longitude offset wi from output longitude 0, and output
longitude wo reads input longitude (wi + pscale*wo) mod Wi.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class PsiCSR:
    """CSR filter.  Rows r = k*Ho + ho; columns (col_hi, col_wi); fp32 values."""

    K: int
    Ho: int
    Wo: int
    Hi: int
    Wi: int
    row_ptr: np.ndarray  # int64 [K*Ho + 1]
    col_hi: np.ndarray  # int32 [nnz]
    col_wi: np.ndarray  # int32 [nnz]
    val: np.ndarray  # float32 [nnz]

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])

    @property
    def pscale(self) -> int:
        return self.Wi // self.Wo

    def row(self, k: int, ho: int):
        r = k * self.Ho + ho
        a, b = int(self.row_ptr[r]), int(self.row_ptr[r + 1])
        return self.col_hi[a:b], self.col_wi[a:b], self.val[a:b]


def equiangular_colatitudes(n: int) -> np.ndarray:
    """Colatitudes pi*j/(n-1), j = 0..n-1 (both poles included)."""
    if n < 2:
        raise ValueError("an equiangular grid needs at least two latitude rows")
    return np.pi * np.arange(n, dtype=np.float64) / (n - 1)


def quadrature_weights(H: int, W: int) -> np.ndarray:
    """Per-latitude weights sin(theta)*dtheta*dphi, exactly zero at the poles."""
    theta = equiangular_colatitudes(H)
    s = np.sin(theta)
    s[0] = 0.0
    s[-1] = 0.0
    return s * (np.pi / (H - 1)) * (2.0 * np.pi / W)


def legendre_gauss_colatitudes(n: int):
    """(colatitudes, Gauss weights) for n Gauss-Legendre latitudes, north to south."""
    x, w = np.polynomial.legendre.leggauss(n)
    order = np.argsort(-x)  # x = cos(theta) decreasing: theta increasing
    return np.arccos(x[order]), w[order]


def grid_colatitudes(grid: str, H: int) -> np.ndarray:
    if grid == "equiangular":
        return equiangular_colatitudes(H)
    if grid == "legendre-gauss":
        return legendre_gauss_colatitudes(H)[0]
    raise ValueError(f"unknown grid {grid}")


def grid_quadrature(grid: str, H: int, W: int) -> np.ndarray:
    """Per-latitude quadrature weights of the grid (sum over the sphere = W * sum = 4 pi)."""
    if grid == "equiangular":
        return quadrature_weights(H, W)
    if grid == "legendre-gauss":
        return legendre_gauss_colatitudes(H)[1] * (2.0 * np.pi / W)
    raise ValueError(f"unknown grid {grid}")


def geodesic_distance(theta_o, theta_i, dphi):
    """Great-circle distance (haversine form, colatitudes)."""
    h = np.sin(0.5 * (theta_i - theta_o)) ** 2 + np.sin(theta_o) * np.sin(theta_i) * np.sin(0.5 * dphi) ** 2
    return 2.0 * np.arcsin(np.sqrt(np.clip(h, 0.0, 1.0)))


def bearing(theta_o, theta_i, dphi):
    """Bearing of the input point seen from the output point (from local north)."""
    y = np.sin(dphi) * np.sin(theta_i)
    x = np.sin(theta_o) * np.cos(theta_i) - np.cos(theta_o) * np.sin(theta_i) * np.cos(dphi)
    return np.arctan2(y, x)


def radial_hats(d, theta_c: float, n_r: int) -> np.ndarray:
    """hat_m(d) for m = 0..n_r-1, shape (n_r,) + d.shape."""
    dr = theta_c / n_r
    out = np.empty((n_r,) + np.shape(d), dtype=np.float64)
    for m in range(n_r):
        h = 1.0 - np.abs(d - m * dr) / dr
        out[m] = np.where(d < theta_c, np.maximum(h, 0.0), 0.0)
    return out


def azimuthal_factors(alpha, n_a: int) -> np.ndarray:
    if n_a == 1:
        return np.ones((1,) + np.shape(alpha))
    if n_a == 2:
        return np.stack([np.cos(alpha), np.sin(alpha)])
    if n_a == 3:
        return np.stack([np.ones_like(np.asarray(alpha, dtype=np.float64)), np.cos(alpha), np.sin(alpha)])
    if n_a == 4:
        return np.stack([np.cos(alpha), np.sin(alpha), np.cos(2 * alpha), np.sin(2 * alpha)])
    raise ValueError(f"unsupported number of azimuthal factors {n_a}")


def basis_values(theta_o, theta_i, dphi, theta_c: float, n_r: int, n_a: int, q) -> np.ndarray:
    """Dense fp64 values of all K = n_r*n_a basis functions times quadrature.

    Returns shape (K,) + broadcast shape.  Entries outside every hat are 0.
    """
    d = geodesic_distance(theta_o, theta_i, dphi)
    hats = radial_hats(d, theta_c, n_r)
    az = azimuthal_factors(bearing(theta_o, theta_i, dphi), n_a)
    vals = hats[:, None] * az[None, :] * q
    return vals.reshape((n_r * n_a,) + vals.shape[2:]), hats


def build_psi(Hi: int, Wi: int, Ho: int, Wo: int, theta_c: float, n_r: int, n_a: int = 1,
              grid_in: str = "equiangular", grid_out: str = "equiangular") -> PsiCSR:
    """Build the CSR psi for a Hi x Wi -> Ho x Wo convolution on the given latitude grids."""
    if Wi % Wo != 0:
        raise ValueError("Wi must be an integer multiple of Wo")
    K = n_r * n_a
    theta_in = grid_colatitudes(grid_in, Hi)
    theta_out = grid_colatitudes(grid_out, Ho)
    q = grid_quadrature(grid_in, Hi, Wi)
    dphi_all = 2.0 * np.pi * np.arange(Wi, dtype=np.float64) / Wi

    # rows are emitted per (k, ho); collect per ho first, then order by k
    per_row_hi = [[None] * Ho for _ in range(K)]
    per_row_wi = [[None] * Ho for _ in range(K)]
    per_row_val = [[None] * Ho for _ in range(K)]
    for ho in range(Ho):
        to = theta_out[ho]
        # only rows within theta_c in colatitude can be within theta_c in distance
        his = np.nonzero((np.abs(theta_in - to) < theta_c) & (q > 0))[0]
        if his.size == 0:
            for k in range(K):
                per_row_hi[k][ho] = np.zeros(0, np.int32)
                per_row_wi[k][ho] = np.zeros(0, np.int32)
                per_row_val[k][ho] = np.zeros(0, np.float32)
            continue
        TI = theta_in[his][:, None]
        DP = dphi_all[None, :]
        vals, hats = basis_values(to, TI, DP, theta_c, n_r, n_a, q[his][:, None])
        for m in range(n_r):
            mask = hats[m] > 0.0  # (n_hi, Wi), row-major => ascending (hi, wi)
            hh, ww = np.nonzero(mask)
            for a in range(n_a):
                k = m * n_a + a
                per_row_hi[k][ho] = his[hh].astype(np.int32)
                per_row_wi[k][ho] = ww.astype(np.int32)
                per_row_val[k][ho] = vals[k][mask].astype(np.float32)

    counts = np.array([per_row_hi[k][ho].size for k in range(K) for ho in range(Ho)], dtype=np.int64)
    row_ptr = np.zeros(K * Ho + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_hi = np.concatenate([per_row_hi[k][ho] for k in range(K) for ho in range(Ho)])
    col_wi = np.concatenate([per_row_wi[k][ho] for k in range(K) for ho in range(Ho)])
    val = np.concatenate([per_row_val[k][ho] for k in range(K) for ho in range(Ho)])
    return PsiCSR(K, Ho, Wo, Hi, Wi, row_ptr, col_hi.astype(np.int32), col_wi.astype(np.int32),
                  val.astype(np.float32))


def random_psi(K: int, Ho: int, Wo: int, Hi: int, Wi: int, density: float, seed: int,
               empty_rows=()) -> PsiCSR:
    """Random CSR psi for edge-case tests: uniform columns, N(0,1) values.

    Rows listed in ``empty_rows`` (flat r = k*Ho + ho) get no entries.
    """
    rng = np.random.default_rng(seed)
    his, wis, vals, counts = [], [], [], []
    empty = set(int(r) for r in empty_rows)
    for r in range(K * Ho):
        if r in empty:
            counts.append(0)
            continue
        mask = rng.random((Hi, Wi)) < density
        hh, ww = np.nonzero(mask)
        his.append(hh.astype(np.int32))
        wis.append(ww.astype(np.int32))
        vals.append(rng.standard_normal(hh.size).astype(np.float32))
        counts.append(hh.size)
    row_ptr = np.zeros(K * Ho + 1, dtype=np.int64)
    np.cumsum(np.asarray(counts, dtype=np.int64), out=row_ptr[1:])
    cat = lambda xs, dt: np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt)
    return PsiCSR(K, Ho, Wo, Hi, Wi, row_ptr, cat(his, np.int32), cat(wis, np.int32), cat(vals, np.float32))

"""fp64 CPU oracle of the DISCO CSR contraction (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP product path
(``sparse_gather_contraction_amd``) never imports it, and it imports nothing
from there.

The arithmetic lives in ``disco_oracle.c`` (plain serial fp64 loops, OpenMP
only across independent planes); this module builds that file with gcc and
marshals numpy arrays into it.  See the header of ``disco_oracle.c`` for the
formulas and their source (torch-harmonics "disco-kernel-dev" page, section
"Architecture snapshot").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "disco_oracle.c")
# DISCO_ORACLE_LIB: load this library file instead (the mutation test points it at copies of the
# source with a planted mistake, to show that the pins catch each one)
_BUILT = os.path.join(_HERE, "libdisco_oracle.so")
_LIB = os.environ.get("DISCO_ORACLE_LIB") or _BUILT
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, OpenMP across planes)."""
    if force or not os.path.exists(_BUILT):
        tmp = _BUILT + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                        "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _BUILT)
    return _BUILT


def _load():
    global _lib
    if _lib is None:
        if _LIB == _BUILT and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, P = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_fwd.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, i32]
        lib.oracle_bwd.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, i32]
        lib.oracle_fused.argtypes = [i32] * 8 + [P] * 6 + [i32, P, P, i32]
        lib.oracle_einsum.argtypes = [i32, i32, i32, i32, i64, P, P, P, i32]
        lib.oracle_fused_bwd.argtypes = [i32] * 8 + [P] * 7 + [P, P, i32]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _np_f32(t):
    """Accept numpy arrays or torch tensors (fp32, bf16 or fp16); widen exactly to fp32."""
    if hasattr(t, "detach"):
        t = t.detach().cpu().float().numpy()
    return np.ascontiguousarray(t, dtype=np.float32)


def _psi_args(psi):
    rp, rp_p = _c(psi.row_ptr, np.int64)
    ch, ch_p = _c(psi.col_hi, np.int32)
    cw, cw_p = _c(psi.col_wi, np.int32)
    v, v_p = _c(psi.val, np.float32)
    return (rp, ch, cw, v), (rp_p, ch_p, cw_p, v_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def fwd(psi, x, abs_mode: bool = False) -> np.ndarray:
    """out[..., k, ho, wo] in fp64 for x of shape [..., Hi, Wi]."""
    lib = _load()
    x = _np_f32(x)
    lead = x.shape[:-2]
    assert x.shape[-2:] == (psi.Hi, psi.Wi)
    P = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (psi.K, psi.Ho, psi.Wo), dtype=np.float64)
    keep, ptrs = _psi_args(psi)
    lib.oracle_fwd(P, psi.K, psi.Ho, psi.Wo, psi.Hi, psi.Wi, *ptrs,
                   x.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p), int(abs_mode))
    return out


def bwd(psi, gout, abs_mode: bool = False) -> np.ndarray:
    """gx[..., hi, wi] in fp64 for gout of shape [..., K, Ho, Wo] (scatter form)."""
    lib = _load()
    g = _np_f32(gout)
    lead = g.shape[:-3]
    assert g.shape[-3:] == (psi.K, psi.Ho, psi.Wo)
    P = int(np.prod(lead)) if lead else 1
    gx = np.empty(lead + (psi.Hi, psi.Wi), dtype=np.float64)
    keep, ptrs = _psi_args(psi)
    lib.oracle_bwd(P, psi.K, psi.Ho, psi.Wo, psi.Hi, psi.Wi, *ptrs,
                   g.ctypes.data_as(ctypes.c_void_p), gx.ctypes.data_as(ctypes.c_void_p), int(abs_mode))
    return gx


def fused(psi, x, W, ho_list=None, abs_mode: bool = False) -> np.ndarray:
    """y[b, o, h, wo] in fp64 for the output latitudes ``ho_list`` (default: all)."""
    lib = _load()
    x = _np_f32(x)
    W = _np_f32(W)
    B, C = x.shape[:2]
    Co = W.shape[0]
    assert x.shape[2:] == (psi.Hi, psi.Wi) and W.shape == (Co, C, psi.K)
    if ho_list is None:
        ho_list = np.arange(psi.Ho)
    hl, hl_p = _c(ho_list, np.int32)
    y = np.empty((B, Co, hl.size, psi.Wo), dtype=np.float64)
    keep, ptrs = _psi_args(psi)
    lib.oracle_fused(B, C, Co, psi.K, psi.Ho, psi.Wo, psi.Hi, psi.Wi, *ptrs,
                     x.ctypes.data_as(ctypes.c_void_p), W.ctypes.data_as(ctypes.c_void_p),
                     hl.size, hl_p, y.ctypes.data_as(ctypes.c_void_p), int(abs_mode))
    return y


def einsum(W, t, abs_mode: bool = False) -> np.ndarray:
    """y[b, o, ...] in fp64 for a contraction t [B, C, K, ...] (fp64, or fp32/bf16/fp16 widened
    exactly) and W [Co, C, K]: the fused convolution's einsum alone."""
    lib = _load()
    if hasattr(t, "detach"):
        t = t.detach().cpu().double().numpy()
    t = np.ascontiguousarray(t, dtype=np.float64)
    W = _np_f32(W)
    B, C, K = t.shape[:3]
    Co = W.shape[0]
    assert W.shape == (Co, C, K)
    pos = t.shape[3:]
    P = int(np.prod(pos)) if pos else 1
    y = np.empty((B, Co) + pos, dtype=np.float64)
    lib.oracle_einsum(B, C, Co, K, P, W.ctypes.data_as(ctypes.c_void_p), t.ctypes.data_as(ctypes.c_void_p),
                      y.ctypes.data_as(ctypes.c_void_p), int(abs_mode))
    return y

def fused_bwd(psi, x, W, gy, abs_mode: bool = False):
    """(gx [B, C, Hi, Wi], dW [Co, C, K]) in fp64: the gradients of <gy, y> for the fused op."""
    lib = _load()
    x = _np_f32(x)
    W = _np_f32(W)
    gy = _np_f32(gy)
    B, C = x.shape[:2]
    Co = W.shape[0]
    assert x.shape[2:] == (psi.Hi, psi.Wi) and W.shape == (Co, C, psi.K)
    assert gy.shape == (B, Co, psi.Ho, psi.Wo)
    gx = np.empty((B, C, psi.Hi, psi.Wi), dtype=np.float64)
    dW = np.empty((Co, C, psi.K), dtype=np.float64)
    keep, ptrs = _psi_args(psi)
    lib.oracle_fused_bwd(B, C, Co, psi.K, psi.Ho, psi.Wo, psi.Hi, psi.Wi, *ptrs,
                         x.ctypes.data_as(ctypes.c_void_p), W.ctypes.data_as(ctypes.c_void_p),
                         gy.ctypes.data_as(ctypes.c_void_p), gx.ctypes.data_as(ctypes.c_void_p),
                         dW.ctypes.data_as(ctypes.c_void_p), int(abs_mode))
    return gx, dW

"""Python binding of libdisco.so — argument marshalling only.

Every step of the DISCO contraction runs in the library's HIP kernels; this
module turns torch tensors into ``disco_tensor`` views (device pointer, dtype,
shape), passes torch's current HIP stream, and raises on a non-OK status.
The names mirror the C ABI in ``include/disco.h``:

    psi = disco_psi_create(csr, device)      # csr: K, Ho, Wo, Hi, Wi, row_ptr, col_hi, col_wi, val
    out = disco_fwd(psi, x)                  # (B,C,Hi,Wi) -> (B,C,K,Ho,Wo)
    gx  = disco_bwd(psi, gout)               # (B,C,K,Ho,Wo) -> (B,C,Hi,Wi)
    y   = disco_fused_conv(psi, x, W)        # (B,C,Hi,Wi), (Co,C,K) -> (B,Co,Ho,Wo)

There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdisco.so")

DISCO_OK = 0
STATUS_NAMES = {
    0: "DISCO_OK",
    1: "DISCO_ERR_INVALID_ARGUMENT",
    2: "DISCO_ERR_SHAPE",
    3: "DISCO_ERR_DTYPE",
    4: "DISCO_ERR_PSI",
    5: "DISCO_ERR_UNSUPPORTED_DEVICE",
    6: "DISCO_ERR_OOM",
    7: "DISCO_ERR_HIP",
}
DISCO_F32 = 0
DISCO_BF16 = 1
DISCO_F16 = 2
EXPORTED = ("disco_psi_create", "disco_psi_destroy", "disco_fwd", "disco_bwd", "disco_fused_conv",
            "disco_fused_conv_save", "disco_einsum", "disco_fused_conv_bwd_workspace", "disco_fused_conv_bwd",
            "disco_fused_conv_bwd_saved", "disco_fused_conv_bwd_noalloc", "disco_last_error")


class DiscoError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class CSRDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("Ho", ctypes.c_int32), ("Wo", ctypes.c_int32), ("Hi", ctypes.c_int32),
                ("Wi", ctypes.c_int32), ("nnz", ctypes.c_int64), ("row_ptr", ctypes.c_void_p),
                ("col_hi", ctypes.c_void_p), ("col_wi", ctypes.c_void_p), ("val", ctypes.c_void_p)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 5)]


_lib = None


def load_library():
    """Load libdisco.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_gather_contraction_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.disco_psi_create.argtypes = [ctypes.POINTER(CSRDesc), ctypes.c_int, ctypes.POINTER(P)]
        lib.disco_psi_destroy.argtypes = [P]
        lib.disco_fwd.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(TensorDesc), P]
        lib.disco_bwd.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(TensorDesc), P]
        lib.disco_fused_conv.argtypes = [P, ctypes.POINTER(TensorDesc), ctypes.POINTER(TensorDesc),
                                         ctypes.POINTER(TensorDesc), P]
        lib.disco_einsum.argtypes = [ctypes.POINTER(TensorDesc)] * 3 + [P]
        lib.disco_fused_conv_save.argtypes = [P] + [ctypes.POINTER(TensorDesc)] * 4 + [P]
        lib.disco_fused_conv_bwd_saved.argtypes = [P] + [ctypes.POINTER(TensorDesc)] * 5 + [P, ctypes.c_size_t, P]
        lib.disco_fused_conv_bwd_workspace.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        lib.disco_fused_conv_bwd.argtypes = [P] + [ctypes.POINTER(TensorDesc)] * 5 + [P, ctypes.c_size_t, P]
        lib.disco_fused_conv_bwd_noalloc.argtypes = [P] + [ctypes.POINTER(TensorDesc)] * 5 + [P]
        lib.disco_last_error.restype = ctypes.c_char_p
        for f in ("disco_psi_create", "disco_psi_destroy", "disco_fwd", "disco_bwd", "disco_fused_conv",
                  "disco_fused_conv_save", "disco_einsum", "disco_fused_conv_bwd_workspace", "disco_fused_conv_bwd",
                  "disco_fused_conv_bwd_saved", "disco_fused_conv_bwd_noalloc"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(status: int):
    if status != DISCO_OK:
        raise DiscoError(status, load_library().disco_last_error().decode())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return DISCO_F32
    if t.dtype == torch.bfloat16:
        return DISCO_BF16
    if t.dtype == torch.float16:
        return DISCO_F16
    return 99  # rejected by the library with DISCO_ERR_DTYPE


def tensor_desc(t) -> TensorDesc:
    """View of a contiguous torch tensor for the C ABI."""
    if not t.is_contiguous():
        raise ValueError("disco tensors must be contiguous")
    d = TensorDesc()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i, s in enumerate(t.shape[:5]):
        d.shape[i] = int(s)
    return d


def _stream(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def csr_desc(csr):
    """CSRDesc over host numpy arrays; returns (desc, arrays kept alive)."""
    rp = np.ascontiguousarray(csr.row_ptr, dtype=np.int64)
    ch = np.ascontiguousarray(csr.col_hi, dtype=np.int32)
    cw = np.ascontiguousarray(csr.col_wi, dtype=np.int32)
    v = np.ascontiguousarray(csr.val, dtype=np.float32)
    d = CSRDesc(int(csr.K), int(csr.Ho), int(csr.Wo), int(csr.Hi), int(csr.Wi), int(rp[-1]) if rp.size else 0,
                rp.ctypes.data, ch.ctypes.data, cw.ctypes.data, v.ctypes.data)
    return d, (rp, ch, cw, v)


class Psi:
    """Owner of a disco_psi handle (device plans of one CSR filter)."""

    def __init__(self, handle: int, csr, device: int):
        self.handle = ctypes.c_void_p(handle)
        self.K, self.Ho, self.Wo, self.Hi, self.Wi = (int(csr.K), int(csr.Ho), int(csr.Wo), int(csr.Hi), int(csr.Wi))
        self.nnz = int(np.asarray(csr.row_ptr)[-1])
        self.device = device

    def close(self):
        if self.handle:
            load_library().disco_psi_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def disco_psi_create(csr, device=None) -> Psi:
    import torch

    lib = load_library()
    if device is None:
        device = torch.cuda.current_device()
    desc, keep = csr_desc(csr)
    h = ctypes.c_void_p()
    _check(lib.disco_psi_create(ctypes.byref(desc), int(device), ctypes.byref(h)))
    return Psi(h.value, csr, int(device))


def disco_fwd(psi: Psi, x, out=None):
    import torch

    if out is None:
        out = torch.empty((x.shape[0], x.shape[1], psi.K, psi.Ho, psi.Wo), dtype=x.dtype, device=x.device)
    xd, od = tensor_desc(x), tensor_desc(out)
    _check(load_library().disco_fwd(psi.handle, ctypes.byref(xd), ctypes.byref(od), _stream(x.device)))
    return out


def disco_bwd(psi: Psi, gout, gx=None):
    import torch

    if gx is None:
        gx = torch.empty((gout.shape[0], gout.shape[1], psi.Hi, psi.Wi), dtype=gout.dtype, device=gout.device)
    gd, xd = tensor_desc(gout), tensor_desc(gx)
    _check(load_library().disco_bwd(psi.handle, ctypes.byref(gd), ctypes.byref(xd), _stream(gout.device)))
    return gx


def disco_fused_conv(psi: Psi, x, W, y=None):
    import torch

    if y is None:
        y = torch.empty((x.shape[0], W.shape[0], psi.Ho, psi.Wo), dtype=x.dtype, device=x.device)
    xd, wd, yd = tensor_desc(x), tensor_desc(W), tensor_desc(y)
    _check(load_library().disco_fused_conv(psi.handle, ctypes.byref(xd), ctypes.byref(wd), ctypes.byref(yd),
                                           _stream(x.device)))
    return y




def disco_fused_conv_save(psi: Psi, x, W, y=None, out=None):
    """(y, out): the fused convolution and the contraction F x it multiplied (kept for the backward)."""
    import torch

    if y is None:
        y = torch.empty((x.shape[0], W.shape[0], psi.Ho, psi.Wo), dtype=x.dtype, device=x.device)
    if out is None:
        out = torch.empty((x.shape[0], x.shape[1], psi.K, psi.Ho, psi.Wo), dtype=x.dtype, device=x.device)
    xd, wd, yd, od = tensor_desc(x), tensor_desc(W), tensor_desc(y), tensor_desc(out)
    _check(load_library().disco_fused_conv_save(psi.handle, ctypes.byref(xd), ctypes.byref(wd), ctypes.byref(yd),
                                                ctypes.byref(od), _stream(x.device)))
    return y, out

def disco_einsum(W, t, y=None):
    """y[b, o, ho, wo] = sum_{c,k} W[o, c, k] t[b, c, k, ho, wo] on the current device (no psi)."""
    import torch

    if y is None:
        y = torch.empty((t.shape[0], W.shape[0], t.shape[3], t.shape[4]), dtype=t.dtype, device=t.device)
    wd, td, yd = tensor_desc(W), tensor_desc(t), tensor_desc(y)
    _check(load_library().disco_einsum(ctypes.byref(wd), ctypes.byref(td), ctypes.byref(yd), _stream(t.device)))
    return y

def disco_fused_conv_bwd_workspace(psi: Psi, B: int, C: int, Co: int) -> int:
    """Workspace bytes disco_fused_conv_bwd needs for these sizes."""
    n = ctypes.c_size_t()
    _check(load_library().disco_fused_conv_bwd_workspace(psi.handle, int(B), int(C), int(Co), ctypes.byref(n)))
    return int(n.value)


def disco_fused_conv_bwd(psi: Psi, x, W, gy, gx=None, dW=None, workspace=None):
    """(gx, dW): gradients of <gy, disco_fused_conv(x, W)>.  The workspace (a uint8 device tensor)
    is allocated here when not given."""
    import torch

    if gx is None:
        gx = torch.empty_like(x)
    if dW is None:
        dW = torch.empty_like(W)
    need = disco_fused_conv_bwd_workspace(psi, x.shape[0], x.shape[1], W.shape[0])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    descs = [tensor_desc(t) for t in (x, W, gy, gx, dW)]
    _check(load_library().disco_fused_conv_bwd(psi.handle, *[ctypes.byref(d) for d in descs],
                                               ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                               _stream(x.device)))
    return gx, dW


def disco_fused_conv_bwd_noalloc(psi: Psi, x, W, gy, gx=None, dW=None):
    """(gx, dW) as disco_fused_conv_bwd, with the library's per-device scratch array as workspace
    (no device allocation inside the call; gx and dW are allocated here when not given)."""
    import torch

    if gx is None:
        gx = torch.empty_like(x)
    if dW is None:
        dW = torch.empty_like(W)
    descs = [tensor_desc(t) for t in (x, W, gy, gx, dW)]
    _check(load_library().disco_fused_conv_bwd_noalloc(psi.handle, *[ctypes.byref(d) for d in descs],
                                                       _stream(x.device)))
    return gx, dW


def disco_fused_conv_bwd_saved(psi: Psi, out, W, gy, gx=None, dW=None, workspace=None):
    """(gx, dW) as disco_fused_conv_bwd, with the contraction `out` from disco_fused_conv_save in place of x."""
    import torch

    B, C = out.shape[0], out.shape[1]
    if gx is None:
        gx = torch.empty((B, C, psi.Hi, psi.Wi), dtype=out.dtype, device=out.device)
    if dW is None:
        dW = torch.empty_like(W)
    need = disco_fused_conv_bwd_workspace(psi, B, C, W.shape[0])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=out.device)
    descs = [tensor_desc(t) for t in (out, W, gy, gx, dW)]
    _check(load_library().disco_fused_conv_bwd_saved(psi.handle, *[ctypes.byref(d) for d in descs],
                                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                                     _stream(out.device)))
    return gx, dW

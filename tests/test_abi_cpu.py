"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/disco.h, and rejects malformed arguments on the host
before touching a device (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_gather_contraction_amd as sgc
from disco_inputs import WORKLOADS, workload_psi
from disco_inputs.psi import PsiCSR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "disco.h")).read()
    return sorted(set(re.findall(r"^\s*(?:disco_status|const char\s*\*)\s*(disco_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(sgc.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = sgc.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def _create(psi, device=0):
    lib = sgc.load_library()
    desc, keep = sgc.csr_desc(psi)
    h = ctypes.c_void_p()
    st = lib.disco_psi_create(ctypes.byref(desc), device, ctypes.byref(h))
    return st, h, lib.disco_last_error().decode()


def _small():
    return workload_psi(WORKLOADS["tiny_fwd_f32_16x32"])


def _mod(psi, **kw):
    d = dict(K=psi.K, Ho=psi.Ho, Wo=psi.Wo, Hi=psi.Hi, Wi=psi.Wi, row_ptr=psi.row_ptr.copy(),
             col_hi=psi.col_hi.copy(), col_wi=psi.col_wi.copy(), val=psi.val.copy())
    d.update(kw)
    return PsiCSR(**d)


def test_rejects_decreasing_row_ptr():
    p = _small()
    rp = p.row_ptr.copy()
    rp[5], rp[6] = rp[6], rp[5] - 1
    st, h, msg = _create(_mod(p, row_ptr=rp))
    assert sgc.STATUS_NAMES[st] == "DISCO_ERR_PSI" and not h.value and "row_ptr" in msg


def test_rejects_column_out_of_range():
    p = _small()
    ch = p.col_hi.copy()
    ch[3] = p.Hi
    st, h, msg = _create(_mod(p, col_hi=ch))
    assert sgc.STATUS_NAMES[st] == "DISCO_ERR_PSI" and "outside" in msg
    cw = p.col_wi.copy()
    cw[0] = -1
    st, h, msg = _create(_mod(p, col_wi=cw))
    assert sgc.STATUS_NAMES[st] == "DISCO_ERR_PSI"


def test_rejects_duplicate_columns():
    p = _small()
    ch, cw = p.col_hi.copy(), p.col_wi.copy()
    a = int(p.row_ptr[0])
    ch[a + 1], cw[a + 1] = ch[a], cw[a]
    st, h, msg = _create(_mod(p, col_hi=ch, col_wi=cw))
    assert sgc.STATUS_NAMES[st] == "DISCO_ERR_PSI" and "duplicate" in msg


def test_rejects_non_integer_subsampling():
    p = _small()
    st, h, msg = _create(_mod(p, Wo=p.Wo - 2))
    assert sgc.STATUS_NAMES[st] == "DISCO_ERR_SHAPE" and "multiple" in msg


def test_rejects_null_arguments():
    lib = sgc.load_library()
    h = ctypes.c_void_p()
    assert sgc.STATUS_NAMES[lib.disco_psi_create(None, 0, ctypes.byref(h))] == "DISCO_ERR_INVALID_ARGUMENT"
    x = sgc.TensorDesc()
    o = sgc.TensorDesc()
    assert sgc.STATUS_NAMES[lib.disco_fwd(None, ctypes.byref(x), ctypes.byref(o), None)] == "DISCO_ERR_INVALID_ARGUMENT"
    assert sgc.STATUS_NAMES[lib.disco_bwd(None, ctypes.byref(x), ctypes.byref(o), None)] == "DISCO_ERR_INVALID_ARGUMENT"
    assert lib.disco_psi_destroy(None) == 0
    assert "NULL" in lib.disco_last_error().decode()


def test_python_binding_raises_on_error():
    p = _small()
    rp = p.row_ptr.copy()
    rp[-1] += 1
    with pytest.raises(sgc.DiscoError) as ei:
        sgc.disco_psi_create(_mod(p, row_ptr=rp), device=0)
    assert ei.value.status_name == "DISCO_ERR_PSI"

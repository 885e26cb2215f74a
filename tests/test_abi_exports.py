"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/sla.h declares, and rejects bad arguments before any
device work."""
import ctypes
import os
import re

import pytest

from differentiable_sparse_linear_csr_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "sla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(sla_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("sla_csr_create", "sla_spmv", "sla_pcg_solve", "sla_adjoint_backward",
                     "sla_csr_destroy", "sla_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _lib.load()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(_lib.EXPORTS) == set(declared_functions())


def test_version_and_error_string():
    L = _lib.load()
    assert L.sla_version().decode().startswith("sla ")
    assert isinstance(L.sla_last_error(), bytes)


def _create(**kw):
    L = _lib.load()
    args = dict(fmt=0, n=4, nnz=0, batch=1, rit=0, rows=None, cit=0, cols=None, vt=1,
                vals=None, flags=0)
    args.update(kw)
    h = ctypes.c_void_p()
    out = kw.get("out", ctypes.byref(h))
    st = L.sla_csr_create(out, args["fmt"], args["n"], args["nnz"], args["batch"], args["rit"],
                          args["rows"], args["cit"], args["cols"], args["vt"], args["vals"],
                          args["flags"], None)
    return st, L.sla_last_error().decode()


@pytest.mark.parametrize("kw,frag", [
    (dict(out=None), "out is null"),
    (dict(n=0), "n must be"),
    (dict(n=1 << 31), "n must be"),
    (dict(batch=0), "batch"),
    (dict(batch=257), "batch"),
    (dict(fmt=7), "format"),
    (dict(rit=5), "index type"),
    (dict(vt=9), "value type"),
    (dict(flags=8), "flag"),
    (dict(nnz=3), "null"),
    (dict(fmt=1), "row_ptr is null"),
])
def test_create_rejects_bad_arguments_before_device_work(kw, frag):
    st, msg = _create(**kw)
    assert st == _lib.SLA_ERR_INVALID_ARG
    assert frag in msg


def test_null_handle_calls_fail_cleanly():
    L = _lib.load()
    info = (_lib.Info * 1)()
    assert L.sla_pcg_solve(None, None, None, 1e-8, 10, info, None) == _lib.SLA_ERR_INVALID_ARG
    assert L.sla_spmv(None, None, None, None) == _lib.SLA_ERR_INVALID_ARG
    assert L.sla_csr_set_option(None, 1, 4) == _lib.SLA_ERR_INVALID_ARG
    n = ctypes.c_int64()
    assert L.sla_profile_get(None, 0, ctypes.byref(n), None) == _lib.SLA_ERR_INVALID_ARG
    L.sla_csr_destroy(None)  # no-op

"""The allocation-free Jacobi-PCG entry point (sla_pcg_solve_noalloc), called
through the C ABI, against sla_pcg_solve on a handle of the same matrix and
against the oracle: outcome, iterations within 2, x within 1e-8 (fp64 at
tol 1e-10). Two calls in a row, the second with a smaller system (the
workspace keeps the first call's contents), the largest system it takes
(2^21 rows), and the errors it reports (size limit, CSR checks on the
device, bad diagonal)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from differentiable_sparse_linear_csr_amd import _lib
from workloads import make_workload

from gpu_util import csr_handle, dev, host, rel

pytestmark = pytest.mark.gpu
MAX_ROWS = 1 << 21


def csr_of(w):
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    return (ref["row_ptr"].astype(np.int32), ref["col"].astype(np.int32),
            np.ascontiguousarray(ref["vals"], dtype=np.float64), ref)


def noalloc(n, rp, col, val, b, tol, maxit, nnz=None):
    """returns (status, x, info) of one call through the C ABI"""
    L = _lib.load()
    x = torch.empty(n, dtype=torch.float64, device="cuda:0")
    info = _lib.Info()
    P = ctypes.c_void_p
    st = L.sla_pcg_solve_noalloc(n, int(col.numel() if nnz is None else nnz), P(rp.data_ptr()),
                                 P(col.data_ptr()), P(val.data_ptr()), P(b.data_ptr()),
                                 P(x.data_ptr()), float(tol), int(maxit), ctypes.byref(info),
                                 None)
    torch.cuda.synchronize()
    return st, x, info


def against_handle_and_oracle(w, tol=None, maxit=None):
    tol = w.tol if tol is None else tol
    maxit = w.maxit if maxit is None else maxit
    rp, col, val, ref = csr_of(w)
    drp, dcol, dval, db = dev(rp), dev(col), dev(val), dev(w.b)
    print(f"noalloc n={w.n} nnz={col.size}", flush=True)
    st, x, info = noalloc(w.n, drp, dcol, dval, db, tol, maxit)
    assert st == _lib.SLA_OK, _lib.load().sla_last_error()
    A = csr_handle(rp, col, val, rp_dtype=torch.int32)
    xh, ih = A.solve_raw(db, tol, maxit)
    assert info.status == ih.status[0]
    assert abs(info.iterations - ih.iterations[0]) <= 2, (info.iterations, ih.iterations[0])
    assert rel(host(x), host(xh)) <= 1e-8, rel(host(x), host(xh))
    return x, info, ref


def test_two_calls_in_a_row_second_smaller():
    w1 = make_workload("diffusion3d_128", size=64)
    x1, i1, ref1 = against_handle_and_oracle(w1)
    xo, ito, _, oco = oracle.pcg(ref1["row_ptr"], ref1["col"], ref1["vals"], w1.b, w1.tol, w1.maxit)
    assert i1.status == oco == oracle.CONVERGED and abs(i1.iterations - ito) <= 2
    assert rel(host(x1), xo) <= 1e-8
    w2 = make_workload("poisson2d_64")
    x2, i2, ref2 = against_handle_and_oracle(w2)
    xo, ito, _, oco = oracle.pcg(ref2["row_ptr"], ref2["col"], ref2["vals"], w2.b, w2.tol, w2.maxit)
    assert i2.status == oco == oracle.CONVERGED and abs(i2.iterations - ito) <= 2
    assert rel(host(x2), xo) <= 1e-8


def test_largest_system():
    w = make_workload("diffusion3d_128")
    assert w.n == MAX_ROWS
    against_handle_and_oracle(w)


def test_outcomes_and_errors():
    w = make_workload("poisson2d_64")
    rp, col, val, ref = csr_of(w)
    drp, dcol, dval = dev(rp), dev(col), dev(val)
    # budget, zero right-hand side
    st, x, info = noalloc(w.n, drp, dcol, dval, dev(w.b), 1e-14, 7)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, 1e-14, 7)
    assert st == _lib.SLA_OK and info.status == _lib.SLA_MAXIT and info.iterations == ito == 7
    assert rel(host(x), xo) <= 1e-12
    st, x, info = noalloc(w.n, drp, dcol, dval, dev(np.zeros(w.n)), 1e-10, 100)
    assert st == _lib.SLA_OK and info.iterations == 0 and info.status == _lib.SLA_CONVERGED
    assert not host(x).any()
    # more rows than the workspace holds: refused on the host
    big = torch.zeros(MAX_ROWS + 2, dtype=torch.int32, device="cuda:0")
    st, _, _ = noalloc(MAX_ROWS + 1, big, dcol, dval, dev(np.zeros(MAX_ROWS + 1)), 1e-10, 10,
                       nnz=0)
    assert st == _lib.SLA_ERR_INVALID_ARG
    assert b"2^21" in _lib.load().sla_last_error()
    # a column outside [0, n), a decreasing row pointer, a missing diagonal:
    # found by the device check before any solve kernel runs
    bad = col.copy()
    bad[5] = w.n
    st, _, _ = noalloc(w.n, drp, dev(bad), dval, dev(w.b), 1e-10, 10)
    assert st == _lib.SLA_ERR_INDEX_RANGE
    bad_rp = rp.copy()
    bad_rp[10] = bad_rp[12]
    st, _, _ = noalloc(w.n, dev(bad_rp), dcol, dval, dev(w.b), 1e-10, 10)
    assert st == _lib.SLA_ERR_INVALID_CSR
    v0 = val.copy()
    v0[ref["row_ptr"][3] + np.searchsorted(ref["col"][ref["row_ptr"][3]:ref["row_ptr"][4]], 3)] = 0.0
    st, _, _ = noalloc(w.n, drp, dcol, dev(v0), dev(w.b), 1e-10, 10)
    assert st == _lib.SLA_ERR_BAD_DIAGONAL
    # and a good call afterwards still solves correctly
    st, x, info = noalloc(w.n, drp, dcol, dval, dev(w.b), w.tol, w.maxit)
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, w.tol, w.maxit)
    assert st == _lib.SLA_OK and abs(info.iterations - ito) <= 2 and rel(host(x), xo) <= 1e-8

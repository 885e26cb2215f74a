"""Python access to the CPU oracle (oracle.c) — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product package never does.

All index arrays are handed to the C code as int64, values as float64 (fp64
storage) or float32 (fp32 storage, fp64 arithmetic inside). Batched inputs use
a leading batch axis: values [B, nnz], vectors [B, n].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ERR_INVALID_ARG, ERR_INDEX_RANGE, ERR_INVALID_CSR, ERR_BAD_DIAGONAL, ERR_OOM = 0, 1, 2, 3, 5, 6
CONVERGED, MAXIT, BREAKDOWN = 0, 1, 2

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no floating-point contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        L.orc_set_num_threads.restype = None
        L.orc_coo_to_csr.argtypes = [i64, i64, i32, P, P, i32, P, P, P, P, P, P]
        L.orc_check_csr.argtypes = [i64, i64, P, P]
        L.orc_is_symmetric_f64.argtypes = [i64, P, P, P]
        L.orc_spmv_f64.argtypes = [i64, P, P, P, P, P]
        L.orc_spmv_f32.argtypes = [i64, P, P, P, P, P]
        L.orc_spmv_backward_f64.argtypes = [i64, P, P, P, P, P, P, P]
        L.orc_spmv_backward_f64.restype = None
        L.orc_spmv_backward_f32.argtypes = [i64, P, P, P, P, P, P, P]
        L.orc_jacobi_f64.argtypes = [i64, P, P, P, P]
        L.orc_jacobi_f32.argtypes = [i64, P, P, P, P]
        L.orc_pcg_f64.argtypes = [i64, P, P, P, P, f64, i32, P, P, P, P]
        L.orc_pcg_f32.argtypes = [i64, P, P, P, P, f64, i32, P, P, P, P]
        L.orc_pcg_batched.argtypes = [i64, i32, P, P, i32, P, P, f64, i32, P, P, P, P]
        L.orc_adjoint.argtypes = [i64, i32, P, P, i32, P, P, P, f64, i32, P, P, P, P, P]
        L.orc_bicgstab_f64.argtypes = [i64, P, P, P, P, f64, i32, P, P, P, P]
        L.orc_bicgstab_f32.argtypes = [i64, P, P, P, P, f64, i32, P, P, P, P]
        L.orc_bicgstab_adjoint.argtypes = [i64, P, P, i32, P, P, P, f64, i32, P, P, P, P, P]
        for name in ("orc_coo_to_csr", "orc_check_csr", "orc_is_symmetric_f64", "orc_jacobi_f64",
                     "orc_jacobi_f32", "orc_pcg_f64", "orc_pcg_f32", "orc_pcg_batched", "orc_adjoint",
                     "orc_spmv_backward_f32", "orc_bicgstab_f64", "orc_bicgstab_f32",
                     "orc_bicgstab_adjoint"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


def _vals(a, dtype=None) -> np.ndarray:
    a = np.asarray(a)
    if dtype is None:
        dtype = np.float32 if a.dtype == np.float32 else np.float64
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with status {code}")
        self.code = code


def _check(code: int, what: str):
    if code != OK:
        raise OracleError(code, what)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(k: int) -> None:
    """Threads of the oracle's later parallel loops in this thread (results
    do not depend on it)."""
    lib().orc_set_num_threads(int(k))


def coo_to_csr(n: int, rows, cols, vals):
    """Stable (row, col) ordering with duplicates summed in input order.

    Returns dict(row_ptr, col, vals, slot, nnz); ``vals`` keeps the input's
    leading batch axis if it had one.
    """
    rows, cols = _i64(rows), _i64(cols)
    v = _vals(vals)
    batched = v.ndim == 2
    V = v if batched else v[None, :]
    B, nnz_in = V.shape
    row_ptr = np.zeros(n + 1, np.int64)
    col = np.zeros(max(nnz_in, 1), np.int64)
    out = np.zeros((B, max(nnz_in, 1)), V.dtype)
    slot = np.zeros(max(nnz_in, 1), np.int64)
    nnz = ctypes.c_int64(0)
    code = lib().orc_coo_to_csr(n, nnz_in, B, _p(rows), _p(cols), V.dtype.itemsize, _p(V),
                                _p(row_ptr), _p(col), _p(out), _p(slot), ctypes.byref(nnz))
    _check(code, "coo_to_csr")
    m = nnz.value
    vals_out = np.ascontiguousarray(out[:, :m])
    return dict(row_ptr=row_ptr, col=col[:m].copy(), vals=vals_out if batched else vals_out[0],
                slot=slot[:nnz_in].copy(), nnz=m)


def check_csr(n: int, row_ptr, col) -> int:
    row_ptr, col = _i64(row_ptr), _i64(col)
    return int(lib().orc_check_csr(n, col.shape[0], _p(row_ptr), _p(col)))


def is_symmetric(row_ptr, col, val) -> bool:
    row_ptr, col, val = _i64(row_ptr), _i64(col), _vals(val, np.float64)
    res = lib().orc_is_symmetric_f64(row_ptr.shape[0] - 1, _p(row_ptr), _p(col), _p(val))
    if res < 0:
        raise OracleError(ERR_OOM, "is_symmetric")
    return bool(res)


def spmv(row_ptr, col, val, x):
    """y = A x; batched when val is [B, nnz] and x is [B, n]."""
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    x = _vals(x, val.dtype)
    n = row_ptr.shape[0] - 1
    fn = lib().orc_spmv_f32 if val.dtype == np.float32 else lib().orc_spmv_f64
    if val.ndim == 1:
        y = np.empty(n, val.dtype)
        fn(n, _p(row_ptr), _p(col), _p(val), _p(x), _p(y))
        return y
    y = np.empty((val.shape[0], n), val.dtype)
    for s in range(val.shape[0]):
        vs, xs, ys = np.ascontiguousarray(val[s]), np.ascontiguousarray(x[s]), y[s]
        fn(n, _p(row_ptr), _p(col), _p(vs), _p(xs), _p(ys))
    return y


def spmv_backward(row_ptr, col, val, x, g):
    """Backward of y = A x for an upstream gradient g = dL/dy: returns
    (A^T g, grad_vals) with grad_vals[k] = g[row k] * x[col k] in CSR order;
    batched when val is [B, nnz] (x, g [B, n])."""
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    x, g = _vals(x, val.dtype), _vals(g, val.dtype)
    n = row_ptr.shape[0] - 1
    f32 = val.dtype == np.float32

    def one(vs, xs, gs):
        gx = np.empty(n, val.dtype)
        gv = np.empty(vs.shape[0], val.dtype)
        if f32:
            _check(lib().orc_spmv_backward_f32(n, _p(row_ptr), _p(col), _p(vs), _p(xs), _p(gs),
                                               _p(gx), _p(gv)), "spmv_backward")
        else:
            lib().orc_spmv_backward_f64(n, _p(row_ptr), _p(col), _p(vs), _p(xs), _p(gs), _p(gx),
                                        _p(gv))
        return gx, gv

    if val.ndim == 1:
        return one(val, x, g)
    out = [one(np.ascontiguousarray(val[s]), np.ascontiguousarray(x[s]), np.ascontiguousarray(g[s]))
           for s in range(val.shape[0])]
    return np.stack([o[0] for o in out]), np.stack([o[1] for o in out])


def jacobi(row_ptr, col, val):
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    n = row_ptr.shape[0] - 1
    dinv = np.empty(n, val.dtype)
    fn = lib().orc_jacobi_f32 if val.dtype == np.float32 else lib().orc_jacobi_f64
    _check(fn(n, _p(row_ptr), _p(col), _p(val), _p(dinv)), "jacobi")
    return dinv


def pcg(row_ptr, col, val, b, tol: float, maxit: int):
    """Jacobi-PCG. Returns (x, iterations, rel_residual, outcome); arrays per
    system when val is [B, nnz]."""
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    b = _vals(b, val.dtype)
    n = row_ptr.shape[0] - 1
    batched = val.ndim == 2
    V = val if batched else val[None, :]
    Bv = b if batched else b[None, :]
    B = V.shape[0]
    x = np.empty((B, n), val.dtype)
    iters = np.zeros(B, np.int32)
    rel = np.zeros(B, np.float64)
    outc = np.zeros(B, np.int32)
    code = lib().orc_pcg_batched(n, B, _p(row_ptr), _p(col), V.dtype.itemsize, _p(V), _p(Bv),
                                 float(tol), int(maxit), _p(x), _p(iters), _p(rel), _p(outc))
    _check(code, "pcg")
    if batched:
        return x, iters, rel, outc
    return x[0], int(iters[0]), float(rel[0]), int(outc[0])


def adjoint(row_ptr, col, val, x, g, tol: float, maxit: int):
    """Backward of x = A^{-1} b for upstream g: returns (lambda = dL/db,
    grad_vals [CSR order], iterations, rel_residual, outcome)."""
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    x = _vals(x, val.dtype)
    g = _vals(g, val.dtype)
    n = row_ptr.shape[0] - 1
    nnz = col.shape[0]
    batched = val.ndim == 2
    V = val if batched else val[None, :]
    X = x if batched else x[None, :]
    G = g if batched else g[None, :]
    B = V.shape[0]
    lam = np.empty((B, n), val.dtype)
    grad = np.empty((B, nnz), val.dtype)
    iters = np.zeros(B, np.int32)
    rel = np.zeros(B, np.float64)
    outc = np.zeros(B, np.int32)
    code = lib().orc_adjoint(n, B, _p(row_ptr), _p(col), V.dtype.itemsize, _p(V), _p(X), _p(G),
                             float(tol), int(maxit), _p(lam), _p(grad), _p(iters), _p(rel), _p(outc))
    _check(code, "adjoint")
    if batched:
        return lam, grad, iters, rel, outc
    return lam[0], grad[0], int(iters[0]), float(rel[0]), int(outc[0])


def bicgstab(row_ptr, col, val, b, tol: float, maxit: int):
    """Jacobi-preconditioned BiCGStab for a general (non-symmetric) system.
    Returns (x, iterations, rel_residual, outcome)."""
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    b = _vals(b, val.dtype)
    n = row_ptr.shape[0] - 1
    x = np.empty(n, val.dtype)
    it, outc = ctypes.c_int32(0), ctypes.c_int32(0)
    rel = ctypes.c_double(0.0)
    fn = lib().orc_bicgstab_f32 if val.dtype == np.float32 else lib().orc_bicgstab_f64
    _check(fn(n, _p(row_ptr), _p(col), _p(val), _p(b), float(tol), int(maxit), _p(x),
              ctypes.byref(it), ctypes.byref(rel), ctypes.byref(outc)), "bicgstab")
    return x, it.value, rel.value, outc.value


def bicgstab_adjoint(row_ptr, col, val, x, g, tol: float, maxit: int):
    """Backward of x = A^{-1} b solved by BiCGStab, for upstream g: returns
    (lambda = dL/db, grad_vals [CSR order], iterations, rel_residual, outcome)."""
    row_ptr, col = _i64(row_ptr), _i64(col)
    val = _vals(val)
    x, g = _vals(x, val.dtype), _vals(g, val.dtype)
    n = row_ptr.shape[0] - 1
    lam = np.empty(n, val.dtype)
    grad = np.empty(max(col.shape[0], 1), val.dtype)
    it, outc = ctypes.c_int32(0), ctypes.c_int32(0)
    rel = ctypes.c_double(0.0)
    _check(lib().orc_bicgstab_adjoint(n, _p(row_ptr), _p(col), val.dtype.itemsize, _p(val), _p(x),
                                      _p(g), float(tol), int(maxit), _p(lam), _p(grad),
                                      ctypes.byref(it), ctypes.byref(rel), ctypes.byref(outc)),
           "bicgstab_adjoint")
    return lam, grad[:col.shape[0]], it.value, rel.value, outc.value

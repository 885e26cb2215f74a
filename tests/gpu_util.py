"""Helpers shared by the GPU parity tests (host-side marshalling only)."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from differentiable_sparse_linear_csr_amd import _lib, SparseCSR

DEV = "cuda:0"


def dev(a, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def coo_handle(n, rows, cols, vals, idx=torch.int64, check_symmetric=False) -> SparseCSR:
    return SparseCSR.from_coo(dev(rows, idx), dev(cols, idx), dev(vals), n,
                              check_symmetric=check_symmetric)


def csr_handle(row_ptr, cols, vals, rp_dtype=torch.int64, col_dtype=torch.int32) -> SparseCSR:
    return SparseCSR.from_csr(dev(row_ptr, rp_dtype), dev(cols, col_dtype), dev(vals))


def raw_create(fmt, n, nnz_in, batch, a, b, vals, rit, cit, vt):
    """Call sla_csr_create directly; returns (status, handle pointer or None)."""
    L = _lib.load()
    h = ctypes.c_void_p()
    st = L.sla_csr_create(ctypes.byref(h), fmt, n, nnz_in, batch, rit,
                          ctypes.c_void_p(a.data_ptr()), cit, ctypes.c_void_p(b.data_ptr()), vt,
                          ctypes.c_void_p(vals.data_ptr()), 0, None)
    torch.cuda.synchronize()
    if st == 0:
        return st, h
    return st, None


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.dtype == b.dtype and a.shape == b.shape and a.tobytes() == b.tobytes()


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))

"""ctypes binding of libsla.so: argument marshalling only.

The library is loaded from the package directory. If it has not been built,
loading fails with an error; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsla.so")

# status codes (include/sla.h)
SLA_OK = 0
SLA_ERR_INVALID_ARG = 1
SLA_ERR_INDEX_RANGE = 2
SLA_ERR_INVALID_CSR = 3
SLA_ERR_NOT_SYMMETRIC = 4
SLA_ERR_BAD_DIAGONAL = 5
SLA_ERR_OOM = 6
SLA_ERR_HIP = 7
STATUS_NAMES = {0: "SLA_OK", 1: "SLA_ERR_INVALID_ARG", 2: "SLA_ERR_INDEX_RANGE",
                3: "SLA_ERR_INVALID_CSR", 4: "SLA_ERR_NOT_SYMMETRIC", 5: "SLA_ERR_BAD_DIAGONAL",
                6: "SLA_ERR_OOM", 7: "SLA_ERR_HIP"}

SLA_F32, SLA_F64 = 0, 1
SLA_I32, SLA_I64 = 0, 1
SLA_INPUT_COO, SLA_INPUT_CSR = 0, 1
SLA_FLAG_CHECK_SYMMETRIC, SLA_FLAG_REORDER, SLA_FLAG_NO_REORDER = 1, 2, 4
SLA_CONVERGED, SLA_MAXIT, SLA_BREAKDOWN = 0, 1, 2
SLA_OPT_CHECK_INTERVAL, SLA_OPT_USE_GRAPH, SLA_OPT_PROFILE, SLA_OPT_RESIDENT = 1, 2, 3, 4
SLA_OPT_FUSED_UPDATE = 5
SLA_OPT_COOPERATIVE = 6
SLA_OPT_SPIN_LIMIT = 7
SLA_OPT_SPMV_RING = 8
SLA_OPT_FOLD_DIRECTION = 9
SLA_OPT_RESIDENT_WALK = 10
SLA_OPT_RESIDENT_DIA = 11
SLA_OPT_SPMV_DIA = 12
SLA_PATH_NONE, SLA_PATH_SINGLE_KERNEL, SLA_PATH_PER_STEP = 0, 1, 2
SLA_FALLBACK_COOPERATIVE_REFUSED, SLA_FALLBACK_WAIT_TIMED_OUT = 1, 2
KERNELS = {"spmv_dot": 0, "update": 1, "direction": 2, "init": 3, "spmv": 4, "grad": 5,
           "cg_resident": 6}

EXPORTS = ["sla_csr_create", "sla_csr_create_segmented", "sla_csr_get_segments",
           "sla_csr_set_values", "sla_csr_get", "sla_csr_get_pattern",
           "sla_csr_get_values",
           "sla_csr_gather_to_input", "sla_csr_set_option", "sla_spmv", "sla_spmv_backward",
           "sla_pcg_solve", "sla_adjoint_backward", "sla_bicgstab_solve", "sla_bicgstab_adjoint",
           "sla_profile_get", "sla_profile_reset", "sla_csr_memory", "sla_csr_get_layout",
           "sla_csr_get_last_path", "sla_csr_get_diagonals", "sla_csr_destroy", "sla_last_error", "sla_version",
           "sla_pcg_solve_noalloc"]


class SlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Info(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int32), ("status", ctypes.c_int32),
                ("rel_residual", ctypes.c_double)]


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -m differentiable_sparse_linear_csr_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, u32, f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                             ctypes.c_double)
    pP = ctypes.POINTER(ctypes.c_void_p)
    pi64 = ctypes.POINTER(ctypes.c_int64)
    pi32 = ctypes.POINTER(ctypes.c_int32)
    pf64 = ctypes.POINTER(ctypes.c_double)
    L.sla_csr_create.argtypes = [pP, i32, i64, i64, i32, i32, P, i32, P, i32, P, u32, P]
    L.sla_csr_create_segmented.argtypes = [pP, i32, i64, i64, i32, P, i32, P, i32, P, i32, P, u32, P]
    L.sla_csr_get_segments.argtypes = [P, pi32, P]
    L.sla_csr_set_values.argtypes = [P, P, P]
    L.sla_csr_get.argtypes = [P, pi64, pi64, pi64, pi32, pi32, pi32, pP, pP, pP]
    L.sla_csr_get_pattern.argtypes = [P, P, P, P, P]
    L.sla_csr_get_values.argtypes = [P, P, P]
    L.sla_csr_gather_to_input.argtypes = [P, P, P, P]
    L.sla_csr_set_option.argtypes = [P, i32, i64]
    L.sla_spmv.argtypes = [P, P, P, P]
    L.sla_spmv_backward.argtypes = [P, P, P, P, P, P]
    L.sla_pcg_solve.argtypes = [P, P, P, f64, i32, ctypes.POINTER(Info), P]
    L.sla_adjoint_backward.argtypes = [P, P, P, P, P, f64, i32, ctypes.POINTER(Info), P]
    L.sla_bicgstab_solve.argtypes = [P, P, P, f64, i32, ctypes.POINTER(Info), P]
    L.sla_bicgstab_adjoint.argtypes = [P, P, P, P, P, f64, i32, ctypes.POINTER(Info), P]
    L.sla_profile_get.argtypes = [P, i32, pi64, pf64]
    L.sla_profile_reset.argtypes = [P]
    L.sla_csr_memory.argtypes = [P, pi64]
    L.sla_csr_get_layout.argtypes = [P, pi32, pi32, pi64, pi64]
    L.sla_csr_get_last_path.argtypes = [P, pi32, ctypes.POINTER(ctypes.c_uint32)]
    L.sla_csr_get_diagonals.argtypes = [P, pi32, pi32]
    L.sla_pcg_solve_noalloc.argtypes = [i64, i64, P, P, P, P, P, f64, i32, ctypes.POINTER(Info), P]
    L.sla_csr_destroy.argtypes = [P]
    L.sla_csr_destroy.restype = None
    L.sla_last_error.argtypes = []
    L.sla_last_error.restype = ctypes.c_char_p
    L.sla_version.argtypes = []
    L.sla_version.restype = ctypes.c_char_p
    for name in EXPORTS:
        fn = getattr(L, name)
        if name not in ("sla_csr_destroy", "sla_last_error", "sla_version"):
            fn.restype = ctypes.c_int
    _lib = L
    return L


def check(status: int) -> None:
    if status != SLA_OK:
        msg = load().sla_last_error().decode(errors="replace")
        raise SlaError(status, msg)

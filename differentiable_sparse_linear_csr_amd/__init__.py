"""MI355X-native differentiable sparse linear solves on CSR matrices.

Jacobi-preconditioned CG, SpMV and the adjoint backward run in hand-written
HIP kernels for gfx950 (libsla.so, C ABI in include/sla.h); PyTorch supplies
device memory and streams. See :class:`SparseCSR`.
"""
from ._lib import SlaError, LIB_PATH  # noqa: F401
from .sparse import SparseCSR, SparseTensorList, SolveInfo  # noqa: F401
from . import _lib  # noqa: F401


def solve(A: "SparseCSR", b, tol: float = 1e-10, maxit: int = 10000, values=None):
    """Differentiable x = A^{-1} b (gradients to b and to A's values)."""
    return A.solve(b, values=values, tol=tol, maxit=maxit)


__all__ = ["SparseCSR", "SparseTensorList", "SolveInfo", "SlaError", "solve"]

"""Python face of the library: a CSR matrix handle (one matrix or a batch of
value sets sharing one pattern) with .matvec and a differentiable .solve.

Mirrors torch-sla's SparseTensor (tensor-types passage of its API section) and
its autograd wrapping (forward runs the solver and keeps (A, x); backward runs
the adjoint solve; autograd-wrapping paragraph). PyTorch supplies device
memory and the current stream; every step runs in libsla.so.
"""
from __future__ import annotations

import ctypes
import warnings
from typing import List, Optional, Tuple

import torch

from . import _lib
from ._lib import Info, check

_VT = {torch.float32: _lib.SLA_F32, torch.float64: _lib.SLA_F64}
_IT = {torch.int32: _lib.SLA_I32, torch.int64: _lib.SLA_I64}


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[ctypes.c_void_p]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(t: torch.Tensor, what: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


class SolveInfo:
    """Per-system outcome of a solve."""

    def __init__(self, infos: List[Info]):
        self.iterations = [int(i.iterations) for i in infos]
        self.status = [int(i.status) for i in infos]
        self.rel_residual = [float(i.rel_residual) for i in infos]

    def __repr__(self) -> str:
        names = {0: "converged", 1: "maxit", 2: "breakdown"}
        return (f"SolveInfo(iterations={self.iterations}, "
                f"status={[names.get(s, s) for s in self.status]}, "
                f"rel_residual={self.rel_residual})")


class SparseCSR:
    """A CSR matrix (or a batch of value sets on one pattern) on the GPU.

    Build with :meth:`from_coo` or :meth:`from_csr`. ``values`` is [nnz] for
    one matrix or [batch, nnz] for a batch; vectors are [n] or [batch, n].
    """

    def __init__(self, handle: ctypes.c_void_p, device: torch.device, dtype: torch.dtype):
        self._h = handle
        self.device = device
        self.dtype = dtype
        L = _lib.load()
        n, nnz, nnz_in = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        batch, vt, rit = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        rp, ci, sl = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        check(L.sla_csr_get(self._h, ctypes.byref(n), ctypes.byref(nnz), ctypes.byref(nnz_in),
                            ctypes.byref(batch), ctypes.byref(vt), ctypes.byref(rit),
                            ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(sl)))
        self.n, self.nnz, self.nnz_in, self.batch = n.value, nnz.value, nnz_in.value, batch.value
        self.row_index_dtype = torch.int64 if rit.value == _lib.SLA_I64 else torch.int32
        nseg = ctypes.c_int32()
        check(L.sla_csr_get_segments(self._h, ctypes.byref(nseg), None))
        self.nseg = nseg.value
        self.nsys = self.nseg if self.nseg > 0 else self.batch   # entries of a solve's info
        self._values_ref: Optional[torch.Tensor] = None
        self.last_info: Optional[SolveInfo] = None
        self.last_adjoint_info: Optional[SolveInfo] = None

    # ------------------------------------------------------------------ construction
    @classmethod
    def _create(cls, fmt, n, nnz_in, batch, a, b, values, check_symmetric, reorder):
        L = _lib.load()
        dev = values.device
        h = ctypes.c_void_p()
        flags = _lib.SLA_FLAG_CHECK_SYMMETRIC if check_symmetric else 0
        if reorder is True:
            flags |= _lib.SLA_FLAG_REORDER
        elif reorder is False:
            flags |= _lib.SLA_FLAG_NO_REORDER
        with torch.cuda.device(dev):
            check(L.sla_csr_create(ctypes.byref(h), fmt, n, nnz_in, batch, _IT[a.dtype], _ptr(a),
                                   _IT[b.dtype], _ptr(b), _VT[values.dtype], _ptr(values), flags,
                                   _stream(dev)))
        obj = cls(h, dev, values.dtype)
        obj._values_ref = values
        return obj

    @classmethod
    def from_coo(cls, row: torch.Tensor, col: torch.Tensor, values: torch.Tensor, n: int,
                 check_symmetric: bool = False, reorder: Optional[bool] = None) -> "SparseCSR":
        """COO triples; duplicates are summed in input order (stable (row, col) order).
        reorder: None lets the library decide whether the solver runs on a
        reverse Cuthill-McKee permutation (for locality), True/False force it."""
        for t, w in ((row, "row"), (col, "col"), (values, "values")):
            _need_cuda(t, w)
        if values.dtype not in _VT or row.dtype not in _IT or col.dtype not in _IT:
            raise TypeError("values must be float32/float64 and indices int32/int64")
        nnz_in = row.shape[0]
        batch = 1 if values.dim() == 1 else values.shape[0]
        if col.shape[0] != nnz_in or values.shape[-1] != nnz_in:
            raise ValueError("row, col and values disagree on the number of entries")
        return cls._create(_lib.SLA_INPUT_COO, int(n), nnz_in, batch, row, col, values,
                           check_symmetric, reorder)

    @classmethod
    def from_csr(cls, row_ptr: torch.Tensor, col: torch.Tensor, values: torch.Tensor,
                 check_symmetric: bool = False, reorder: Optional[bool] = None) -> "SparseCSR":
        """CSR arrays (columns strictly increasing inside each row), adopted as is."""
        for t, w in ((row_ptr, "row_ptr"), (col, "col"), (values, "values")):
            _need_cuda(t, w)
        if values.dtype not in _VT or row_ptr.dtype not in _IT or col.dtype not in _IT:
            raise TypeError("values must be float32/float64 and indices int32/int64")
        n = row_ptr.shape[0] - 1
        batch = 1 if values.dim() == 1 else values.shape[0]
        return cls._create(_lib.SLA_INPUT_CSR, n, col.shape[0], batch, row_ptr, col, values,
                           check_symmetric, reorder)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.load().sla_csr_destroy(h)
            except Exception:
                pass
            self._h = None

    # ------------------------------------------------------------------ accessors
    def _vec_shape(self) -> Tuple[int, ...]:
        return (self.n,) if self.batch == 1 else (self.batch, self.n)

    def _check_vec(self, v: torch.Tensor, what: str) -> None:
        _need_cuda(v, what)
        if v.dtype != self.dtype:
            raise TypeError(f"{what} must have dtype {self.dtype}")
        if tuple(v.shape) != self._vec_shape():
            raise ValueError(f"{what} must have shape {self._vec_shape()}, got {tuple(v.shape)}")

    def set_values(self, values: torch.Tensor) -> None:
        _need_cuda(values, "values")
        exp = (self.nnz_in,) if self.batch == 1 else (self.batch, self.nnz_in)
        if values.dtype != self.dtype or tuple(values.shape) != exp:
            raise ValueError(f"values must be {self.dtype} of shape {exp}")
        check(_lib.load().sla_csr_set_values(self._h, _ptr(values), _stream(self.device)))
        self._values_ref = values

    def csr(self) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """Copies of (row_ptr, col_idx, values[batch?, nnz]) in CSR order."""
        L = _lib.load()
        row_ptr = torch.empty(self.n + 1, dtype=self.row_index_dtype, device=self.device)
        col = torch.empty(max(self.nnz, 1), dtype=torch.int32, device=self.device)
        vals = torch.empty((self.batch, max(self.nnz, 1)), dtype=self.dtype, device=self.device)
        s = _stream(self.device)
        check(L.sla_csr_get_pattern(self._h, _ptr(row_ptr), _ptr(col), None, s))
        check(L.sla_csr_get_values(self._h, _ptr(vals), s))
        col, vals = col[:self.nnz], vals[:, :self.nnz]
        return row_ptr, col, (vals[0] if self.batch == 1 else vals)

    def slot(self) -> torch.Tensor:
        """input entry -> CSR position (int64 [nnz_in])."""
        out = torch.empty(max(self.nnz_in, 1), dtype=torch.int64, device=self.device)
        check(_lib.load().sla_csr_get_pattern(self._h, None, None, _ptr(out),
                                              _stream(self.device)))
        return out[:self.nnz_in]

    def set_option(self, key: int, value: int) -> None:
        check(_lib.load().sla_csr_set_option(self._h, key, int(value)))

    def memory_bytes(self) -> int:
        b = ctypes.c_int64()
        check(_lib.load().sla_csr_memory(self._h, ctypes.byref(b)))
        return b.value

    def profile(self) -> dict:
        L = _lib.load()
        out = {}
        for name, k in _lib.KERNELS.items():
            n, ms = ctypes.c_int64(), ctypes.c_double()
            check(L.sla_profile_get(self._h, k, ctypes.byref(n), ctypes.byref(ms)))
            out[name] = (n.value, ms.value)
        return out

    def layout(self) -> dict:
        """How the solver holds the matrix: reordered (P A P^T), 16-bit column
        offsets in every SpMV tile, every tile small enough for the four-tile
        pipelined SpMV, tile and long-row counts."""
        r, nc = ctypes.c_int32(), ctypes.c_int32()
        t, lr = ctypes.c_int64(), ctypes.c_int64()
        check(_lib.load().sla_csr_get_layout(self._h, ctypes.byref(r), ctypes.byref(nc),
                                             ctypes.byref(t), ctypes.byref(lr)))
        return {"reordered": bool(r.value), "narrow_columns": bool(nc.value),
                "ring_tiles": nc.value == 2, "tiles": t.value, "long_rows": lr.value}

    def diagonals(self) -> int:
        """Diagonals the single-kernel solve holds the matrix by (0: row
        tiles, or no single-kernel solve yet)."""
        m = ctypes.c_int32()
        check(_lib.load().sla_csr_get_diagonals(self._h, ctypes.byref(m), None))
        return m.value

    def step_diagonals(self) -> int:
        """Diagonals the per-step SpMV reads (0: row tiles)."""
        m = ctypes.c_int32()
        check(_lib.load().sla_csr_get_diagonals(self._h, None, ctypes.byref(m)))
        return m.value

    def profile_reset(self) -> None:
        check(_lib.load().sla_profile_reset(self._h))

    def last_path(self) -> dict:
        """How the last solve ran: path ("none", "single_kernel", "per_step")
        and the fallback bits (cooperative launch refused; a grid-wide wait
        gave up and the solve ran again without it)."""
        p, f = ctypes.c_int32(), ctypes.c_uint32()
        check(_lib.load().sla_csr_get_last_path(self._h, ctypes.byref(p), ctypes.byref(f)))
        return {"path": {0: "none", 1: "single_kernel", 2: "per_step"}[p.value],
                "cooperative_refused": bool(f.value & _lib.SLA_FALLBACK_COOPERATIVE_REFUSED),
                "wait_timed_out": bool(f.value & _lib.SLA_FALLBACK_WAIT_TIMED_OUT)}

    # ------------------------------------------------------------------ operations
    def matvec(self, x: torch.Tensor) -> torch.Tensor:
        """y = A x (no autograd)."""
        self._check_vec(x, "x")
        y = torch.empty_like(x)
        check(_lib.load().sla_spmv(self._h, _ptr(x), _ptr(y), _stream(self.device)))
        return y

    def matvec_backward_raw(self, x: torch.Tensor, grad_y: torch.Tensor, want_x: bool = True,
                            want_vals: bool = True):
        """Backward of y = A x: (A^T grad_y, grad_vals in CSR order); either may be None."""
        self._check_vec(x, "x")
        self._check_vec(grad_y, "grad_y")
        gx = torch.empty_like(x) if want_x else None
        gv = None
        if want_vals:
            shape = (self.nnz,) if self.batch == 1 else (self.batch, self.nnz)
            gv = torch.empty(shape, dtype=self.dtype, device=self.device)
        check(_lib.load().sla_spmv_backward(self._h, _ptr(x), _ptr(grad_y), _ptr(gx), _ptr(gv),
                                            _stream(self.device)))
        return gx, gv

    def mv(self, x: torch.Tensor, values: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Differentiable y = A x: gradients flow to ``x`` and to ``values`` (the
        input-order value tensor this handle was built or last set with, or
        the one passed here, which is loaded into the handle)."""
        vals = self._values_ref if values is None else values
        return _MatvecFn.apply(self, vals, x)

    def solve_raw(self, b: torch.Tensor, tol: float = 1e-10, maxit: int = 10000,
                  out: Optional[torch.Tensor] = None,
                  method: str = "cg") -> Tuple[torch.Tensor, SolveInfo]:
        """x = A^{-1} b (no autograd) by Jacobi-PCG (method "cg", SPD A) or
        Jacobi-BiCGStab (method "bicgstab", general A, one system). Returns
        (x, info)."""
        self._check_vec(b, "b")
        x = torch.empty_like(b) if out is None else out
        infos = (Info * self.nsys)()
        fn = _solver(method)[0]
        check(fn(self._h, _ptr(b), _ptr(x), float(tol), int(maxit), infos, _stream(self.device)))
        info = SolveInfo(list(infos))
        self.last_info = info
        return x, info

    def adjoint_raw(self, x: torch.Tensor, grad_x: torch.Tensor, tol: float = 1e-10,
                    maxit: int = 10000, want_b: bool = True, want_vals: bool = True,
                    method: str = "cg"):
        """(grad_b [like x] or None, grad_vals [batch?, nnz] in CSR order or None, info);
        the adjoint system is solved by the forward solve's method."""
        self._check_vec(x, "x")
        self._check_vec(grad_x, "grad_x")
        gb = torch.empty_like(x) if want_b else None
        gv = None
        if want_vals:
            shape = (self.nnz,) if self.batch == 1 else (self.batch, self.nnz)
            gv = torch.empty(shape, dtype=self.dtype, device=self.device)
        infos = (Info * self.nsys)()
        fn = _solver(method)[1]
        check(fn(self._h, _ptr(x), _ptr(grad_x), _ptr(gb), _ptr(gv), float(tol), int(maxit), infos,
                 _stream(self.device)))
        info = SolveInfo(list(infos))
        self.last_adjoint_info = info
        return gb, gv, info

    def gather_to_input(self, csr_order: torch.Tensor) -> torch.Tensor:
        """[batch?, nnz] CSR order -> [batch?, nnz_in] input order (via the slot map)."""
        shape = (self.nnz_in,) if self.batch == 1 else (self.batch, self.nnz_in)
        out = torch.empty(shape, dtype=self.dtype, device=self.device)
        check(_lib.load().sla_csr_gather_to_input(self._h, _ptr(csr_order), _ptr(out),
                                                  _stream(self.device)))
        return out

    def solve(self, b: torch.Tensor, values: Optional[torch.Tensor] = None, tol: float = 1e-10,
              maxit: int = 10000, adjoint_tol: Optional[float] = None,
              method: str = "cg") -> torch.Tensor:
        """Differentiable x = A^{-1} b: gradients flow to ``b`` and to ``values``
        (the input-order value tensor this handle was built or last set with,
        or the one passed here, which is loaded into the handle). ``method``:
        "cg" (Jacobi-PCG, SPD A) or "bicgstab" (Jacobi-BiCGStab, general A;
        the backward solves A^T lambda = dL/dx with it)."""
        vals = self._values_ref if values is None else values
        return _SolveFn.apply(self, vals, b, float(tol), int(maxit),
                              float(tol if adjoint_tol is None else adjoint_tol), method)


def _solver(method: str):
    L = _lib.load()
    if method == "cg":
        return L.sla_pcg_solve, L.sla_adjoint_backward
    if method == "bicgstab":
        return L.sla_bicgstab_solve, L.sla_bicgstab_adjoint
    raise ValueError(f"unknown method {method!r} (\"cg\" or \"bicgstab\")")


def _report(info: SolveInfo, what: str, method: str = "cg") -> None:
    if any(s == _lib.SLA_BREAKDOWN for s in info.status):
        why = ("PCG breakdown (p.Ap <= 0: matrix not SPD?)" if method == "cg" else
               "BiCGStab breakdown (a zero r^.v, t.t, omega or r^.r)")
        raise FloatingPointError(f"{what}: {why} {info}")
    if any(s == _lib.SLA_MAXIT for s in info.status):
        warnings.warn(f"{what}: iteration budget reached before the tolerance {info}",
                      RuntimeWarning, stacklevel=3)


class _SolveFn(torch.autograd.Function):
    """One autograd node per solve (independent of the iteration count)."""

    @staticmethod
    def forward(ctx, A: SparseCSR, values: torch.Tensor, b: torch.Tensor, tol: float, maxit: int,
                adjoint_tol: float, method: str = "cg"):
        if values is not None and values is not A._values_ref:
            A.set_values(values.detach())
        x, info = A.solve_raw(b.detach(), tol, maxit, method=method)
        _report(info, "solve", method)
        ctx.A = A
        ctx.tol, ctx.maxit, ctx.method = adjoint_tol, maxit, method
        ctx.save_for_backward(x)
        return x

    @staticmethod
    def backward(ctx, grad_x: torch.Tensor):
        (x,) = ctx.saved_tensors
        A: SparseCSR = ctx.A
        want_vals = ctx.needs_input_grad[1]
        want_b = ctx.needs_input_grad[2]
        if not (want_vals or want_b):
            return None, None, None, None, None, None, None
        gb, gv, info = A.adjoint_raw(x, grad_x.contiguous(), ctx.tol, ctx.maxit, want_b=True,
                                     want_vals=want_vals, method=ctx.method)
        _report(info, "adjoint solve", ctx.method)
        g_vals = A.gather_to_input(gv) if want_vals else None
        return None, g_vals, (gb if want_b else None), None, None, None, None


class _MatvecFn(torch.autograd.Function):
    """y = A x as one autograd node: backward is sla_spmv_backward."""

    @staticmethod
    def forward(ctx, A: SparseCSR, values: torch.Tensor, x: torch.Tensor):
        if values is not None and values is not A._values_ref:
            A.set_values(values.detach())
        xd = x.detach().contiguous()
        y = A.matvec(xd)
        ctx.A = A
        ctx.save_for_backward(xd)
        return y

    @staticmethod
    def backward(ctx, grad_y: torch.Tensor):
        (x,) = ctx.saved_tensors
        A: SparseCSR = ctx.A
        want_vals, want_x = ctx.needs_input_grad[1], ctx.needs_input_grad[2]
        if not (want_vals or want_x):
            return None, None, None
        gx, gv = A.matvec_backward_raw(x, grad_y.contiguous(), want_x=want_x, want_vals=want_vals)
        return None, (A.gather_to_input(gv) if want_vals else None), gx


class SparseTensorList(SparseCSR):
    """Independent systems with distinct patterns solved together: one
    block-diagonal handle whose segments each run their own Jacobi-PCG.

    Build with :meth:`from_coo_list`. Vectors are either the concatenation of
    the members' vectors ([sum n_q]) or lists of per-member tensors (``split``
    and ``cat`` convert); ``solve`` takes and returns lists."""

    @classmethod
    def from_coo_list(cls, rows: List[torch.Tensor], cols: List[torch.Tensor],
                      values: List[torch.Tensor], sizes: List[int],
                      check_symmetric: bool = False) -> "SparseTensorList":
        if not (len(rows) == len(cols) == len(values) == len(sizes)) or not sizes:
            raise ValueError("rows, cols, values and sizes must be non-empty lists of one length")
        offs = [0]
        for n in sizes:
            offs.append(offs[-1] + int(n))
        # argument marshalling: member indices shifted to their diagonal block
        r = torch.cat([ri.to(torch.int64) + o for ri, o in zip(rows, offs)])
        c = torch.cat([ci.to(torch.int64) + o for ci, o in zip(cols, offs)])
        v = torch.cat(list(values))
        for t, w in ((r, "rows"), (c, "cols"), (v, "values")):
            _need_cuda(t, w)
        L = _lib.load()
        h = ctypes.c_void_p()
        seg = (ctypes.c_int64 * (len(sizes) + 1))(*offs)
        flags = _lib.SLA_FLAG_CHECK_SYMMETRIC if check_symmetric else 0
        with torch.cuda.device(v.device):
            check(L.sla_csr_create_segmented(ctypes.byref(h), _lib.SLA_INPUT_COO, offs[-1],
                                             r.shape[0], _lib.SLA_I64, _ptr(r), _lib.SLA_I64,
                                             _ptr(c), _VT[v.dtype], _ptr(v), len(sizes), seg,
                                             flags, _stream(v.device)))
        obj = cls(h, v.device, v.dtype)
        obj._values_ref = v
        obj.sizes = [int(n) for n in sizes]
        obj.offsets = offs
        obj.nnz_sizes = [int(t.shape[0]) for t in values]
        return obj

    @classmethod
    def from_block_diagonal_coo(cls, rows: torch.Tensor, cols: torch.Tensor,
                                values: torch.Tensor, seg_rows: List[int],
                                check_symmetric: bool = False) -> "SparseTensorList":
        """COO triples of the block-diagonal matrix itself (indices already
        offset) and the segment row boundaries [0, ..., n]."""
        for t, w in ((rows, "rows"), (cols, "cols"), (values, "values")):
            _need_cuda(t, w)
        L = _lib.load()
        h = ctypes.c_void_p()
        nseg = len(seg_rows) - 1
        seg = (ctypes.c_int64 * (nseg + 1))(*[int(v) for v in seg_rows])
        flags = _lib.SLA_FLAG_CHECK_SYMMETRIC if check_symmetric else 0
        with torch.cuda.device(values.device):
            check(L.sla_csr_create_segmented(ctypes.byref(h), _lib.SLA_INPUT_COO, int(seg_rows[-1]),
                                             rows.shape[0], _IT[rows.dtype], _ptr(rows),
                                             _IT[cols.dtype], _ptr(cols), _VT[values.dtype],
                                             _ptr(values), nseg, seg, flags,
                                             _stream(values.device)))
        obj = cls(h, values.device, values.dtype)
        obj._values_ref = values
        obj.offsets = [int(v) for v in seg_rows]
        obj.sizes = [obj.offsets[q + 1] - obj.offsets[q] for q in range(nseg)]
        obj.nnz_sizes = None
        return obj

    def split(self, v: torch.Tensor) -> List[torch.Tensor]:
        return list(torch.split(v, self.sizes))

    def cat(self, vs: List[torch.Tensor]) -> torch.Tensor:
        return torch.cat(list(vs))

    def split_values(self, v: torch.Tensor) -> List[torch.Tensor]:
        """an input-order value tensor ([sum nnz_q]) -> per-member tensors"""
        return list(torch.split(v, self.nnz_sizes))

    def solve(self, b, values=None, tol: float = 1e-10, maxit: int = 10000,
              adjoint_tol: Optional[float] = None):
        """Differentiable solves of every member: b (list or concatenation) ->
        list of x_q. Gradients flow to b and to the concatenated values."""
        bc = self.cat(b) if isinstance(b, (list, tuple)) else b
        x = super().solve(bc, values=values, tol=tol, maxit=maxit, adjoint_tol=adjoint_tol)
        return self.split(x)

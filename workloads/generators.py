"""Deterministic generators for the five solve workloads and their scaled-down twins.

The workloads follow the benchmark matrices described on the torch-sla page
("torch-sla: Differentiable Sparse Linear Algebra with Adjoint Solvers and
Sparse Tensor Parallelism for PyTorch"): the 2D five-point Poisson problem with
homogeneous Dirichlet boundary of its Figure 2 study (64x64 interior grid), and
large single-GPU / per-GPU shares of the same stencil (Table 3 / Table 4 text).
The pages leave scaling, boundary treatment and coefficients open; the readings
used here are:

* stencils are unscaled: an off-diagonal entry is minus the coefficient of the
  face between the two cells, the diagonal is the sum of all faces of the cell,
  boundary faces included (homogeneous Dirichlet), no 1/h^2 factor;
* variable coefficients live on faces, one value per face, drawn log-uniformly;
* the unstructured workload is an OR-symmetrised 16-nearest-neighbour graph of
  uniform points with Gaussian edge weights exp(-d^2/h^2), h the expected
  16-NN radius (3*16/(4*pi*n))^(1/3), plus 0.01 on the diagonal.

Entries are emitted in row-major order, columns ascending inside a row, with no
duplicates. Right-hand sides are standard normal from numpy's PCG64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def normal_vector(seed: int, shape) -> np.ndarray:
    """Standard-normal float64 array from ``numpy.random.default_rng(seed)``."""
    return np.random.default_rng(seed).standard_normal(shape)


def _log_uniform(rng: np.random.Generator, lo_exp: float, hi_exp: float, shape) -> np.ndarray:
    return 10.0 ** rng.uniform(lo_exp, hi_exp, shape)


# --------------------------------------------------------------------------- 2D unit Poisson

def poisson2d_coo(N: int, index_dtype=np.int32):
    """Unit five-point Laplacian on an N x N interior grid (diag 4, neighbours -1).

    Node (y, x) has index y*N + x. Returns (rows, cols, vals) sorted by (row, col).
    """
    n = N * N
    idx = np.arange(n, dtype=np.int64)
    y, x = np.divmod(idx, N)
    cand = np.stack([idx - N, idx - 1, idx, idx + 1, idx + N], axis=1)
    valid = np.stack([y > 0, x > 0, np.ones(n, bool), x < N - 1, y < N - 1], axis=1)
    vals = np.broadcast_to(np.array([-1.0, -1.0, 4.0, -1.0, -1.0]), cand.shape)
    rows = np.broadcast_to(idx[:, None], cand.shape)[valid].astype(index_dtype)
    cols = cand[valid].astype(index_dtype)
    return rows, cols, np.ascontiguousarray(vals[valid], dtype=np.float64)


def poisson2d_csr(N: int, rowptr_dtype=np.int64, col_dtype=np.int32):
    """Same matrix as :func:`poisson2d_coo`, emitted directly as CSR arrays.

    Built one grid row (N nodes) at a time from three templates (bottom,
    interior and top grid row) broadcast over the grid rows, so that very
    large grids are generated quickly. Entry order and values are identical to
    the COO generator's.
    """
    n = N * N
    nnz = 5 * n - 4 * N
    xs = np.arange(N, dtype=np.int64)

    def template(has_down: bool, has_up: bool):
        cand = np.stack([xs - N, xs - 1, xs, xs + 1, xs + N], axis=1)
        valid = np.stack([np.full(N, has_down), xs > 0, np.ones(N, bool), xs < N - 1,
                          np.full(N, has_up)], axis=1)
        vals = np.broadcast_to(np.array([-1.0, -1.0, 4.0, -1.0, -1.0]), cand.shape)[valid]
        off = np.zeros(N + 1, dtype=np.int64)
        off[1:] = np.cumsum(valid.sum(axis=1))
        return cand[valid], vals, off

    if N == 1:
        return (np.array([0, 1], dtype=rowptr_dtype), np.array([0], dtype=col_dtype),
                np.array([4.0]))
    c_bot, v_bot, o_bot = template(False, True)
    c_mid, v_mid, o_mid = template(True, True)
    c_top, v_top, o_top = template(True, False)
    nb, nm = c_bot.shape[0], c_mid.shape[0]
    cols = np.empty(nnz, dtype=col_dtype)
    vals = np.empty(nnz, dtype=np.float64)
    row_ptr = np.empty(n + 1, dtype=rowptr_dtype)
    # bottom grid row
    cols[:nb] = c_bot
    vals[:nb] = v_bot
    row_ptr[:N] = o_bot[:N]
    # interior grid rows y = 1 .. N-2
    ny = N - 2
    if ny > 0:
        ys = np.arange(1, N - 1, dtype=np.int64)
        mid = cols[nb:nb + ny * nm].reshape(ny, nm)
        np.add(c_mid[None, :], (ys * N)[:, None], out=mid, casting="unsafe")
        vals[nb:nb + ny * nm].reshape(ny, nm)[:] = v_mid[None, :]
        rp_mid = row_ptr[N:N + ny * N].reshape(ny, N)
        np.add(o_mid[None, :N], (nb + (ys - 1) * nm)[:, None], out=rp_mid, casting="unsafe")
    # top grid row
    base = nb + ny * nm
    cols[base:] = c_top + (N - 1) * N
    vals[base:] = v_top
    row_ptr[(N - 1) * N:n] = base + o_top[:N]
    row_ptr[n] = nnz
    assert base + c_top.shape[0] == nnz
    return row_ptr, cols, vals


# --------------------------------------------------------------------------- variable coefficients

def diffusion2d_coo(N: int, cx: np.ndarray, cy: np.ndarray, index_dtype=np.int32):
    """Five-point variable-coefficient diffusion on an N x N grid.

    cx[..., y, x] (shape [..., N, N+1]) is the face to the left of node (y, x);
    cy[..., y, x] (shape [..., N+1, N]) is the face below node (y, x). Leading
    axes are value sets sharing one pattern. Values are computed in float64.
    Returns rows, cols (shared) and vals of shape [..., nnz].
    """
    n = N * N
    lead = cx.shape[:-2]
    idx = np.arange(n, dtype=np.int64)
    y, x = np.divmod(idx, N)
    cxl = cx[..., :, :N].reshape(lead + (n,))       # face left of the node
    cxr = cx[..., :, 1:].reshape(lead + (n,))       # face right of the node
    cyd = cy[..., :N, :].reshape(lead + (n,))       # face below
    cyu = cy[..., 1:, :].reshape(lead + (n,))       # face above
    diag = ((cxl + cxr) + cyd) + cyu
    cand = np.stack([idx - N, idx - 1, idx, idx + 1, idx + N], axis=1)
    valid = np.stack([y > 0, x > 0, np.ones(n, bool), x < N - 1, y < N - 1], axis=1)
    v = np.stack([-cyd, -cxl, diag, -cxr, -cyu], axis=-1)        # [..., n, 5]
    rows = np.broadcast_to(idx[:, None], cand.shape)[valid].astype(index_dtype)
    cols = cand[valid].astype(index_dtype)
    vals = v[..., valid]
    return rows, cols, np.ascontiguousarray(vals)


def convdiff2d_coo(N: int, wx: np.ndarray, wy: np.ndarray, index_dtype=np.int32):
    """Convection-diffusion -Laplace(u) + w . grad(u) on an N x N grid with unit
    spacing, the convection term by first-order upwind differences, Dirichlet
    boundaries (outside neighbours dropped): a non-symmetric, row-wise weakly
    diagonally dominant M-matrix. wx, wy [N, N] are node velocities. Row i:
    diagonal 4 + |wx| + |wy|; west -1 - max(wx, 0), east -1 - max(-wx, 0),
    south -1 - max(wy, 0), north -1 - max(-wy, 0).
    """
    n = N * N
    idx = np.arange(n, dtype=np.int64)
    y, x = np.divmod(idx, N)
    ux, uy = wx.reshape(n), wy.reshape(n)
    diag = (4.0 + np.abs(ux)) + np.abs(uy)
    cand = np.stack([idx - N, idx - 1, idx, idx + 1, idx + N], axis=1)
    valid = np.stack([y > 0, x > 0, np.ones(n, bool), x < N - 1, y < N - 1], axis=1)
    v = np.stack([-1.0 - np.maximum(uy, 0.0), -1.0 - np.maximum(ux, 0.0), diag,
                  -1.0 - np.maximum(-ux, 0.0), -1.0 - np.maximum(-uy, 0.0)], axis=1)
    rows = np.broadcast_to(idx[:, None], cand.shape)[valid].astype(index_dtype)
    cols = cand[valid].astype(index_dtype)
    return rows, cols, np.ascontiguousarray(v[valid])


def rotating_flow(N: int, peak: float):
    """Node velocities of a solid-body rotation about the grid centre, scaled so
    that the largest speed is ``peak`` (cells per unit time)."""
    c = (N - 1) / 2.0
    y, x = np.mgrid[0:N, 0:N].astype(np.float64)
    wx, wy = -(y - c), (x - c)
    scale = peak / max(np.sqrt(wx * wx + wy * wy).max(), 1.0)
    return wx * scale, wy * scale


def diffusion3d_coo(N: int, cx: np.ndarray, cy: np.ndarray, cz: np.ndarray, index_dtype=np.int32):
    """Seven-point variable-coefficient diffusion on an N^3 grid, index z*N*N + y*N + x.

    cx has shape (N, N, N+1) [z][y][x] (face at the low-x side of node x),
    cy (N, N+1, N), cz (N+1, N, N). Boundary faces add to the diagonal only.
    """
    n = N * N * N
    idx = np.arange(n, dtype=np.int64)
    z, rem = np.divmod(idx, N * N)
    y, x = np.divmod(rem, N)
    cxl = cx[:, :, :N].reshape(n)
    cxr = cx[:, :, 1:].reshape(n)
    cyd = cy[:, :N, :].reshape(n)
    cyu = cy[:, 1:, :].reshape(n)
    czd = cz[:N, :, :].reshape(n)
    czu = cz[1:, :, :].reshape(n)
    diag = ((((cxl + cxr) + cyd) + cyu) + czd) + czu
    NN = N * N
    cand = np.stack([idx - NN, idx - N, idx - 1, idx, idx + 1, idx + N, idx + NN], axis=1)
    valid = np.stack([z > 0, y > 0, x > 0, np.ones(n, bool), x < N - 1, y < N - 1, z < N - 1], axis=1)
    v = np.stack([-czd, -cyd, -cxl, diag, -cxr, -cyu, -czu], axis=1)
    rows = np.broadcast_to(idx[:, None], cand.shape)[valid].astype(index_dtype)
    cols = cand[valid].astype(index_dtype)
    return rows, cols, np.ascontiguousarray(v[valid])


# --------------------------------------------------------------------------- kNN graph Laplacian

def knn_laplacian_coo(points: np.ndarray, k: int, h: float, shift: float, index_dtype=np.int32):
    """Graph Laplacian D - W + shift*I of the OR-symmetrised k-NN graph of ``points``.

    w_ij = exp(-d_ij^2 / h^2) with d_ij^2 summed over coordinates in float64.
    The diagonal is the row's weight sum accumulated in ascending column order,
    plus ``shift``.
    """
    from scipy.spatial import cKDTree

    n = points.shape[0]
    tree = cKDTree(points)
    _, nbr = tree.query(points, k=k + 1, workers=-1)
    src = np.repeat(np.arange(n, dtype=np.int64), k)
    dst = nbr[:, 1:].astype(np.int64).ravel()              # drop self (first neighbour)
    keys = np.concatenate([src * n + dst, dst * n + src])
    keys = np.unique(keys)                                   # sorted, OR-symmetrised edge set
    r = keys // n
    c = keys - r * n
    d2 = np.zeros(keys.shape[0], dtype=np.float64)
    for dim in range(points.shape[1]):
        d2 += (points[r, dim] - points[c, dim]) ** 2
    w = np.exp(-d2 / (h * h))
    diag = np.bincount(r, weights=w, minlength=n) + shift
    all_keys = np.concatenate([keys, np.arange(n, dtype=np.int64) * (n + 1)])
    all_vals = np.concatenate([-w, diag])
    order = np.argsort(all_keys, kind="stable")
    all_keys = all_keys[order]
    rows = (all_keys // n).astype(index_dtype)
    cols = (all_keys % n).astype(index_dtype)
    return rows, cols, np.ascontiguousarray(all_vals[order])


# --------------------------------------------------------------------------- workload registry

@dataclass
class Workload:
    name: str
    description: str
    n: int
    batch: int
    dtype: str                    # "f64" or "f32" (storage type of values and vectors)
    fmt: str                      # "coo" or "csr"
    rows: Optional[np.ndarray]    # COO row indices (fmt == "coo")
    row_ptr: Optional[np.ndarray]  # CSR row pointer (fmt == "csr")
    cols: np.ndarray
    vals: np.ndarray              # [nnz] or [batch, nnz]
    b: np.ndarray                 # [n] or [batch, n]
    g: Optional[np.ndarray]       # upstream gradient for the adjoint, same shape as b
    tol: float
    maxit: int
    adjoint: bool
    extra: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.cols.shape[0])


# name -> (seed base, default size)
WORKLOADS = {
    "poisson2d_64": (1000, 64),
    "diffusion3d_128": (2000, 128),
    "batched_diffusion2d_512x32": (3000, 512),
    "knn_laplacian_2m": (4000, 2_000_000),
    "poisson2d_11548": (5000, 11548),
    "list_diffusion2d_16": (6000, 16),
    "convdiff2d_1448": (7000, 1448),
}


def make_workload(name: str, size: Optional[int] = None, batch: Optional[int] = None) -> Workload:
    """Build workload ``name``; ``size`` shrinks the grid edge (or point count) for tests.

    Seeds: with base s, b is drawn from default_rng(s+1), the adjoint's upstream
    gradient from default_rng(s+2), coefficients from default_rng(s+3) and point
    coordinates from default_rng(s+4).
    """
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; choose from {sorted(WORKLOADS)}")
    s, default = WORKLOADS[name]
    N = default if size is None else int(size)

    if name == "poisson2d_64":
        rows, cols, vals = poisson2d_coo(N)
        n = N * N
        return Workload(name, f"2D 5-point Poisson {N}x{N}, Dirichlet, fp64", n, 1, "f64", "coo",
                        rows, None, cols, vals, normal_vector(s + 1, n), normal_vector(s + 2, n),
                        1e-10, 20000, True, {"grid": N})

    if name == "diffusion3d_128":
        rng = np.random.default_rng(s + 3)
        cx = _log_uniform(rng, -1, 1, (N, N, N + 1))
        cy = _log_uniform(rng, -1, 1, (N, N + 1, N))
        cz = _log_uniform(rng, -1, 1, (N + 1, N, N))
        rows, cols, vals = diffusion3d_coo(N, cx, cy, cz)
        n = N ** 3
        return Workload(name, f"3D 7-point variable-coefficient diffusion {N}^3, fp64", n, 1, "f64",
                        "coo", rows, None, cols, vals, normal_vector(s + 1, n),
                        normal_vector(s + 2, n), 1e-10, 20000, True, {"grid": N})

    if name == "batched_diffusion2d_512x32":
        B = 32 if batch is None else int(batch)
        rng = np.random.default_rng(s + 3)
        cx = np.empty((B, N, N + 1))
        cy = np.empty((B, N + 1, N))
        for k in range(B):
            cx[k] = _log_uniform(rng, -2, 2, (N, N + 1))
            cy[k] = _log_uniform(rng, -2, 2, (N + 1, N))
        rows, cols, vals = diffusion2d_coo(N, cx, cy)
        n = N * N
        return Workload(name, f"batched 2D 5-point diffusion {N}x{N}, {B} value sets, fp32", n, B,
                        "f32", "coo", rows, None, cols, vals.astype(np.float32),
                        normal_vector(s + 1, (B, n)).astype(np.float32),
                        normal_vector(s + 2, (B, n)).astype(np.float32), 1e-6, 20000, True,
                        {"grid": N})

    if name == "knn_laplacian_2m":
        n = N
        pts = np.random.default_rng(s + 4).random((n, 3))
        h = (3.0 * 16.0 / (4.0 * math.pi * n)) ** (1.0 / 3.0)
        rows, cols, vals = knn_laplacian_coo(pts, 16, h, 1e-2)
        return Workload(name, f"16-NN Gaussian graph Laplacian + 0.01 I, {n} points, fp64", n, 1,
                        "f64", "coo", rows, None, cols, vals, normal_vector(s + 1, n),
                        normal_vector(s + 2, n), 1e-8, 20000, True, {"h": h})

    if name == "list_diffusion2d_16":
        # a list of systems with distinct patterns (SparseTensorList): member q
        # is 2D 5-point diffusion on a (128 + 16 q)^2 grid (scaled down with
        # size: size members on grids 8 (2 + q)), face coefficients log-uniform in
        # [0.1, 10]; returned as one block-diagonal COO with its segment rows
        M = N
        grids = [128 + 16 * q for q in range(M)] if size is None else [8 * (2 + q) for q in range(M)]
        rng = np.random.default_rng(s + 3)
        rs, cs, vs, seg = [], [], [], [0]
        for G in grids:
            cx = _log_uniform(rng, -1, 1, (G, G + 1))
            cy = _log_uniform(rng, -1, 1, (G + 1, G))
            r, c, v = diffusion2d_coo(G, cx, cy)
            rs.append(r.astype(np.int64) + seg[-1])
            cs.append(c.astype(np.int64) + seg[-1])
            vs.append(v)
            seg.append(seg[-1] + G * G)
        n = seg[-1]
        return Workload(name, f"list of {M} 2D 5-point diffusion grids {grids[0]}^2..{grids[-1]}^2 "
                        "(distinct patterns, one block-diagonal handle), fp64", n, 1, "f64", "coo",
                        np.concatenate(rs), None, np.concatenate(cs), np.concatenate(vs),
                        normal_vector(s + 1, n), normal_vector(s + 2, n), 1e-8, 20000, True,
                        {"seg_rows": seg, "grids": grids})

    if name == "convdiff2d_1448":
        # non-symmetric system for BiCGStab: upwind convection-diffusion in a
        # solid-body rotation (peak speed 4 cells), N^2 = 2.1M unknowns at the
        # default size; fixed iteration budget
        wx, wy = rotating_flow(N, 4.0)
        rows, cols, vals = convdiff2d_coo(N, wx, wy)
        n = N * N
        return Workload(name, f"2D upwind convection-diffusion {N}x{N} (rotating flow, peak "
                        "cell speed 4), non-symmetric, fp64", n, 1, "f64", "coo", rows, None,
                        cols, vals, normal_vector(s + 1, n), normal_vector(s + 2, n), 1e-8, 1000,
                        True, {"grid": N, "method": "bicgstab"})

    # poisson2d_11548: CSR input, int64 row pointer, fixed iteration budget
    row_ptr, cols, vals = poisson2d_csr(N)
    n = N * N
    return Workload(name, f"2D 5-point Poisson {N}x{N}, fp64, int64 row_ptr", n, 1, "f64", "csr",
                    None, row_ptr, cols, vals, normal_vector(s + 1, n), None, 0.0, 500, False,
                    {"grid": N})

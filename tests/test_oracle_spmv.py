"""Pins for the oracle's SpMV (the .matvec of SparseTensor, torch-sla API section).

Checks against a dense product, exact special cases (identity, single-entry
rows, unit-stencil row sums) and the closed-form sine eigenmodes of the
unscaled Dirichlet Laplacian.
"""
import numpy as np
import pytest
import scipy.sparse as sp

import oracle
from workloads import adversarial, make_workload, poisson2d_coo, diffusion3d_coo


def csr_of(n, r, c, v):
    out = oracle.coo_to_csr(n, r, c, v)
    return out["row_ptr"], out["col"], out["vals"]


def test_dense_matvec_random_irregular():
    n = 300
    lengths = np.random.default_rng(0).integers(0, 40, n)
    lengths[[3, 4, 5]] = 0                         # empty rows
    lengths[7] = 299                               # a long row
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=1)
    rp, col, val = csr_of(n, r, c, v)
    x = np.random.default_rng(2).standard_normal(n)
    y = oracle.spmv(rp, col, val, x)
    D = sp.csr_matrix((val, col, rp), shape=(n, n)).toarray()
    yd = D @ x
    scale = np.abs(D) @ np.abs(x)
    assert np.all(np.abs(y - yd) <= 64 * np.finfo(float).eps * scale + 0.0)
    assert np.all(y[[3, 4, 5]] == 0.0)


def test_identity_and_single_entry_exact():
    n = 17
    x = np.random.default_rng(3).standard_normal(n)
    rp, col, val = csr_of(n, np.arange(n), np.arange(n), np.ones(n))
    assert np.array_equal(oracle.spmv(rp, col, val, x), x)
    perm = np.random.default_rng(4).permutation(n)
    w = np.random.default_rng(5).standard_normal(n)
    rp, col, val = csr_of(n, np.arange(n), perm, w)
    assert np.array_equal(oracle.spmv(rp, col, val, x), w * x[perm])


def test_unit_stencil_row_sums_exact():
    N = 13
    r, c, v = poisson2d_coo(N)
    rp, col, val = csr_of(N * N, r, c, v)
    y = oracle.spmv(rp, col, val, np.ones(N * N))
    yy, xx = np.divmod(np.arange(N * N), N)
    boundary_faces = (yy == 0).astype(int) + (yy == N - 1) + (xx == 0) + (xx == N - 1)
    assert np.array_equal(y, boundary_faces.astype(float))


def eig2d(N, j, k):
    h = np.pi / (N + 1)
    iy, ix = np.meshgrid(np.arange(1, N + 1), np.arange(1, N + 1), indexing="ij")
    v = (np.sin(j * iy * h) * np.sin(k * ix * h)).ravel()
    lam = 4 * np.sin(j * h / 2) ** 2 + 4 * np.sin(k * h / 2) ** 2
    return v, lam


def eig3d(N, i, j, k):
    h = np.pi / (N + 1)
    iz, iy, ix = np.meshgrid(*(np.arange(1, N + 1),) * 3, indexing="ij")
    v = (np.sin(i * iz * h) * np.sin(j * iy * h) * np.sin(k * ix * h)).ravel()
    lam = sum(4 * np.sin(m * h / 2) ** 2 for m in (i, j, k))
    return v, lam


@pytest.mark.parametrize("jk", [(1, 1), (3, 5), (20, 7)])
def test_poisson2d_sine_eigenmode(jk):
    N = 32
    r, c, v = poisson2d_coo(N)
    rp, col, val = csr_of(N * N, r, c, v)
    e, lam = eig2d(N, *jk)
    y = oracle.spmv(rp, col, val, e)
    assert np.max(np.abs(y - lam * e)) <= 1e-14 * 8


def test_poisson3d_sine_eigenmode():
    N = 10
    ones = lambda s: np.ones(s)  # noqa: E731
    r, c, v = diffusion3d_coo(N, ones((N, N, N + 1)), ones((N, N + 1, N)), ones((N + 1, N, N)))
    rp, col, val = csr_of(N ** 3, r, c, v)
    assert np.all(val[np.repeat(np.arange(N ** 3), np.diff(rp)) == col] == 6.0)
    e, lam = eig3d(N, 2, 3, 9)
    y = oracle.spmv(rp, col, val, e)
    assert np.max(np.abs(y - lam * e)) <= 1e-14 * 12


def test_fp32_storage_rounds_once():
    n = 200
    r, c, v = adversarial.random_spd_coo(n, 6.0, 9)
    rp, col, val = csr_of(n, r, c, v.astype(np.float32))
    x = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    y = oracle.spmv(rp, col, val, x)
    assert y.dtype == np.float32
    D = sp.csr_matrix((val.astype(np.float64), col, rp), shape=(n, n)).toarray()
    ref = D @ x.astype(np.float64)
    # fp64 accumulation then one rounding: at most 1 ulp from the rounded exact value
    assert np.all(np.abs(y.astype(np.float64) - ref) <= np.spacing(np.abs(ref).astype(np.float32)) + 1e-30)


def test_batched_spmv_equals_per_set():
    w = make_workload("batched_diffusion2d_512x32", size=10, batch=4)
    out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    Y = oracle.spmv(out["row_ptr"], out["col"], out["vals"], w.b)
    for s in range(4):
        assert np.array_equal(Y[s], oracle.spmv(out["row_ptr"], out["col"], out["vals"][s], w.b[s]))

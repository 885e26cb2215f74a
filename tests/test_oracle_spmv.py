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


# ------------------------------------------------------------------ backward of y = A x
# torch-sla lists matvec among the differentiable operations; for an upstream
# gradient g the definitions are dL/dx = A^T g and dL/da_ij = g_i x_j on the
# stored entries.

def test_backward_against_dense_transpose_and_outer_product():
    n = 250
    lengths = np.random.default_rng(20).integers(0, 30, n)
    lengths[[2, 9]] = 0
    lengths[11] = 249
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=21)     # unsymmetric pattern
    rp, col, val = csr_of(n, r, c, v)
    x = np.random.default_rng(22).standard_normal(n)
    g = np.random.default_rng(23).standard_normal(n)
    gx, gv = oracle.spmv_backward(rp, col, val, x, g)
    D = sp.csr_matrix((val, col, rp), shape=(n, n)).toarray()
    scale = np.abs(D).T @ np.abs(g)
    assert np.all(np.abs(gx - D.T @ g) <= 64 * np.finfo(float).eps * scale)
    rows = np.repeat(np.arange(n), np.diff(rp))
    assert np.array_equal(gv, np.outer(g, x)[rows, col])   # one rounded product each
    # a hand-checked 3x3 unsymmetric case: A = [[1,0,2],[0,3,0],[4,0,5]]
    gx3, gv3 = oracle.spmv_backward(np.array([0, 2, 3, 5]), np.array([0, 2, 1, 0, 2]),
                                    np.array([1., 2, 3, 4, 5]), np.array([1., 10, 100]),
                                    np.array([1., 2, 3]))
    assert np.array_equal(gx3, [13., 6., 17.])
    assert np.array_equal(gv3, [1., 100., 20., 3., 300.])


def test_backward_identities_and_finite_differences():
    w = make_workload("diffusion3d_128", size=9)
    rp, col, val = csr_of(w.n, w.rows, w.cols, w.vals)
    x = np.random.default_rng(30).standard_normal(w.n)
    g = np.random.default_rng(31).standard_normal(w.n)
    gx, gv = oracle.spmv_backward(rp, col, val, x, g)
    y = oracle.spmv(rp, col, val, x)
    # <g, A x> = <A^T g, x> = sum_k a_k dL/da_k (the form is bilinear in A)
    L = float(g @ y)
    assert abs(float(gx @ x) - L) <= 1e-12 * (np.abs(g) @ np.abs(y) + 1)
    assert abs(float(gv @ val) - L) <= 1e-12 * (np.abs(g) @ np.abs(y) + 1)
    # central differences of L(a) = g^T A(a) x are exact for a bilinear form
    for k in np.random.default_rng(32).integers(0, val.shape[0], 12):
        vp, vm = val.copy(), val.copy()
        vp[k] += 0.5
        vm[k] -= 0.5
        fd = float(g @ oracle.spmv(rp, col, vp, x) - g @ oracle.spmv(rp, col, vm, x))
        assert abs(fd - gv[k]) <= 1e-12 * (np.abs(g) @ np.abs(y) + 1)
    # and for x: dL/dx_j by central differences
    for j in np.random.default_rng(33).integers(0, w.n, 12):
        xp, xm = x.copy(), x.copy()
        xp[j] += 0.5
        xm[j] -= 0.5
        fd = float(g @ oracle.spmv(rp, col, val, xp) - g @ oracle.spmv(rp, col, val, xm))
        assert abs(fd - gx[j]) <= 1e-12 * (np.abs(g) @ np.abs(y) + 1)


def test_backward_batched_and_fp32():
    w = make_workload("batched_diffusion2d_512x32", size=12, batch=3)
    out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    rp, col, V = out["row_ptr"], out["col"], out["vals"]
    X = np.random.default_rng(40).standard_normal((3, w.n)).astype(np.float32)
    G = np.random.default_rng(41).standard_normal((3, w.n)).astype(np.float32)
    gx, gv = oracle.spmv_backward(rp, col, V, X, G)
    assert gx.dtype == np.float32 and gv.shape == V.shape
    for s in range(3):
        gx64, gv64 = oracle.spmv_backward(rp, col, V[s].astype(np.float64), X[s].astype(np.float64),
                                          G[s].astype(np.float64))
        # fp64 arithmetic rounded once to fp32
        assert np.array_equal(gx[s], gx64.astype(np.float32))
        assert np.array_equal(gv[s], gv64.astype(np.float32))

"""Pins for the oracle's BiCGStab (Jacobi-preconditioned, x0 = 0, shadow
residual b) and its adjoint. torch-sla lists BiCGStab for general systems in
the pytorch-native backend (backend list of the API section); the pages print
no recurrence, so the oracle follows van der Vorst's preconditioned form.

Independent references: SciPy's bicgstab (the same published recurrence, with
M = diag(A)^-1 as a LinearOperator) iterate by iterate; a dense LU solve;
hand-worked 2x2 cases for the two breakdown branches (every quantity there is
a short binary fraction, so the floating-point result is exact); the exact
half-step convergence of a diagonal system; agreement with the oracle's PCG
on an SPD matrix; dense adjoint solves and central finite differences for the
gradient.
"""
import numpy as np
import pytest
import scipy.sparse as sp
import scipy.sparse.linalg as spla

import oracle
from workloads import adversarial, convdiff2d_coo, poisson2d_coo, rotating_flow


def csr_of(n, r, c, v):
    out = oracle.coo_to_csr(n, r, c, v)
    return out["row_ptr"], out["col"], out["vals"]


def dense(rp, col, val):
    n = rp.shape[0] - 1
    return sp.csr_matrix((val, col, rp), shape=(n, n)).toarray()


def convdiff(N, peak=3.0):
    wx, wy = rotating_flow(N, peak)
    return csr_of(N * N, *convdiff2d_coo(N, wx, wy))


def scipy_iterates(rp, col, val, b, k):
    """x after each of the first k BiCGStab iterations (tolerances zero)."""
    A = sp.csr_matrix((val, col, rp), shape=(b.shape[0],) * 2)
    dinv = 1.0 / A.diagonal()
    M = spla.LinearOperator(A.shape, matvec=lambda v: dinv * v, dtype=np.float64)
    xs = []
    spla.bicgstab(A, b, rtol=0.0, atol=0.0, maxiter=k, M=M, callback=lambda x: xs.append(x.copy()))
    return xs


def test_iterates_match_scipy():
    rp, col, val = convdiff(12)
    b = np.random.default_rng(1).standard_normal(144)
    ref = scipy_iterates(rp, col, val, b, 12)
    assert len(ref) == 12
    for k in range(1, 13):
        x, it, _, oc = oracle.bicgstab(rp, col, val, b, 0.0, k)
        assert (it, oc) == (k, oracle.MAXIT)
        err = np.linalg.norm(x - ref[k - 1]) / np.linalg.norm(ref[k - 1])
        assert err <= 1e-11, (k, err)


def test_irregular_unsymmetric_matches_scipy():
    n = 400
    lengths = np.random.default_rng(2).integers(0, 6, n)
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=3)
    # add a dominant diagonal of mixed sign
    d = np.where(np.random.default_rng(4).random(n) < 0.5, -1.0, 1.0) * (8.0 + np.arange(n) % 3)
    r = np.concatenate([r, np.arange(n)])
    c = np.concatenate([c, np.arange(n)])
    v = np.concatenate([v, d])
    rp, col, val = csr_of(n, r, c, v)
    b = np.random.default_rng(5).standard_normal(n)
    ref = scipy_iterates(rp, col, val, b, 6)
    for k in (1, 2, 6):
        x, *_ = oracle.bicgstab(rp, col, val, b, 0.0, k)
        assert np.linalg.norm(x - ref[k - 1]) <= 1e-12 * np.linalg.norm(ref[k - 1])


def test_converged_solution_against_dense_lu():
    rp, col, val = convdiff(16)
    n = 256
    b = np.random.default_rng(6).standard_normal(n)
    tol = 1e-11
    x, it, rel, oc = oracle.bicgstab(rp, col, val, b, tol, 2000)
    assert oc == oracle.CONVERGED and 1 < it < 2000 and rel <= tol
    A = dense(rp, col, val)
    xs = np.linalg.solve(A, b)
    cond = np.linalg.cond(A)
    assert np.linalg.norm(x - xs) <= 10 * cond * tol * np.linalg.norm(xs)
    # the true residual, formed densely, is near the recurrence's
    assert np.linalg.norm(b - A @ x) <= 10 * tol * np.linalg.norm(b)


def test_diagonal_system_converges_at_the_first_half_step():
    n = 50
    d = np.linspace(-5.0, 7.0, n)
    d[d == 0] = 1.0
    b = np.random.default_rng(7).standard_normal(n)
    rp, col, val = csr_of(n, np.arange(n), np.arange(n), d)
    x, it, rel, oc = oracle.bicgstab(rp, col, val, b, 1e-12, 10)
    assert (it, oc) == (1, oracle.CONVERGED)
    assert np.allclose(x, b / d, rtol=1e-14, atol=0)


def test_breakdown_at_sigma_keeps_x():
    # A = [[1, 0], [-2, 1]], b = (1, 1): p^ = b, v = A b = (1, -1), r^.v = 0
    rp, col, val = csr_of(2, [0, 1, 1], [0, 0, 1], [1.0, -2.0, 1.0])
    x, it, rel, oc = oracle.bicgstab(rp, col, val, np.array([1.0, 1.0]), 1e-10, 50)
    assert (it, oc) == (1, oracle.BREAKDOWN)
    assert not x.any() and rel == 1.0


def test_breakdown_at_omega_keeps_the_half_step():
    # A = [[1, -3], [-1, -1]] (negative diagonal), b = (-3, -3):
    # p^ = D^-1 b = (-3, 3), v = A p^ = (-12, 0), r^.v = 36, alpha = 18/36 = 1/2,
    # s = b - v/2 = (3, -3), s^ = (3, 3), t = A s^ = (-6, -6), t.s = 0 -> omega = 0
    rp, col, val = csr_of(2, [0, 0, 1, 1], [0, 1, 0, 1], [1.0, -3.0, -1.0, -1.0])
    b = np.array([-3.0, -3.0])
    x, it, rel, oc = oracle.bicgstab(rp, col, val, b, 1e-10, 50)
    assert (it, oc) == (1, oracle.BREAKDOWN)
    assert np.array_equal(x, [-1.5, 1.5])          # x = alpha p^
    assert rel == 1.0                              # ||s|| = ||b||


def test_zero_rhs_and_zero_budget():
    rp, col, val = convdiff(6)
    x, it, rel, oc = oracle.bicgstab(rp, col, val, np.zeros(36), 1e-8, 100)
    assert (it, oc, rel) == (0, oracle.CONVERGED, 0.0) and not x.any()
    b = np.ones(36)
    x, it, rel, oc = oracle.bicgstab(rp, col, val, b, 1e-8, 0)
    assert (it, oc, rel) == (0, oracle.MAXIT, 1.0) and not x.any()


def test_missing_or_zero_diagonal_is_rejected():
    rp, col, val = csr_of(2, [0, 1], [1, 0], [1.0, 1.0])
    with pytest.raises(oracle.OracleError) as e:
        oracle.bicgstab(rp, col, val, np.ones(2), 1e-8, 10)
    assert e.value.code == oracle.ERR_BAD_DIAGONAL
    rp, col, val = csr_of(2, [0, 1, 1], [0, 0, 1], [0.0, 1.0, 1.0])
    with pytest.raises(oracle.OracleError):
        oracle.bicgstab(rp, col, val, np.ones(2), 1e-8, 10)


def test_spd_system_agrees_with_pcg():
    r, c, v = poisson2d_coo(20)
    rp, col, val = csr_of(400, r, c, v)
    b = np.random.default_rng(8).standard_normal(400)
    xb, itb, _, ocb = oracle.bicgstab(rp, col, val, b, 1e-12, 1000)
    xp, itp, _, ocp = oracle.pcg(rp, col, val, b, 1e-12, 1000)
    assert ocb == ocp == oracle.CONVERGED
    assert np.linalg.norm(xb - xp) <= 1e-9 * np.linalg.norm(xp)


def test_fp32_storage_tracks_fp64():
    rp, col, val = convdiff(20)
    b = np.random.default_rng(9).standard_normal(400)
    x64, *_ = oracle.bicgstab(rp, col, val, b, 0.0, 8)
    x32, it, _, oc = oracle.bicgstab(rp, col, val.astype(np.float32), b.astype(np.float32), 0.0, 8)
    assert x32.dtype == np.float32 and (it, oc) == (8, oracle.MAXIT)
    assert np.linalg.norm(x32 - x64) <= 1e-5 * np.linalg.norm(x64)
    x32, it, rel, oc = oracle.bicgstab(rp, col, val.astype(np.float32), b.astype(np.float32),
                                       1e-5, 1000)
    assert oc == oracle.CONVERGED and rel <= 1e-5


def test_adjoint_against_dense_solves_and_finite_differences():
    rp, col, val = convdiff(5, peak=4.0)
    n = 25
    A = dense(rp, col, val)
    assert not np.allclose(A, A.T)
    b = np.random.default_rng(10).standard_normal(n)
    w = np.random.default_rng(11).standard_normal(n)
    tol = 1e-13
    x, *_ = oracle.bicgstab(rp, col, val, b, tol, 500)
    lam, gv, it, rel, oc = oracle.bicgstab_adjoint(rp, col, val, x, w, tol, 500)
    assert oc == oracle.CONVERGED
    assert np.linalg.norm(lam - np.linalg.solve(A.T, w)) <= 1e-10 * np.linalg.norm(lam)
    # L(vals) = w . A(vals)^-1 b, central differences through dense LU
    rows = np.repeat(np.arange(n), np.diff(rp))
    h = 1e-6
    fd = np.empty(val.shape[0])
    for k in range(val.shape[0]):
        vp, vm = val.copy(), val.copy()
        vp[k] += h
        vm[k] -= h
        fd[k] = (w @ np.linalg.solve(dense(rp, col, vp), b) -
                 w @ np.linalg.solve(dense(rp, col, vm), b)) / (2 * h)
    assert np.max(np.abs(gv - fd)) <= 1e-6 * np.max(np.abs(fd))
    # orientation: dL/dA_ij = -lambda_i x_j, not -lambda_j x_i
    assert np.max(np.abs(gv + lam[rows] * x[col])) <= 1e-14 * np.max(np.abs(gv))


def test_fp32_adjoint_tracks_fp64():
    rp, col, val = convdiff(10, peak=4.0)
    b = np.random.default_rng(12).standard_normal(100)
    w = np.random.default_rng(13).standard_normal(100)
    x, *_ = oracle.bicgstab(rp, col, val, b, 1e-12, 1000)
    lam, gv, *_ = oracle.bicgstab_adjoint(rp, col, val, x, w, 1e-12, 1000)
    f = np.float32
    lam32, gv32, it, rel, oc = oracle.bicgstab_adjoint(rp, col, val.astype(f), x.astype(f),
                                                       w.astype(f), 1e-6, 1000)
    assert lam32.dtype == gv32.dtype == np.float32 and oc == oracle.CONVERGED
    assert np.linalg.norm(lam32 - lam) <= 1e-4 * np.linalg.norm(lam)
    assert np.linalg.norm(gv32 - gv) <= 1e-4 * np.linalg.norm(gv)

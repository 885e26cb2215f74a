"""Pins for the oracle's Jacobi-preconditioned CG (pytorch-native CG backend with
Jacobi preconditioning, torch-sla backend list and Table 3 / Table 4 text).

Independent references: dense LU, closed-form eigenmodes (one iteration), CG's
finite termination in (#distinct eigenvalues) steps, SciPy's cg iteration
counts, condition-number growth, exact special cases and outcome codes.
"""
import numpy as np
import pytest
import scipy.sparse as sp
import scipy.sparse.linalg as spla

import oracle
from workloads import adversarial, make_workload, poisson2d_coo


def csr_of(n, r, c, v):
    out = oracle.coo_to_csr(n, r, c, v)
    return out["row_ptr"], out["col"], out["vals"]


def dense(rp, col, val):
    n = rp.shape[0] - 1
    return sp.csr_matrix((val, col, rp), shape=(n, n)).toarray()


@pytest.mark.parametrize("case", ["poisson16", "spd300", "poisson64"])
def test_matches_dense_lu(case):
    if case == "poisson16":
        r, c, v = poisson2d_coo(16)
        n = 256
    elif case == "poisson64":
        r, c, v = poisson2d_coo(64)
        n = 4096
    else:
        n = 300
        r, c, v = adversarial.random_spd_coo(n, 8.0, 21, max_row=120)
    rp, col, val = csr_of(n, r, c, v)
    b = np.random.default_rng(1).standard_normal(n)
    tol = 1e-10
    x, it, rel, outc = oracle.pcg(rp, col, val, b, tol, 10000)
    assert outc == oracle.CONVERGED
    D = dense(rp, col, val)
    xl = np.linalg.solve(D, b)
    kappa = np.linalg.cond(D)
    assert np.linalg.norm(x - xl) / np.linalg.norm(xl) <= kappa * tol * 2
    assert rel <= tol
    # recursive residual tracks the true residual
    true_rel = np.linalg.norm(b - D @ x) / np.linalg.norm(b)
    assert true_rel <= 10 * tol


@pytest.mark.parametrize("jk", [(1, 1), (3, 5), (11, 2)])
def test_eigenmode_converges_in_one_iteration(jk):
    N = 24
    r, c, v = poisson2d_coo(N)
    rp, col, val = csr_of(N * N, r, c, v)
    h = np.pi / (N + 1)
    iy, ix = np.meshgrid(np.arange(1, N + 1), np.arange(1, N + 1), indexing="ij")
    e = (np.sin(jk[0] * iy * h) * np.sin(jk[1] * ix * h)).ravel()
    lam = 4 * np.sin(jk[0] * h / 2) ** 2 + 4 * np.sin(jk[1] * h / 2) ** 2
    x, it, rel, outc = oracle.pcg(rp, col, val, e, 1e-12, 100)
    assert it == 1 and outc == oracle.CONVERGED
    assert np.linalg.norm(x - e / lam) / np.linalg.norm(e / lam) <= 1e-14


def test_finite_termination_distinct_eigenvalues():
    # 3x3 grid: eigenvalues 4 sin^2(j pi/8) + 4 sin^2(k pi/8), j,k in 1..3 -> 5 distinct values
    r, c, v = poisson2d_coo(3)
    rp, col, val = csr_of(9, r, c, v)
    lam = np.linalg.eigvalsh(dense(rp, col, val))
    assert len(np.unique(np.round(lam, 12))) == 5
    b = np.random.default_rng(0).standard_normal(9)
    x, it, rel, outc = oracle.pcg(rp, col, val, b, 1e-13, 100)
    assert outc == oracle.CONVERGED and it <= 5
    assert np.linalg.norm(x - np.linalg.solve(dense(rp, col, val), b)) <= 1e-13 * np.linalg.norm(x)


def scipy_cg_iterations(rp, col, val, b, tol, maxit):
    n = rp.shape[0] - 1
    A = sp.csr_matrix((val, col, rp), shape=(n, n))
    dinv = 1.0 / A.diagonal()
    M = spla.LinearOperator((n, n), matvec=lambda y: dinv * y)
    count = [0]

    def cb(_):
        count[0] += 1

    x, info = spla.cg(A, b, rtol=tol, atol=0.0, maxiter=maxit, M=M, callback=cb)
    return count[0], x


@pytest.mark.parametrize("name,size,tol", [("poisson2d_64", None, 1e-10),
                                           ("diffusion3d_128", 16, 1e-10),
                                           ("knn_laplacian_2m", 5000, 1e-8),
                                           ("batched_diffusion2d_512x32", 24, 1e-6)])
def test_iteration_count_matches_scipy_cg(name, size, tol):
    w = make_workload(name, size=size, batch=1 if name.startswith("batched") else None)
    vals = w.vals if w.vals.ndim == 1 else w.vals[0].astype(np.float64)
    b = w.b if w.b.ndim == 1 else w.b[0].astype(np.float64)
    rp, col, val = csr_of(w.n, w.rows, w.cols, vals)
    x, it, rel, outc = oracle.pcg(rp, col, val, b, tol, 20000)
    it_sp, x_sp = scipy_cg_iterations(rp, col, val, b, tol, 20000)
    assert outc == oracle.CONVERGED
    assert abs(it - it_sp) <= 1, (it, it_sp)
    assert np.linalg.norm(x - x_sp) / np.linalg.norm(x) <= 1e-6


def test_generators_are_symmetric():
    for name, size in [("poisson2d_64", None), ("diffusion3d_128", 12), ("knn_laplacian_2m", 4000)]:
        w = make_workload(name, size=size)
        rp, col, val = csr_of(w.n, w.rows, w.cols, w.vals)
        assert oracle.is_symmetric(rp, col, val), name
    w = make_workload("batched_diffusion2d_512x32", size=16, batch=3)
    out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    for s in range(3):
        assert oracle.is_symmetric(out["row_ptr"], out["col"], out["vals"][s].astype(np.float64))
    # and a planted one-ulp asymmetry in an off-diagonal entry is seen
    val = out["vals"][0].astype(np.float64).copy()
    rows_of = np.repeat(np.arange(w.n), np.diff(out["row_ptr"]))
    k = int(np.nonzero(rows_of != out["col"])[0][7])
    val[k] = np.nextafter(val[k], 0.0)
    assert not oracle.is_symmetric(out["row_ptr"], out["col"], val)


def test_iterations_grow_like_grid_edge():
    # kappa ~ n for 2D Poisson under Jacobi (Table 3 text) => iterations ~ sqrt(kappa) ~ N
    its = []
    for N in (16, 32, 64):
        r, c, v = poisson2d_coo(N)
        rp, col, val = csr_of(N * N, r, c, v)
        b = np.random.default_rng(N).standard_normal(N * N)
        its.append(oracle.pcg(rp, col, val, b, 1e-10, 10000)[1])
    assert 1.5 <= its[1] / its[0] <= 2.5 and 1.5 <= its[2] / its[1] <= 2.5


def test_outcomes_and_special_cases():
    r, c, v = poisson2d_coo(8)
    rp, col, val = csr_of(64, r, c, v)
    b = np.random.default_rng(0).standard_normal(64)
    # zero rhs: x = 0 after 0 iterations
    x, it, rel, outc = oracle.pcg(rp, col, val, np.zeros(64), 1e-10, 100)
    assert it == 0 and outc == oracle.CONVERGED and not x.any()
    # iteration budget
    x, it, rel, outc = oracle.pcg(rp, col, val, b, 1e-14, 3)
    assert it == 3 and outc == oracle.MAXIT and rel > 1e-14
    x0, it0, rel0, outc0 = oracle.pcg(rp, col, val, b, 1e-10, 0)
    assert it0 == 0 and outc0 == oracle.MAXIT and not x0.any() and rel0 == 1.0
    # tol 0 runs the whole budget
    assert oracle.pcg(rp, col, val, b, 0.0, 40)[1] == 40
    # indefinite: [[1,2],[2,1]] with b = (1,-1) gives p.Ap = -2 at the first step
    rp2, col2, val2 = csr_of(2, np.array([0, 0, 1, 1]), np.array([0, 1, 0, 1]),
                             np.array([1.0, 2.0, 2.0, 1.0]))
    x, it, rel, outc = oracle.pcg(rp2, col2, val2, np.array([1.0, -1.0]), 1e-10, 10)
    assert outc == oracle.BREAKDOWN and it == 1 and not x.any()
    # bad diagonals: zero, negative, NaN, missing
    for bad in (0.0, -1.0, np.nan):
        v2 = val.copy()
        v2[np.searchsorted(col[rp[3]:rp[4]], 3) + rp[3]] = bad
        with pytest.raises(oracle.OracleError) as e:
            oracle.pcg(rp, col, v2, b, 1e-10, 10)
        assert e.value.code == oracle.ERR_BAD_DIAGONAL
    keep = ~((r == 5) & (c == 5))
    rp3, col3, val3 = csr_of(64, r[keep], c[keep], v[keep])
    with pytest.raises(oracle.OracleError):
        oracle.pcg(rp3, col3, val3, b, 1e-10, 10)


def test_scaling_invariance_of_iterates():
    # Jacobi-PCG iterates are invariant under A -> cA with x -> x/c (c a power of 2: exact)
    r, c, v = poisson2d_coo(20)
    rp, col, val = csr_of(400, r, c, v)
    b = np.random.default_rng(2).standard_normal(400)
    x1, it1, rel1, _ = oracle.pcg(rp, col, val, b, 1e-10, 1000)
    x2, it2, rel2, _ = oracle.pcg(rp, col, val * 8.0, b, 1e-10, 1000)
    assert it1 == it2 and rel1 == rel2 and np.array_equal(x1, x2 * 8.0)


def test_fp32_storage_close_to_fp64():
    w = make_workload("batched_diffusion2d_512x32", size=32, batch=2)
    out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    x32, it32, rel32, oc32 = oracle.pcg(out["row_ptr"], out["col"], out["vals"], w.b, 1e-6, 20000)
    assert x32.dtype == np.float32 and np.all(oc32 == oracle.CONVERGED) and np.all(rel32 <= 1e-6)
    for s in range(2):
        D = dense(out["row_ptr"], out["col"], out["vals"][s].astype(np.float64))
        xl = np.linalg.solve(D, w.b[s].astype(np.float64))
        assert np.linalg.norm(x32[s] - xl) / np.linalg.norm(xl) <= 1e-3


def test_batched_slices_equal_single_solves_bitwise():
    w = make_workload("batched_diffusion2d_512x32", size=20, batch=5)
    out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    X, its, rels, outs = oracle.pcg(out["row_ptr"], out["col"], out["vals"], w.b, 1e-6, 20000)
    for s in range(5):
        x, it, rel, oc = oracle.pcg(out["row_ptr"], out["col"], out["vals"][s], w.b[s], 1e-6, 20000)
        assert np.array_equal(x, X[s]) and it == its[s] and rel == rels[s] and oc == outs[s]

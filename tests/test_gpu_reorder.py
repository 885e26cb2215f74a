"""GPU parity of the reordered solver (P A P^T with a reverse Cuthill-McKee P):
every call takes and returns the caller's order, so results are compared with
the oracle on A itself, to the same bars as the unpermuted path: SpMV 1e-12
(fp64) / 1e-5 (fp32) normwise, iterations within +-2, x within 1e-8 (fp32
1e-4), lambda and grad_vals within 1e-8 (fp32 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
from differentiable_sparse_linear_csr_amd import SparseCSR
from workloads import adversarial, make_workload

from gpu_util import dev, host, rel

pytestmark = pytest.mark.gpu


def handle(n, r, c, v, reorder):
    return SparseCSR.from_coo(dev(r, torch.int64), dev(c, torch.int64), dev(v), n, reorder=reorder)


@pytest.mark.parametrize("dtype,B", [(np.float64, 1), (np.float32, 1), (np.float64, 3),
                                     (np.float32, 8)])
def test_spmv_on_unsymmetric_pattern(dtype, B):
    # rows of prescribed lengths with random columns (pattern not symmetric),
    # empty rows and a long row
    n = 30011
    lengths = np.random.default_rng(1).integers(0, 14, n)
    lengths[[0, 17]] = 0
    lengths[5000] = 900
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=2)
    V = np.random.default_rng(3).standard_normal((B, v.shape[0])).astype(dtype)
    x = np.random.default_rng(4).standard_normal((B, n)).astype(dtype)
    A = handle(n, r, c, V if B > 1 else V[0], True)
    assert A.layout()["reordered"]
    ref = oracle.coo_to_csr(n, r, c, V if B > 1 else V[0])
    y_ref = np.atleast_2d(oracle.spmv(ref["row_ptr"], ref["col"], ref["vals"], x if B > 1 else x[0]))
    y = np.atleast_2d(host(A.matvec(dev(x if B > 1 else x[0]))))
    tol = 1e-12 if dtype == np.float64 else 1e-5
    for s in range(B):
        assert rel(y[s], y_ref[s]) <= tol, (s, rel(y[s], y_ref[s]))


@pytest.mark.parametrize("name,size,batch", [("knn_laplacian_2m", 70000, None),
                                             ("diffusion3d_128", 30, None),
                                             ("batched_diffusion2d_512x32", 40, 4)])
def test_solve_and_adjoint_match_oracle(name, size, batch):
    w = make_workload(name, size=size, batch=batch)
    print(f"reordered {name} n={w.n} nnz={w.nnz} batch={w.batch}", flush=True)
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, w.tol, w.maxit)
    lam_o, gv_o, *_ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, w.g, w.tol, w.maxit)
    A = handle(w.n, w.rows, w.cols, w.vals, True)
    assert A.layout()["reordered"]
    x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    gb, gv, ainfo = A.adjoint_raw(x, dev(w.g), w.tol, w.maxit)
    X, GB, GV = (np.atleast_2d(host(t)) for t in (x, gb, gv))
    XO, LO, GO = (np.atleast_2d(t) for t in (xo, lam_o, gv_o))
    ito, oco = np.atleast_1d(ito), np.atleast_1d(oco)
    xtol = 1e-8 if w.dtype == "f64" else 1e-4
    gtol = 1e-8 if w.dtype == "f64" else 1e-3
    for s in range(w.batch):
        assert info.status[s] == oco[s] == oracle.CONVERGED
        assert abs(info.iterations[s] - ito[s]) <= 2, (s, info.iterations[s], ito[s])
        assert rel(X[s], XO[s]) <= xtol, (s, rel(X[s], XO[s]))
        assert rel(GB[s], LO[s]) <= gtol
        assert rel(GV[s], GO[s]) <= gtol


def test_set_values_reach_the_reordered_solver():
    # duplicated, shuffled COO input; new values after create
    n = 20000
    r, c, v = adversarial.random_spd_coo(n, 10.0, 7, skew=False)
    r, c, v = adversarial.split_duplicates(r, c, v, seed=8, frac=0.2)   # also shuffles
    A = handle(n, r, c, v, True)
    # new values D A D (D positive diagonal): symmetric positive definite again
    s = np.random.default_rng(11).uniform(0.5, 2.0, n)
    v2 = v * s[r] * s[c]
    A.set_values(dev(v2))
    ref = oracle.coo_to_csr(n, r, c, v2)
    b = np.random.default_rng(12).standard_normal(n)
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 5000)
    x, info = A.solve_raw(dev(b), 1e-10, 5000)
    assert abs(info.iterations[0] - ito) <= 2
    assert rel(host(x), xo) <= 1e-8
    g = np.random.default_rng(13).standard_normal(n)
    _, gv_o, *_ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, 1e-10, 5000)
    _, gv, _ = A.adjoint_raw(x, dev(g), 1e-10, 5000)
    assert rel(host(gv), gv_o) <= 1e-8
    # gradient in input order through the caller's slot map
    gin = host(A.gather_to_input(gv))
    assert np.array_equal(gin, host(gv)[host(A.slot())])


def test_automatic_choice():
    w = make_workload("knn_laplacian_2m", size=100000)     # scattered gathers, n >= 2^16
    assert handle(w.n, w.rows, w.cols, w.vals, None).layout()["reordered"]
    assert not handle(w.n, w.rows, w.cols, w.vals, False).layout()["reordered"]
    w = make_workload("diffusion3d_128", size=48)           # banded already
    assert not handle(w.n, w.rows, w.cols, w.vals, None).layout()["reordered"]

"""GPU BiCGStab (sla_bicgstab_solve / sla_bicgstab_adjoint) against the
oracle's BiCGStab and its adjoint.

Element-wise parity is taken on the first k iterates (tol 0, maxit k): both
sides run the same recurrence and differ only in the summation order of the
inner products (and fused multiply-adds on the device), so after k <= 12
iterations the iterates agree to 1e-9 relative in fp64 and 1e-4 with fp32
storage. Converged solves are compared by outcome, iteration count (within 5%
or 3: the order of rounding shifts when the test first passes) and solution,
whose distance is bounded by the two residuals: ||x - x'|| <= cond(A) (tol +
tol') ||b|| / ||A||, checked as ||A (x - x')|| <= 2.5 tol ||b||. The two-by-two
breakdown cases and the diagonal half step are exact in floating point, so
they are compared exactly.
"""
import numpy as np
import pytest
import scipy.sparse as sp
import torch

import oracle
from differentiable_sparse_linear_csr_amd import SlaError, SparseCSR, _lib
from workloads import adversarial, convdiff2d_coo, make_workload, poisson2d_coo, rotating_flow

from gpu_util import dev, host, rel

pytestmark = pytest.mark.gpu


def convdiff(N, peak=3.0):
    wx, wy = rotating_flow(N, peak)
    return convdiff2d_coo(N, wx, wy)


def handle(n, r, c, v, **kw):
    return SparseCSR.from_coo(dev(r, torch.int64), dev(c, torch.int64), dev(v), n, **kw)


def irregular(n, seed):
    """Unsymmetric pattern with two long rows (601 and 141 entries: one
    workgroup per row) and a dominant diagonal of mixed sign."""
    lengths = np.random.default_rng(seed).integers(0, 9, n)
    lengths[[7, n // 2]] = [600, 140]
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=seed + 1)
    keep = r != c
    r, c, v = r[keep], c[keep], v[keep]
    # |d_i| = 1.1 (sum of |a_ij|, j != i) + 0.5: D^-1 A = I + E with ||E||_inf < 1
    rowsum = np.bincount(r, weights=np.abs(v), minlength=n)
    d = np.where(np.random.default_rng(seed + 2).random(n) < 0.5, -1.0, 1.0) * (1.1 * rowsum + 0.5)
    return (np.concatenate([r, np.arange(n)]), np.concatenate([c, np.arange(n)]),
            np.concatenate([v, d]))


CASES = [
    ("convdiff101", lambda: (10201,) + convdiff(101)),
    ("irregular30001", lambda: (30001,) + irregular(30001, 40)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("reorder", [False, True])
def test_first_iterates_match_oracle(name, make, dtype, reorder):
    n, r, c, v = make()
    v = v.astype(dtype)
    ref = oracle.coo_to_csr(n, r, c, v)
    b = np.random.default_rng(50).standard_normal(n).astype(dtype)
    print(f"bicgstab iterates {name} n={n} {np.dtype(dtype).name} reorder={reorder}", flush=True)
    A = handle(n, r, c, v, reorder=reorder)
    assert A.layout()["reordered"] == reorder
    tol = 1e-9 if dtype == np.float64 else 1e-4
    for k in (1, 2, 5, 12):
        xo, ito, _, oco = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, k)
        x, info = A.solve_raw(dev(b), 0.0, k, method="bicgstab")
        assert (info.iterations[0], info.status[0]) == (ito, oco) == (k, oracle.MAXIT)
        assert rel(host(x), xo) <= tol, (k, rel(host(x), xo))


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_converged_solve_matches_oracle(name, make):
    n, r, c, v = make()
    ref = oracle.coo_to_csr(n, r, c, v)
    b = np.random.default_rng(51).standard_normal(n)
    tol = 1e-10
    xo, ito, relo, oco = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 5000)
    A = handle(n, r, c, v)
    x, info = A.solve_raw(dev(b), tol, 5000, method="bicgstab")
    assert info.status[0] == oco == oracle.CONVERGED
    assert abs(info.iterations[0] - ito) <= max(3, 0.05 * ito), (info.iterations[0], ito)
    assert info.rel_residual[0] <= tol
    M = sp.csr_matrix((ref["vals"], ref["col"], ref["row_ptr"]), shape=(n, n))
    X = host(x)
    assert np.linalg.norm(b - M @ X) <= 1.5 * tol * np.linalg.norm(b)
    assert np.linalg.norm(M @ (X - xo)) <= 2.5 * tol * np.linalg.norm(b)


def test_exact_cases():
    # diagonal of mixed sign: the first half step is exact (x = b / d)
    n = 1000
    d = np.linspace(-5.0, 7.0, n)
    d[d == 0] = 1.0
    b = np.random.default_rng(52).standard_normal(n)
    A = handle(n, np.arange(n), np.arange(n), d)
    x, info = A.solve_raw(dev(b), 1e-12, 10, method="bicgstab")
    xo, ito, _, oco = oracle.bicgstab(np.arange(n + 1), np.arange(n), d, b, 1e-12, 10)
    assert (info.iterations[0], info.status[0]) == (ito, oco) == (1, oracle.CONVERGED)
    assert np.allclose(host(x), b / d, rtol=1e-14, atol=0)
    # breakdown at r^.v: x stays 0
    A = handle(2, np.array([0, 1, 1]), np.array([0, 0, 1]), np.array([1.0, -2.0, 1.0]))
    x, info = A.solve_raw(dev(np.array([1.0, 1.0])), 1e-10, 50, method="bicgstab")
    assert (info.iterations[0], info.status[0]) == (1, _lib.SLA_BREAKDOWN)
    assert not host(x).any() and info.rel_residual[0] == 1.0
    # breakdown at omega (negative diagonal): x keeps the half step
    A = handle(2, np.array([0, 0, 1, 1]), np.array([0, 1, 0, 1]),
               np.array([1.0, -3.0, -1.0, -1.0]))
    x, info = A.solve_raw(dev(np.array([-3.0, -3.0])), 1e-10, 50, method="bicgstab")
    assert (info.iterations[0], info.status[0]) == (1, _lib.SLA_BREAKDOWN)
    assert np.array_equal(host(x), [-1.5, 1.5]) and info.rel_residual[0] == 1.0


def test_zero_rhs_zero_budget_and_errors():
    n, r, c, v = (10201,) + convdiff(101)
    A = handle(n, r, c, v)
    x, info = A.solve_raw(dev(np.zeros(n)), 1e-8, 100, method="bicgstab")
    assert (info.iterations[0], info.status[0]) == (0, _lib.SLA_CONVERGED) and not host(x).any()
    x, info = A.solve_raw(dev(np.ones(n)), 1e-8, 0, method="bicgstab")
    assert (info.iterations[0], info.status[0], info.rel_residual[0]) == (0, _lib.SLA_MAXIT, 1.0)
    # a zero diagonal is refused; a negative one is refused by PCG only
    vz = v.copy()
    vz[(r == 5) & (c == 5)] = 0.0
    with pytest.raises(SlaError) as e:
        handle(n, r, c, vz).solve_raw(dev(np.ones(n)), 1e-8, 10, method="bicgstab")
    assert e.value.status == _lib.SLA_ERR_BAD_DIAGONAL
    vn = v.copy()
    vn[(r == 5) & (c == 5)] *= -1.0
    An = handle(n, r, c, vn)
    An.solve_raw(dev(np.ones(n)), 1e-8, 10, method="bicgstab")
    with pytest.raises(SlaError) as e:
        An.solve_raw(dev(np.ones(n)), 1e-8, 10)
    assert e.value.status == _lib.SLA_ERR_BAD_DIAGONAL
    # one system per handle
    rp, cp, vp = poisson2d_coo(10)
    Ab = SparseCSR.from_coo(dev(rp, torch.int64), dev(cp, torch.int64),
                            dev(np.stack([vp, vp])), 100)
    with pytest.raises(SlaError) as e:
        Ab.solve_raw(dev(np.ones((2, 100))), 1e-8, 10, method="bicgstab")
    assert e.value.status == _lib.SLA_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("reorder", [False, True])
def test_adjoint_iterates_match_oracle(dtype, reorder):
    # reordered: A^T lambda = g is solved on the inner handle's transpose
    n, r, c, v = (30001,) + irregular(30001, 60)
    v = v.astype(dtype)
    ref = oracle.coo_to_csr(n, r, c, v)
    b = np.random.default_rng(53).standard_normal(n).astype(dtype)
    g = np.random.default_rng(54).standard_normal(n).astype(dtype)
    A = handle(n, r, c, v, reorder=reorder)
    assert A.layout()["reordered"] == reorder
    x, _ = A.solve_raw(dev(b), 1e-6, 30, method="bicgstab")
    X = host(x)
    tol = 1e-9 if dtype == np.float64 else 1e-4
    for k in (1, 3, 10):
        lam_o, gv_o, ito, _, oco = oracle.bicgstab_adjoint(ref["row_ptr"], ref["col"], ref["vals"],
                                                           X, g, 0.0, k)
        gb, gv, info = A.adjoint_raw(x, dev(g), 0.0, k, method="bicgstab")
        assert (info.iterations[0], info.status[0]) == (ito, oco) == (k, oracle.MAXIT)
        assert rel(host(gb), lam_o) <= tol, (k, rel(host(gb), lam_o))
        assert rel(host(gv), gv_o) <= tol
    # no grad_b requested: lambda goes to the handle's own buffer
    _, gv2, _ = A.adjoint_raw(x, dev(g), 0.0, 10, want_b=False, method="bicgstab")
    assert np.array_equal(host(gv2), host(gv))


def test_autograd_converged_against_oracle_and_new_values():
    """Solve and backward to tol 1e-11 (the oracle at 1e-11 and 1e-14 differ by
    about 5e-10 here), then new values of the same pattern (a faster flow)."""
    n = 10201
    # duplicates split the same way for both value sets (the split pattern
    # depends on the seed and the entry count only)
    r, c, v = adversarial.split_duplicates(*convdiff(101, peak=5.0), seed=55, frac=0.2)
    _, _, v6 = adversarial.split_duplicates(*convdiff(101, peak=6.0), seed=55, frac=0.2)
    A = handle(n, r, c, v)
    for step, vals_np in enumerate([v, v6]):
        print(f"bicgstab autograd step {step}", flush=True)
        ref = oracle.coo_to_csr(n, r, c, vals_np)
        vals = dev(vals_np).requires_grad_(True)
        b = dev(np.random.default_rng(57).standard_normal(n)).requires_grad_(True)
        w = dev(np.random.default_rng(58).standard_normal(n))
        x = A.solve(b, values=vals, tol=1e-11, maxit=5000, method="bicgstab")
        gvals, gb = torch.autograd.grad((x * w).sum(), [vals, b])
        xo, *_ = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], host(b), 1e-11, 5000)
        lam, gvo, *_ = oracle.bicgstab_adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo,
                                               host(w), 1e-11, 5000)
        assert rel(host(x), xo) <= 1e-7, step
        assert rel(host(gb), lam) <= 1e-7, step
        assert rel(host(gvals), gvo[ref["slot"]]) <= 1e-7, step


@pytest.mark.parametrize("reorder", [False, True])
def test_symmetric_handle_solves_its_own_adjoint(reorder):
    # reordered: the inner handle solves its own adjoint
    rp, cp, vp = poisson2d_coo(90)
    n = 8100
    A = handle(n, rp, cp, vp, check_symmetric=True, reorder=reorder)
    assert A.layout()["reordered"] == reorder
    ref = oracle.coo_to_csr(n, rp, cp, vp)
    b = np.random.default_rng(59).standard_normal(n)
    g = np.random.default_rng(60).standard_normal(n)
    x, _ = A.solve_raw(dev(b), 1e-12, 3000, method="bicgstab")
    for k in (2, 7):
        lam_o, gv_o, *_ = oracle.bicgstab_adjoint(ref["row_ptr"], ref["col"], ref["vals"],
                                                  host(x), g, 0.0, k)
        gb, gv, _ = A.adjoint_raw(x, dev(g), 0.0, k, method="bicgstab")
        assert rel(host(gb), lam_o) <= 1e-9 and rel(host(gv), gv_o) <= 1e-9


def test_full_size_first_iterates():
    """The measured workload at full size (2.1M unknowns), first 20 iterates
    of the solve and of the adjoint, element-wise against the oracle."""
    w = make_workload("convdiff2d_1448")
    print(f"bicgstab full size n={w.n} nnz={w.nnz}", flush=True)
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    A = handle(w.n, w.rows, w.cols, w.vals)
    xo, ito, _, oco = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], w.b, 0.0, 20)
    x, info = A.solve_raw(dev(w.b), 0.0, 20, method="bicgstab")
    assert (info.iterations[0], info.status[0]) == (ito, oco) == (20, oracle.MAXIT)
    assert rel(host(x), xo) <= 1e-9
    lam_o, gv_o, *_ = oracle.bicgstab_adjoint(ref["row_ptr"], ref["col"], ref["vals"], host(x),
                                              w.g, 0.0, 20)
    gb, gv, _ = A.adjoint_raw(x, dev(w.g), 0.0, 20, method="bicgstab")
    assert rel(host(gb), lam_o) <= 1e-9 and rel(host(gv), gv_o) <= 1e-9


def test_results_independent_of_poll_interval_and_graphs():
    """The device freezes a finished solve, so neither the iterate nor the
    count depends on how often the host polls or on graph replay."""
    n, r, c, v = (10201,) + convdiff(101)
    b = dev(np.random.default_rng(61).standard_normal(n))
    A = handle(n, r, c, v)
    ref_x, ref_info = None, None
    for k, graph in [(16, 1), (1, 1), (7, 1), (64, 1), (16, 0)]:
        A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, k)
        A.set_option(_lib.SLA_OPT_USE_GRAPH, graph)
        x, info = A.solve_raw(b, 1e-9, 3000, method="bicgstab")
        X = host(x)
        if ref_x is None:
            ref_x, ref_info = X, (info.iterations[0], info.status[0], info.rel_residual[0])
        assert (info.iterations[0], info.status[0], info.rel_residual[0]) == ref_info, (k, graph)
        assert np.array_equal(X, ref_x), (k, graph)


def test_fp32_converged_and_reordered_adjoint():
    n, r, c, v = (30001,) + irregular(30001, 70)
    ref32 = oracle.coo_to_csr(n, r, c, v.astype(np.float32))
    b = np.random.default_rng(62).standard_normal(n).astype(np.float32)
    g = np.random.default_rng(63).standard_normal(n).astype(np.float32)
    for reorder in (False, True):
        A = handle(n, r, c, v.astype(np.float32), reorder=reorder)
        x, info = A.solve_raw(dev(b), 1e-5, 500, method="bicgstab")
        xo, ito, _, oco = oracle.bicgstab(ref32["row_ptr"], ref32["col"], ref32["vals"], b, 1e-5, 500)
        assert info.status[0] == oco == oracle.CONVERGED
        assert abs(info.iterations[0] - ito) <= 2
        assert rel(host(x), xo) <= 1e-4
        gb, gv, ainfo = A.adjoint_raw(x, dev(g), 1e-5, 500, method="bicgstab")
        lam, gvo, ita, _, oca = oracle.bicgstab_adjoint(ref32["row_ptr"], ref32["col"],
                                                        ref32["vals"], host(x), g, 1e-5, 500)
        assert ainfo.status[0] == oca == oracle.CONVERGED
        assert rel(host(gb), lam) <= 1e-4 and rel(host(gv), gvo) <= 1e-4


def test_list_handle_is_refused():
    from differentiable_sparse_linear_csr_amd import SparseTensorList
    rp, cp, vp = poisson2d_coo(10)
    L = SparseTensorList.from_coo_list([dev(rp, torch.int64)] * 2, [dev(cp, torch.int64)] * 2,
                                       [dev(vp)] * 2, [100, 100])
    with pytest.raises(SlaError) as e:
        L.solve_raw(dev(np.ones(200)), 1e-8, 10, method="bicgstab")
    assert e.value.status == _lib.SLA_ERR_INVALID_ARG
    with pytest.raises(SlaError) as e:
        L.adjoint_raw(dev(np.ones(200)), dev(np.ones(200)), 1e-8, 10, method="bicgstab")
    assert e.value.status == _lib.SLA_ERR_INVALID_ARG


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 65])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_tiny_systems_and_ragged_tails(n, dtype):
    """Sizes below one 16-byte group and with every tail length (the vector
    kernels' last rows are done one per lane)."""
    rng = np.random.default_rng(100 + n)
    r, c = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    keep = (np.abs(r - c) <= 2).ravel()
    r, c = r.ravel()[keep], c.ravel()[keep]
    v = rng.uniform(-1.0, 1.0, r.shape[0])
    v[r == c] = np.where(rng.random(n) < 0.5, -1.0, 1.0) * 6.0
    v = v.astype(dtype)
    b = rng.standard_normal(n).astype(dtype)
    ref = oracle.coo_to_csr(n, r, c, v)
    A = handle(n, r, c, v)
    tol = 1e-9 if dtype == np.float64 else 1e-4
    for k in (1, 3):
        xo, ito, relo, oco = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, k)
        if relo < 1e-9:
            # solved to rounding: from here on the steps act on rounding noise,
            # which differs between the two sides (fused multiply-adds)
            continue
        x, info = A.solve_raw(dev(b), 0.0, k, method="bicgstab")
        assert (info.iterations[0], info.status[0]) == (ito, oco)
        assert rel(host(x), xo) <= tol, (k, rel(host(x), xo))
    xo, ito, _, oco = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-12 if dtype == np.float64 else 1e-5, 200)
    x, info = A.solve_raw(dev(b), 1e-12 if dtype == np.float64 else 1e-5, 200, method="bicgstab")
    assert info.status[0] == oco == oracle.CONVERGED and abs(info.iterations[0] - ito) <= 1
    assert rel(host(x), xo) <= (1e-9 if dtype == np.float64 else 1e-4)

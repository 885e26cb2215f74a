"""GPU Jacobi-PCG and adjoint versus the oracle at sizes the oracle finishes in
seconds (several tiles and ragged tails): iterations within +-2, fp64
solution within 1e-8 relative (fp32 storage: 1e-4), outcomes, exactness of
the k-interval host poll, determinism, and the autograd path."""
import numpy as np
import pytest
import torch

import oracle
from differentiable_sparse_linear_csr_amd import _lib, SlaError
from workloads import adversarial, make_workload, poisson2d_coo

from gpu_util import coo_handle, csr_handle, dev, host, rel

pytestmark = pytest.mark.gpu

CASES = [
    ("poisson2d_64", None, None),
    ("diffusion3d_128", 24, None),
    ("knn_laplacian_2m", 20000, None),
    ("batched_diffusion2d_512x32", 48, 6),
    ("batched_diffusion2d_512x32", 40, 8),
]


def oracle_solve(w):
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    x, it, rl, oc = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, w.tol, w.maxit)
    return ref, x, np.atleast_1d(it), np.atleast_1d(rl), np.atleast_1d(oc)


# resident 0: the per-step kernels; 1: the automatic choice (the single-kernel
# solve wherever it applies)
@pytest.mark.parametrize("resident", [0, 1])
@pytest.mark.parametrize("name,size,batch", CASES)
def test_solve_matches_oracle(name, size, batch, resident):
    w = make_workload(name, size=size, batch=batch)
    print(f"pcg {name} n={w.n} nnz={w.nnz} batch={w.batch} resident={resident}", flush=True)
    ref, xo, ito, rlo, oco = oracle_solve(w)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    A.set_option(_lib.SLA_OPT_RESIDENT, resident)
    x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    xg = np.atleast_2d(host(x))
    xo = np.atleast_2d(xo)
    xtol = 1e-8 if w.dtype == "f64" else 1e-4
    for s in range(w.batch):
        assert info.status[s] == oco[s] == oracle.CONVERGED
        assert abs(info.iterations[s] - ito[s]) <= 2, (s, info.iterations[s], ito[s])
        assert rel(xg[s], xo[s]) <= xtol, (s, rel(xg[s], xo[s]))
        assert info.rel_residual[s] <= w.tol
        if info.iterations[s] == ito[s]:
            assert abs(info.rel_residual[s] - rlo[s]) <= 1e-3 * rlo[s]


@pytest.mark.parametrize("resident", [0, 1])
@pytest.mark.parametrize("name,size,batch", CASES)
def test_adjoint_matches_oracle(name, size, batch, resident):
    w = make_workload(name, size=size, batch=batch)
    ref, xo, *_ = oracle_solve(w)
    lam_o, gv_o, it_o, rl_o, oc_o = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, w.g,
                                                   w.tol, w.maxit)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    A.set_option(_lib.SLA_OPT_RESIDENT, resident)
    x, _ = A.solve_raw(dev(w.b), w.tol, w.maxit)
    gb, gv, info = A.adjoint_raw(x, dev(w.g), w.tol, w.maxit)
    tol = 1e-8 if w.dtype == "f64" else 1e-3
    gb, gv = np.atleast_2d(host(gb)), np.atleast_2d(host(gv))
    lam_o, gv_o = np.atleast_2d(lam_o), np.atleast_2d(gv_o)
    it_o = np.atleast_1d(it_o)
    for s in range(w.batch):
        assert abs(info.iterations[s] - it_o[s]) <= 2
        assert rel(gb[s], lam_o[s]) <= tol
        assert rel(gv[s], gv_o[s]) <= tol


@pytest.mark.parametrize("name,size", [("diffusion3d_128", 40), ("poisson2d_64", None),
                                       ("knn_laplacian_2m", 50000)])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_fused_update_direction_matches_two_kernels(name, size, dtype):
    # single system on the per-step path: update + direction fused (beta
    # broadcast inside the kernel) against the two-kernel form, and the oracle
    w = make_workload(name, size=size)
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    tol = w.tol if dtype == np.float64 else max(w.tol, 1e-5)
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v)
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, w.maxit)
    A = coo_handle(w.n, w.rows, w.cols, v)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, 0)   # unfused: update, then direction
    out = []
    for fused in (1, 0):
        A.set_option(_lib.SLA_OPT_FUSED_UPDATE, fused)
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(b), tol, w.maxit)
        prof = A.profile()
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        assert (prof["direction"][0] == 0) == bool(fused), prof
        assert abs(info.iterations[0] - ito) <= 2
        assert rel(host(x), xo) <= (1e-8 if dtype == np.float64 else 1e-4)
        out.append(host(x))
    # same recurrence; the r.z / r.r partials are grouped per workgroup, and
    # the two forms use different grids, so agreement is to rounding
    assert rel(out[0], out[1]) <= (1e-8 if dtype == np.float64 else 1e-4)


@pytest.mark.parametrize("B,dtype", [(4, np.float64), (8, np.float64), (8, np.float32),
                                     (16, np.float32)])
def test_batched_fused_update_direction(B, dtype):
    """Batches that fit one resident pass: update + direction in one kernel
    with a per-system beta broadcast, against the two-kernel form (graphs on,
    toggled between solves) and every system's oracle solve."""
    w = make_workload("batched_diffusion2d_512x32", size=40, batch=B)
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    tol = 1e-10 if dtype == np.float64 else 1e-5
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 5000)
    A = coo_handle(w.n, w.rows, w.cols, v)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)   # the per-step kernels
    A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, 0)   # unfused: update, then direction
    out = []
    for fused in (1, 0, 1):
        A.set_option(_lib.SLA_OPT_FUSED_UPDATE, fused)
        x, info = A.solve_raw(dev(b), tol, 5000)
        X = host(x)
        for s in range(B):
            assert info.status[s] == oco[s] and abs(info.iterations[s] - ito[s]) <= 2, s
            assert rel(X[s], xo[s]) <= (1e-8 if dtype == np.float64 else 1e-4), s
        out.append(X)
        # the fused path runs no separate direction kernel
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        A.solve_raw(dev(b), tol, 3)
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        assert (A.profile()["direction"][0] == 0) == bool(fused)
    assert np.array_equal(out[0], out[2])          # bitwise repeatable
    assert rel(out[0], out[1]) <= (1e-8 if dtype == np.float64 else 1e-4)


def test_check_interval_and_graph_do_not_change_results():
    w = make_workload("diffusion3d_128", size=20)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)   # the polled multi-kernel path
    b = dev(w.b)
    outs = []
    for k, graph in [(1, 1), (7, 1), (16, 1), (64, 1), (16, 0)]:
        A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, k)
        A.set_option(_lib.SLA_OPT_USE_GRAPH, graph)
        x, info = A.solve_raw(b, w.tol, w.maxit)
        outs.append((host(x).tobytes(), info.iterations[0], info.rel_residual[0]))
    assert all(o == outs[0] for o in outs)


def test_batched_slices_equal_single_solves():
    w = make_workload("batched_diffusion2d_512x32", size=32, batch=4)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    X, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    for s in range(4):
        As = coo_handle(w.n, w.rows, w.cols, np.ascontiguousarray(w.vals[s]))
        xs, inf_s = As.solve_raw(dev(w.b[s]), w.tol, w.maxit)
        assert inf_s.iterations[0] == info.iterations[s]
        assert rel(host(xs), host(X[s])) <= 1e-5


@pytest.mark.parametrize("resident", [1, 0])
def test_outcomes(resident):
    r, c, v = poisson2d_coo(30)
    A = coo_handle(900, r, c, v)
    A.set_option(_lib.SLA_OPT_RESIDENT, resident)
    b = np.random.default_rng(0).standard_normal(900)
    x, info = A.solve_raw(dev(np.zeros(900)), 1e-10, 100)
    assert info.iterations[0] == 0 and info.status[0] == _lib.SLA_CONVERGED
    assert not host(x).any() and info.rel_residual[0] == 0.0
    x, info = A.solve_raw(dev(b), 1e-10, 0)
    assert info.iterations[0] == 0 and info.status[0] == _lib.SLA_MAXIT and not host(x).any()
    ref = oracle.coo_to_csr(900, r, c, v)
    for maxit in (1, 3, 17):
        x, info = A.solve_raw(dev(b), 1e-14, maxit)
        xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-14, maxit)
        assert info.iterations[0] == ito == maxit and info.status[0] == _lib.SLA_MAXIT
        assert rel(host(x), xo) <= 1e-12
        assert abs(info.rel_residual[0] - rlo) <= 1e-12 * rlo
    x, info = A.solve_raw(dev(b), 0.0, 50)
    assert info.iterations[0] == 50 and info.status[0] == _lib.SLA_MAXIT
    # indefinite -> breakdown at the first step, x untouched
    A2 = coo_handle(2, np.array([0, 0, 1, 1]), np.array([0, 1, 0, 1]), np.array([1.0, 2, 2, 1]))
    A2.set_option(_lib.SLA_OPT_RESIDENT, resident)
    x, info = A2.solve_raw(dev(np.array([1.0, -1.0])), 1e-10, 10)
    assert info.status[0] == _lib.SLA_BREAKDOWN and info.iterations[0] == 1 and not host(x).any()
    # bad diagonal -> error
    v2 = v.copy()
    v2[(r == 7) & (c == 7)] = 0.0
    A3 = coo_handle(900, r, c, v2)
    A3.set_option(_lib.SLA_OPT_RESIDENT, resident)
    with pytest.raises(SlaError) as e:
        A3.solve_raw(dev(b), 1e-10, 10)
    assert e.value.status == _lib.SLA_ERR_BAD_DIAGONAL


def test_batched_mixed_outcomes():
    # systems finish at different iterations; zero rhs and budget limits per system
    w = make_workload("batched_diffusion2d_512x32", size=20, batch=5)
    b = w.b.copy()
    b[2] = 0.0
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    x, info = A.solve_raw(dev(b), w.tol, 40)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, w.tol, 40)
    for s in range(5):
        assert info.status[s] == oco[s]
        assert abs(info.iterations[s] - ito[s]) <= 2
        assert rel(host(x[s]), xo[s]) <= 1e-4
    assert info.iterations[2] == 0 and info.status[2] == _lib.SLA_CONVERGED


def shifted_batch(N, B, dtype, broken=None, seed=0):
    """B value sets on the N x N five-point pattern: system s has its diagonal
    raised by 0.05 s (different iteration counts); system `broken` has its
    off-diagonals scaled by 5 (positive diagonal, indefinite)."""
    r, c, v = poisson2d_coo(N)
    V = np.tile(v, (B, 1))
    diag = r == c
    for s in range(B):
        V[s, diag] += 0.05 * s
    if broken is not None:
        V[broken, ~diag] *= 5.0
    b = np.random.default_rng(seed).standard_normal((B, N * N))
    return r, c, V.astype(dtype), b.astype(dtype)


@pytest.mark.parametrize("dtype,B", [(np.float32, 8), (np.float64, 8), (np.float32, 256),
                                     (np.float64, 256)])
def test_batched_vector_lanes_mixed_outcomes(dtype, B):
    # systems of one lane (4 in fp32, 2 in fp64) converge, break down and stop
    # at different iterations; frozen systems must keep x untouched
    N = 20 if B == 8 else 12
    r, c, V, b = shifted_batch(N, B, dtype, broken=5)
    b[2] = 0.0
    b[5] = 1.0   # z = D^-1 1 makes p.Ap < 0 at the first step
    A = coo_handle(N * N, r, c, V)
    ref = oracle.coo_to_csr(N * N, r, c, V)
    tol = 1e-6 if dtype == np.float32 else 1e-10
    x, info = A.solve_raw(dev(b), tol, 300)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 300)
    X = host(x)
    xtol = 1e-4 if dtype == np.float32 else 1e-8
    assert info.status[2] == _lib.SLA_CONVERGED and info.iterations[2] == 0
    assert info.status[5] == _lib.SLA_BREAKDOWN and info.iterations[5] == 1
    assert not X[2].any() and not X[5].any()
    assert len(set(info.iterations)) > 3
    for s in range(B):
        assert info.status[s] == oco[s], s
        assert abs(info.iterations[s] - ito[s]) <= 2, (s, info.iterations[s], ito[s])
        assert rel(X[s], xo[s]) <= xtol, (s, rel(X[s], xo[s]))


def test_irregular_spd_with_long_rows_and_duplicates():
    n = 40000
    r, c, v = adversarial.random_spd_coo(n, 10.0, 13, max_row=30000)
    r, c, v = adversarial.split_duplicates(r, c, v, seed=3)
    ref = oracle.coo_to_csr(n, r, c, v)
    b = np.random.default_rng(1).standard_normal(n)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 5000)
    A = coo_handle(n, r, c, v)
    x, info = A.solve_raw(dev(b), 1e-10, 5000)
    assert abs(info.iterations[0] - ito) <= 2 and rel(host(x), xo) <= 1e-8


def test_int64_row_ptr_path():
    w = make_workload("poisson2d_11548", size=90)
    rows = np.repeat(np.arange(w.n), np.diff(w.row_ptr))
    ref = oracle.coo_to_csr(w.n, rows, w.cols, w.vals)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, 1e-10, 2000)
    A = csr_handle(w.row_ptr, w.cols, w.vals, rp_dtype=torch.int64)
    assert A.row_index_dtype == torch.int64
    x, info = A.solve_raw(dev(w.b), 1e-10, 2000)
    assert abs(info.iterations[0] - ito) <= 2 and rel(host(x), xo) <= 1e-8
    # fixed budget, tol 0 (as the large-grid workload runs)
    x, info = A.solve_raw(dev(w.b), 0.0, 25)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, 0.0, 25)
    assert info.iterations[0] == 25 and rel(host(x), xo) <= 1e-12
    assert abs(info.rel_residual[0] - rlo) <= 1e-10 * rlo


def test_repeatable_bitwise():
    w = make_workload("knn_laplacian_2m", size=10000)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    b = dev(w.b)
    x1, i1 = A.solve_raw(b, w.tol, w.maxit)
    x2, i2 = A.solve_raw(b, w.tol, w.maxit)
    assert host(x1).tobytes() == host(x2).tobytes() and i1.iterations == i2.iterations


def test_autograd_through_solve_with_duplicates():
    n = 3000
    r, c, v = adversarial.random_spd_coo(n, 6.0, 21)
    r, c, v = adversarial.split_duplicates(r, c, v, seed=7)
    rng = np.random.default_rng(4)
    b, g = rng.standard_normal(n), rng.standard_normal(n)
    A = coo_handle(n, r, c, v)
    vals = dev(v).requires_grad_(True)
    bt = dev(b).requires_grad_(True)
    x = A.solve(bt, values=vals, tol=1e-12, maxit=5000)
    (x * dev(g)).sum().backward()
    ref = oracle.coo_to_csr(n, r, c, v)
    xo, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-12, 5000)
    lam, gv, *_ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, 1e-12, 5000)
    assert rel(host(bt.grad), lam) <= 1e-9
    # every duplicate receives the gradient of the entry it was merged into
    assert rel(host(vals.grad), gv[ref["slot"]]) <= 1e-9
    # new values through the same handle
    v2 = v * 1.5
    vals2 = dev(v2).requires_grad_(True)
    x2 = A.solve(dev(b), values=vals2, tol=1e-12, maxit=5000)
    assert rel(host(x2), xo / 1.5) <= 1e-9


def block_chains_coo(n=65536, block=512, seed=5):
    """Block-diagonal SPD matrix: independent 1D chains of `block` rows
    (diagonal 2 + U(0, 1), couplings -1 inside a chain). At 65 536 rows the
    single-kernel solve runs 128 workgroups of 512 rows, one chain each, so no
    workgroup waits for another before a product (empty dependency lists)."""
    rng = np.random.default_rng(seed)
    i = np.arange(n)
    inner = (i % block) != block - 1          # row i couples to i + 1
    up = i[inner]
    r = np.concatenate([i, up, up + 1])
    c = np.concatenate([i, up + 1, up])
    v = np.concatenate([2.0 + rng.uniform(0.0, 1.0, n), -np.ones(2 * up.size)])
    return n, r.astype(np.int64), c.astype(np.int64), v


def resident_cases():
    r, c, v = adversarial.random_spd_coo(30011, 9.0, 21, skew=False)  # irregular, none past 128
    return {
        "block_chains_65536": block_chains_coo(),
        "poisson2d_64": make_workload("poisson2d_64"),
        "diffusion3d_128_s40": make_workload("diffusion3d_128", size=40),
        "knn_laplacian_2m_s60000": make_workload("knn_laplacian_2m", size=60000),
        "random_spd_30011": (30011, r, c, v),
        "diffusion3d_128_s70": make_workload("diffusion3d_128", size=70),
    }


@pytest.mark.parametrize("name", ["poisson2d_64", "diffusion3d_128_s40", "knn_laplacian_2m_s60000",
                                  "random_spd_30011", "diffusion3d_128_s70", "block_chains_65536"])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("dia", [1, 0])
def test_single_kernel_solve_matches_oracle_and_multi_kernel_path(name, dtype, dia):
    """dia 1: the stencils (Poisson, 3D diffusion) are held by diagonals;
    dia 0: every matrix by row tiles."""
    case = resident_cases()[name]
    if isinstance(case, tuple):
        n, r, c, v = case
        b = np.random.default_rng(3).standard_normal(n)
        tol, maxit = 1e-8, 2000
    else:
        n, r, c, v, b, tol, maxit = case.n, case.rows, case.cols, case.vals, case.b, case.tol, case.maxit
    v, b = v.astype(dtype), b.astype(dtype)
    if dtype == np.float32:
        tol = max(tol, 1e-5)
    print(f"single-kernel {name} n={n} {np.dtype(dtype).name}", flush=True)
    ref = oracle.coo_to_csr(n, r, c, v)
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, maxit)
    A = coo_handle(n, r, c, v)      # the automatic choice: the single-kernel solve
    A.set_option(_lib.SLA_OPT_RESIDENT_DIA, dia)
    A.profile_reset()
    A.set_option(_lib.SLA_OPT_PROFILE, 1)
    x1, i1 = A.solve_raw(dev(b), tol, maxit)
    prof = A.profile()
    A.set_option(_lib.SLA_OPT_PROFILE, 0)
    assert prof["cg_resident"][0] == 1 and prof["spmv_dot"][0] == 0, prof
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    x0, i0 = A.solve_raw(dev(b), tol, maxit)
    xtol = 1e-8 if dtype == np.float64 else 1e-4
    for x, info in ((x1, i1), (x0, i0)):
        assert info.status[0] == oco == oracle.CONVERGED
        assert abs(info.iterations[0] - ito) <= 2, (info.iterations[0], ito)
        assert rel(host(x), xo) <= xtol, rel(host(x), xo)
        assert info.rel_residual[0] <= tol
    # deterministic: the same bits on a second run
    A.set_option(_lib.SLA_OPT_RESIDENT, 2)
    x2, i2 = A.solve_raw(dev(b), tol, maxit)
    assert host(x2).tobytes() == host(x1).tobytes() and i2.iterations[0] == i1.iterations[0]


def test_single_kernel_int64_row_ptr_and_adjoint():
    w = make_workload("poisson2d_11548", size=200)     # CSR input with int64 row_ptr
    A = csr_handle(w.row_ptr, w.cols, w.vals)
    A.set_option(_lib.SLA_OPT_RESIDENT, 2)
    g = np.random.default_rng(9).standard_normal(w.n)
    ref = {"row_ptr": w.row_ptr.astype(np.int64), "col": w.cols.astype(np.int64), "vals": w.vals}
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], w.b, 1e-10, 5000)
    lam_o, gv_o, *_ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, 1e-10, 5000)
    A.profile_reset()
    A.set_option(_lib.SLA_OPT_PROFILE, 1)
    x, info = A.solve_raw(dev(w.b), 1e-10, 5000)
    gb, gv, ainfo = A.adjoint_raw(x, dev(g), 1e-10, 5000)
    assert A.profile()["cg_resident"][0] == 2
    assert abs(info.iterations[0] - ito) <= 2
    assert rel(host(x), xo) <= 1e-8
    assert rel(host(gb), lam_o) <= 1e-8 and rel(host(gv), gv_o) <= 1e-8


@pytest.mark.parametrize("B,dtype", [(2, np.float64), (3, np.float64), (4, np.float64),
                                     (8, np.float32), (32, np.float32), (5, np.float32)])
def test_batched_single_kernel_solve(B, dtype):
    """A batch as B independent groups of the single-kernel solve: each system
    against its own oracle solve and against the per-step batched kernels,
    with a zero right-hand side and an indefinite member among them, and the
    adjoint (lambda and grad_vals) of the converged ones."""
    w = make_workload("batched_diffusion2d_512x32", size=48, batch=B)
    v = w.vals.astype(dtype).copy()
    b = w.b.astype(dtype).copy()
    b[0] = 0.0                                   # converged at iteration 0
    if B > 2:
        # off-diagonal couplings four times the diagonal's share: indefinite,
        # the CG step breaks down
        v[1] = np.where(w.rows == w.cols, v[1], 4 * v[1])
    tol = 1e-10 if dtype == np.float64 else 1e-5
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 4000)
    g = np.random.default_rng(7).standard_normal((B, w.n)).astype(dtype)
    A = coo_handle(w.n, w.rows, w.cols, v)
    print(f"batched single-kernel B={B} n={w.n} {np.dtype(dtype).name}", flush=True)
    A.profile_reset()
    A.set_option(_lib.SLA_OPT_PROFILE, 1)
    x1, i1 = A.solve_raw(dev(b), tol, 4000)
    prof = A.profile()
    A.set_option(_lib.SLA_OPT_PROFILE, 0)
    assert prof["cg_resident"][0] == 1 and prof["spmv_dot"][0] == 0, prof
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    x0, i0 = A.solve_raw(dev(b), tol, 4000)
    A.set_option(_lib.SLA_OPT_RESIDENT, 1)
    xtol = 1e-8 if dtype == np.float64 else 1e-4
    for x, info in ((x1, i1), (x0, i0)):
        X = host(x)
        for s in range(B):
            assert info.status[s] == oco[s], (s, info.status[s], oco[s])
            if oco[s] == oracle.CONVERGED and ito[s] > 0:
                assert abs(info.iterations[s] - ito[s]) <= 2, (s, info.iterations[s], ito[s])
                assert rel(X[s], xo[s]) <= xtol, (s, rel(X[s], xo[s]))
            else:
                assert info.iterations[s] == ito[s], s
    assert not host(x1)[0].any()
    # the adjoint on the same path
    gb, gv, ainfo = A.adjoint_raw(x1, dev(g), tol, 4000)
    lam, gvo, ita, _, oca = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], host(x1), g,
                                           tol, 4000)
    GB, GV = host(gb), host(gv)
    gtol = 1e-8 if dtype == np.float64 else 1e-3
    for s in range(B):
        assert ainfo.status[s] == oca[s]
        if oca[s] == oracle.CONVERGED:
            assert rel(GB[s], lam[s]) <= gtol and rel(GV[s], gvo[s]) <= gtol, s
    # deterministic
    x2, i2 = A.solve_raw(dev(b), tol, 4000)
    assert host(x2).tobytes() == host(x1).tobytes()


def test_ordinary_launch_of_the_single_kernel_solve():
    """SLA_OPT_COOPERATIVE = 0 starts the same kernel on the same grid with an
    ordinary launch: the same bits and the same iteration count as the
    cooperative launch, forward and adjoint."""
    w = make_workload("diffusion3d_128", size=32)
    g = np.random.default_rng(11).standard_normal(w.n)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    out = []
    for coop in (1, 0):
        A.set_option(_lib.SLA_OPT_COOPERATIVE, coop)
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
        gb, gv, ainfo = A.adjoint_raw(x, dev(g), w.tol, w.maxit)
        assert A.profile()["cg_resident"][0] == 2
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        out.append((host(x), host(gb), host(gv), info.iterations[0], ainfo.iterations[0]))
    (x1, gb1, gv1, i1, a1), (x0, gb0, gv0, i0, a0) = out
    assert i1 == i0 and a1 == a0
    assert x1.tobytes() == x0.tobytes() and gb1.tobytes() == gb0.tobytes()
    assert gv1.tobytes() == gv0.tobytes()


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_batched_single_kernel_largest_register_shape(dtype):
    """32 systems of 65 536 rows: each system's group has 8 workgroups (256
    CUs shared by 32 groups), so every wavefront owns 1024 rows, 16 per lane,
    the largest register shape of the single-kernel solve. Every system's x
    and adjoint against its own oracle solve, whole vectors."""
    N, B = 256, 32
    r, c, V, b = shifted_batch(N, B, dtype, seed=12)
    n = N * N
    tol = 1e-10 if dtype == np.float64 else 1e-5
    ref = oracle.coo_to_csr(n, r, c, V)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 4000)
    g = np.random.default_rng(13).standard_normal((B, n)).astype(dtype)
    lam, gvo, ita, _, oca = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, tol,
                                           4000)
    A = coo_handle(n, r, c, V)
    print(f"batched single-kernel B={B} n={n} {np.dtype(dtype).name}", flush=True)
    A.profile_reset()
    A.set_option(_lib.SLA_OPT_PROFILE, 1)
    x, info = A.solve_raw(dev(b), tol, 4000)
    gb, gv, ainfo = A.adjoint_raw(x, dev(g), tol, 4000)
    prof = A.profile()
    A.set_option(_lib.SLA_OPT_PROFILE, 0)
    assert prof["cg_resident"][0] == 2 and prof["spmv_dot"][0] == 0, prof
    X, GB, GV = host(x), host(gb), host(gv)
    xtol, gtol = (1e-8, 1e-8) if dtype == np.float64 else (1e-4, 1e-3)
    for s in range(B):
        assert info.status[s] == oco[s] == oracle.CONVERGED, s
        assert abs(info.iterations[s] - ito[s]) <= 2, (s, info.iterations[s], ito[s])
        assert rel(X[s], xo[s]) <= xtol, (s, rel(X[s], xo[s]))
        assert ainfo.status[s] == oca[s] == oracle.CONVERGED, s
        assert abs(ainfo.iterations[s] - ita[s]) <= 2, s
        assert rel(GB[s], lam[s]) <= gtol and rel(GV[s], gvo[s]) <= gtol, s


@pytest.mark.parametrize("name,size", [("diffusion3d_128", 64), ("poisson2d_11548", 700)])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("dia", [1, 0])
def test_folded_direction_matches_oracle_and_three_kernels(name, size, dtype, dia):
    """SLA_OPT_FOLD_DIRECTION on the per-step path (single kernel and fused
    update off, so that it applies at these sizes): p = z + beta p formed in
    the SpMV and x += alpha p applied one iteration later, two kernels per
    iteration; fp64 values only (fp32 ones keep three kernels). Against the oracle (converged solve, tol-0 step counts with an
    odd check interval so that captured blocks start on either direction
    buffer, eager launches, the iteration budget, b = 0, the adjoint) and
    against the three-kernel form."""
    w = make_workload(name, size=size)
    n = w.n
    rows = np.repeat(np.arange(n), np.diff(w.row_ptr)) if w.fmt == "csr" else w.rows
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    f64 = dtype == np.float64
    tol = 1e-10 if f64 else 1e-5
    xtol = 1e-8 if f64 else 1e-4
    print(f"folded direction: {name} n={n} {np.dtype(dtype).name}", flush=True)
    ref = oracle.coo_to_csr(n, rows, w.cols, v)
    rp, cc, vv = ref["row_ptr"], ref["col"], ref["vals"]
    xo, ito, _, oco = oracle.pcg(rp, cc, vv, b, tol, 20000)
    A = coo_handle(n, rows, w.cols, v)
    lay = A.layout()
    assert lay["ring_tiles"] and lay["long_rows"] == 0, lay
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 0)
    A.set_option(_lib.SLA_OPT_SPMV_DIA, dia)   # the SpMV by diagonals (dia 1) or the ring
    assert (A.step_diagonals() > 0) == bool(dia)

    def solve(bb, t, maxit, prof=False):
        if prof:
            A.profile_reset()
            A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(bb), t, maxit)
        p = A.profile() if prof else None
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        return host(x), info, p

    out = {}
    for fold in (1, 0):
        A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, fold)
        x, info, p = solve(b, tol, 20000, prof=True)
        # folded (fp64 values only): no direction kernel; one update per
        # SpMV either way
        assert (p["direction"][0] == 0) == (bool(fold) and f64), p
        assert p["update"][0] == p["spmv_dot"][0] > 0, p
        assert info.status[0] == oco == oracle.CONVERGED
        assert abs(info.iterations[0] - ito) <= 2, (info.iterations[0], ito)
        assert rel(x, xo) <= xtol, rel(x, xo)
        if f64:
            # the true residual of the returned x (the last step applied)
            r_true = b - oracle.spmv(rp, cc, vv, x)
            assert np.linalg.norm(r_true) <= 10 * tol * np.linalg.norm(b)
        out[fold] = x
    assert rel(out[1], out[0]) <= xtol
    A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, 1)
    # fixed step counts (tol 0): both buffer parities, graphs and eager
    stol = 1e-11 if f64 else 1e-4
    for k, interval, graph in ((7, 3, 1), (8, 3, 1), (5, 16, 0), (1, 16, 1)):
        A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, interval)
        A.set_option(_lib.SLA_OPT_USE_GRAPH, graph)
        x, info, _ = solve(b, 0.0, k)
        xk, itk, _, ock = oracle.pcg(rp, cc, vv, b, 0.0, k)
        assert info.iterations[0] == itk == k and info.status[0] == ock == oracle.MAXIT
        assert rel(x, xk) <= stol, (k, interval, graph, rel(x, xk))
    A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, 16)
    A.set_option(_lib.SLA_OPT_USE_GRAPH, 1)
    # b = 0: converged at once, x = 0
    x, info, _ = solve(np.zeros_like(b), tol, 100)
    assert info.status[0] == oracle.CONVERGED and info.iterations[0] == 0 and not x.any()
    # the adjoint (the same folded solve on A^T = A)
    g = np.random.default_rng(21).standard_normal(n).astype(dtype)
    lam_o, gv_o, it_o, _, _ = oracle.adjoint(rp, cc, vv, xo, g, tol, 20000)
    xg = A.solve_raw(dev(b), tol, 20000)[0]
    gb, gv, ainfo = A.adjoint_raw(xg, dev(g), tol, 20000)
    assert abs(ainfo.iterations[0] - it_o) <= 2
    assert rel(host(gb), lam_o) <= 10 * xtol
    assert rel(host(gv), gv_o) <= 10 * xtol


@pytest.mark.parametrize("shift,at", [(0.3, 6), (0.5, 5), (0.7, 4), (1.2, 3), (2.5, 2)])
@pytest.mark.parametrize("dia", [1, 0])
def test_folded_direction_breakdown(shift, at, dia):
    """The folded single-system solve applies x += alpha p on every other
    SpMV (two pending steps at once) and the rest at the end: a Poisson
    matrix shifted to be indefinite breaks down at iteration `at` (odd and
    even counts), where x must hold exactly the steps before the breakdown,
    as in the oracle."""
    r, c, v = poisson2d_coo(30)
    v = v.astype(np.float64).copy()
    v[r == c] -= shift
    b = np.random.default_rng(0).standard_normal(900)
    ref = oracle.coo_to_csr(900, r, c, v)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 400)
    assert oco == oracle.BREAKDOWN and ito == at
    A = coo_handle(900, r, c, v)
    assert A.layout()["ring_tiles"]
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 0)
    A.set_option(_lib.SLA_OPT_SPMV_DIA, dia)
    for graph, interval in ((1, 16), (0, 1), (1, 3)):
        A.set_option(_lib.SLA_OPT_USE_GRAPH, graph)
        A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, interval)
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(b), 1e-10, 400)
        prof = A.profile()
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        assert prof["direction"][0] == 0, prof      # folded
        assert info.status[0] == oracle.BREAKDOWN and info.iterations[0] == at
        assert rel(host(x), xo) <= 1e-12, (graph, interval, rel(host(x), xo))


@pytest.mark.parametrize("dtype,B", [(np.float32, 8), (np.float64, 8), (np.float32, 32),
                                     (np.float64, 4)])
def test_batched_folded_direction_mixed_outcomes(dtype, B):
    """The folded direction on a batch (per-step path, fused update off so
    that it applies): systems that converge at once, break down at the first
    step and stop at different iterations, in the same 16-byte lanes. A
    stopped system keeps x and carries its direction into the newer buffer,
    and its last step is applied once at the end. Against the oracle, with
    graphs at poll interval 3 (captured blocks start on either buffer) and
    eager launches."""
    N = 24
    r, c, V, b = shifted_batch(N, B, dtype, broken=3 if B > 3 else None)
    b[2] = 0.0
    if B > 3:
        b[3] = 1.0   # z = D^-1 1 makes p.Ap < 0 at the first step
    A = coo_handle(N * N, r, c, V)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 0)
    ref = oracle.coo_to_csr(N * N, r, c, V)
    tol = 1e-6 if dtype == np.float32 else 1e-10
    xtol = 1e-4 if dtype == np.float32 else 1e-8
    xo, ito, rlo, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 300)
    print(f"batched folded direction: B={B} {np.dtype(dtype).name}", flush=True)
    for interval, graph in ((3, 1), (16, 0)):
        A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, interval)
        A.set_option(_lib.SLA_OPT_USE_GRAPH, graph)
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(b), tol, 300)
        prof = A.profile()
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        # fp64 folds; fp32 keeps the direction kernel (z would add a rounding)
        assert (prof["direction"][0] == 0) == (dtype == np.float64), prof
        assert prof["update"][0] > 0, prof
        X = host(x)
        assert info.status[2] == _lib.SLA_CONVERGED and info.iterations[2] == 0
        assert not X[2].any()
        if B > 3:
            assert info.status[3] == _lib.SLA_BREAKDOWN and info.iterations[3] == 1
            assert not X[3].any()
        for s in range(B):
            assert info.status[s] == oco[s], s
            assert abs(info.iterations[s] - ito[s]) <= 2, (s, info.iterations[s], ito[s])
            assert rel(X[s], xo[s]) <= xtol, (s, rel(X[s], xo[s]))
    A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, 16)
    A.set_option(_lib.SLA_OPT_USE_GRAPH, 1)
    # fixed step counts, odd and even, against the oracle's
    for k in (5, 6):
        x, info = A.solve_raw(dev(b), 0.0, k)
        xk, itk, _, ock = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, k)
        X = host(x)
        for s in range(B):
            assert info.iterations[s] == itk[s] and info.status[s] == ock[s], s
            assert rel(X[s], xk[s]) <= (1e-11 if dtype == np.float64 else 1e-4), (k, s)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_batched_folded_direction_matches_three_kernels(dtype):
    """The 512x512 x 32 workload's family at 40x40 x 8: folded and three-kernel
    forms against the oracle, and the adjoint on the folded form."""
    B = 8
    w = make_workload("batched_diffusion2d_512x32", size=40, batch=B)
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    tol = 1e-10 if dtype == np.float64 else 1e-5
    xtol = 1e-8 if dtype == np.float64 else 1e-4
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 5000)
    A = coo_handle(w.n, w.rows, w.cols, v)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 0)
    out = {}
    for fold in (1, 0):
        A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, fold)
        x, info = A.solve_raw(dev(b), tol, 5000)
        X = host(x)
        for s in range(B):
            assert info.status[s] == oco[s] and abs(info.iterations[s] - ito[s]) <= 2, s
            assert rel(X[s], xo[s]) <= xtol, (fold, s, rel(X[s], xo[s]))
        out[fold] = X
    for s in range(B):
        assert rel(out[1][s], out[0][s]) <= xtol
    A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, 1)
    g = w.g.astype(dtype)
    lam_o, gv_o, it_o, _, _ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, tol,
                                            5000)
    x, _ = A.solve_raw(dev(b), tol, 5000)
    gb, gv, ainfo = A.adjoint_raw(x, dev(g), tol, 5000)
    GB, GV = host(gb), host(gv)
    gtol = 1e-8 if dtype == np.float64 else 1e-3
    for s in range(B):
        assert abs(ainfo.iterations[s] - it_o[s]) <= 2
        assert rel(GB[s], lam_o[s]) <= gtol and rel(GV[s], gv_o[s]) <= gtol, s


def test_folded_direction_on_reordered_handle():
    """The folded solve runs on the reordered handle's P A P^T (options reach
    it through the caller's handle); x in the caller's order against the
    oracle on A, folded and not, and the adjoint's value gradient in the
    caller's CSR order."""
    from differentiable_sparse_linear_csr_amd import SparseCSR
    N = 300
    r, c, v = poisson2d_coo(N)
    n = N * N
    b = np.random.default_rng(31).standard_normal(n)
    A = SparseCSR.from_coo(dev(r), dev(c), dev(v), n, reorder=True)
    assert A.layout()["reordered"]
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 0)
    ref = oracle.coo_to_csr(n, r, c, v)
    tol = 1e-10
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, 20000)
    out = {}
    for fold in (1, 0):
        A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, fold)
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(b), tol, 20000)
        prof = A.profile()
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        assert (prof["direction"][0] == 0) == bool(fold), prof
        assert abs(info.iterations[0] - ito) <= 2
        assert rel(host(x), xo) <= 1e-8
        out[fold] = host(x)
    assert rel(out[1], out[0]) <= 1e-8
    A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, 1)
    g = np.random.default_rng(32).standard_normal(n)
    lam, gvo, ita, _, _ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, tol, 20000)
    x, _ = A.solve_raw(dev(b), tol, 20000)
    gb, gv, ainfo = A.adjoint_raw(x, dev(g), tol, 20000)
    assert abs(ainfo.iterations[0] - ita) <= 2
    assert rel(host(gb), lam) <= 1e-8 and rel(host(gv), gvo) <= 1e-8


@pytest.mark.parametrize("case", ["diffusion3d_64", "knn_300k", "batched_fp32_b4"])
def test_single_kernel_walks_bitwise_equal(case):
    """SLA_OPT_RESIDENT_WALK: the single-kernel solve's SpMV phase with each
    wavefront on a contiguous run of its workgroup's tiles (0) and with the
    tiles interleaved over the wavefronts (1): the same tiles and sums, so
    bitwise equal solutions, iteration counts and adjoint gradients; and the
    solution against the oracle."""
    if case == "diffusion3d_64":
        w = make_workload("diffusion3d_128", size=64)
        r, c, v, b, g = w.rows, w.cols, w.vals, w.b, w.g
    elif case == "knn_300k":
        w = make_workload("knn_laplacian_2m", size=300000)
        r, c, v, b, g = w.rows, w.cols, w.vals, w.b, w.g
    else:
        w = make_workload("batched_diffusion2d_512x32", size=128, batch=4)
        r, c, v, b, g = w.rows, w.cols, w.vals, w.b, w.g
    print(f"resident walks: {case} n={w.n} nnz={w.nnz} batch={w.batch}", flush=True)
    A = coo_handle(w.n, r, c, v)
    A.set_option(_lib.SLA_OPT_RESIDENT_DIA, 0)   # the walks of the row tiles
    out = {}
    for walk in (0, 1):
        A.set_option(_lib.SLA_OPT_RESIDENT_WALK, walk)
        x, info = A.solve_raw(dev(b), w.tol, w.maxit)
        assert A.last_path()["path"] == "single_kernel"
        gb, gv, ainfo = A.adjoint_raw(x, dev(g), w.tol, w.maxit)
        out[walk] = (host(x), list(info.iterations), host(gb), host(gv), list(ainfo.iterations))
    x0, it0, gb0, gv0, ait0 = out[0]
    x1, it1, gb1, gv1, ait1 = out[1]
    assert it0 == it1 and ait0 == ait1
    assert x0.tobytes() == x1.tobytes()
    assert gb0.tobytes() == gb1.tobytes() and gv0.tobytes() == gv1.tobytes()
    ref = oracle.coo_to_csr(w.n, r, c, v)
    xo, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, w.tol, w.maxit)
    tol = 1e-8 if w.dtype == "f64" else 1e-3
    for s in range(w.batch):
        assert rel(np.atleast_2d(x1)[s], np.atleast_2d(xo)[s]) <= tol
    A.set_option(_lib.SLA_OPT_RESIDENT_WALK, 2)
    with pytest.raises(SlaError):
        A.set_option(_lib.SLA_OPT_RESIDENT_WALK, 3)


def nine_point(N):
    """2D 9-point Laplacian (8 on the diagonal, -1 to the 8 neighbours): 9
    diagonals, one more than a matrix held by diagonals may have."""
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    idx = (i * N + j).ravel()
    rows, cols, vals = [idx], [idx], [np.full(N * N, 8.0)]
    for di in (-1, 0, 1):
        for dj in (-1, 0, 1):
            if di == 0 and dj == 0:
                continue
            ok = ((i + di >= 0) & (i + di < N) & (j + dj >= 0) & (j + dj < N)).ravel()
            rows.append(idx[ok])
            cols.append(((i + di) * N + (j + dj)).ravel()[ok])
            vals.append(np.full(int(ok.sum()), -1.0))
    return np.concatenate(rows), np.concatenate(cols), np.concatenate(vals)


@pytest.mark.parametrize("name,size,ndiag", [("poisson2d_64", None, 5), ("diffusion3d_128", 40, 7),
                                             ("diffusion3d_128", 64, 7),
                                             ("poisson2d_11548", 30, 5)])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_single_kernel_by_diagonals(name, size, ndiag, dtype):
    """Stencil matrices (5 and 7 diagonals; 900 rows, not a multiple of a
    wavefront's 64) in the single-kernel solve held by diagonals: converged
    solve, fixed step counts and the adjoint against the oracle, and the
    row-tile form (SLA_OPT_RESIDENT_DIA 0) against the oracle too."""
    w = make_workload(name, size=size)
    n = w.n
    rows = np.repeat(np.arange(n), np.diff(w.row_ptr)) if w.fmt == "csr" else w.rows
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    f64 = dtype == np.float64
    tol = 1e-10 if f64 else 1e-5
    xtol = 1e-8 if f64 else 1e-4
    print(f"by diagonals: {name} n={n} {np.dtype(dtype).name}", flush=True)
    ref = oracle.coo_to_csr(n, rows, w.cols, v)
    rp, cc, vv = ref["row_ptr"], ref["col"], ref["vals"]
    xo, ito, _, oco = oracle.pcg(rp, cc, vv, b, tol, 20000)
    g = np.random.default_rng(22).standard_normal(n).astype(dtype)
    lam_o, gv_o, it_o, _, _ = oracle.adjoint(rp, cc, vv, xo, g, tol, 20000)
    A = coo_handle(n, rows, w.cols, v)
    for dia in (1, 0):
        A.set_option(_lib.SLA_OPT_RESIDENT_DIA, dia)
        x, info = A.solve_raw(dev(b), tol, 20000)
        assert A.last_path()["path"] == "single_kernel"
        assert A.diagonals() == (ndiag if dia else 0)
        assert info.status[0] == oco == oracle.CONVERGED
        assert abs(info.iterations[0] - ito) <= 2, (dia, info.iterations[0], ito)
        assert rel(host(x), xo) <= xtol, (dia, rel(host(x), xo))
        for k in (1, 2, 7):
            xk, info = A.solve_raw(dev(b), 0.0, k)
            xko, itk, _, _ = oracle.pcg(rp, cc, vv, b, 0.0, k)
            assert info.iterations[0] == k == itk
            assert rel(host(xk), xko) <= (1e-12 if f64 else 1e-5), (dia, k, rel(host(xk), xko))
        gb, gv, ainfo = A.adjoint_raw(x, dev(g), tol, 20000)
        assert abs(ainfo.iterations[0] - it_o) <= 2
        assert rel(host(gb), lam_o) <= 10 * xtol and rel(host(gv), gv_o) <= 10 * xtol, dia


@pytest.mark.parametrize("shift,at", [(0.3, 6), (0.5, 5), (2.5, 2)])
def test_single_kernel_by_diagonals_breakdown(shift, at):
    """A Poisson matrix shifted to be indefinite, held by diagonals in the
    single-kernel solve: breakdown at the oracle's iteration, x as the
    oracle's."""
    r, c, v = poisson2d_coo(30)
    v = v.astype(np.float64).copy()
    v[r == c] -= shift
    b = np.random.default_rng(0).standard_normal(900)
    ref = oracle.coo_to_csr(900, r, c, v)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 400)
    A = coo_handle(900, r, c, v)
    x, info = A.solve_raw(dev(b), 1e-10, 400)
    assert A.last_path()["path"] == "single_kernel" and A.diagonals() == 5
    assert info.status[0] == oco == oracle.BREAKDOWN and info.iterations[0] == ito == at
    assert rel(host(x), xo) <= 1e-12


def test_single_kernel_row_tiles_where_diagonals_do_not_fit():
    """Nine diagonals, a pattern whose diagonals would be mostly empty (a
    tridiagonal matrix with one far symmetric pair), and a batch keep the
    row tiles; each against the oracle."""
    r, c, v = nine_point(40)
    n = 1600
    b = np.random.default_rng(3).standard_normal(n)
    ref = oracle.coo_to_csr(n, r, c, v)
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 2000)
    A = coo_handle(n, r, c, v)
    x, info = A.solve_raw(dev(b), 1e-10, 2000)
    assert A.last_path()["path"] == "single_kernel" and A.diagonals() == 0
    assert abs(info.iterations[0] - ito) <= 2 and rel(host(x), xo) <= 1e-8
    # tridiagonal + one far pair: 5 offsets but 5 n slots for ~3 n entries
    n = 5000
    i = np.arange(n)
    r = np.concatenate([i, i[1:], i[:-1], [0, n - 1]])
    c = np.concatenate([i, i[:-1], i[1:], [n - 1, 0]])
    v = np.concatenate([np.full(n, 4.0), np.full(2 * (n - 1), -1.0), [0.5, 0.5]])
    b = np.random.default_rng(4).standard_normal(n)
    ref = oracle.coo_to_csr(n, r, c, v)
    xo, ito, _, _ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 1e-10, 2000)
    A = coo_handle(n, r, c, v)
    x, info = A.solve_raw(dev(b), 1e-10, 2000)
    assert A.last_path()["path"] == "single_kernel" and A.diagonals() == 0
    assert abs(info.iterations[0] - ito) <= 2 and rel(host(x), xo) <= 1e-8
    # a batch of stencil systems
    w = make_workload("batched_diffusion2d_512x32", size=40, batch=4)
    A = coo_handle(w.n, w.rows, w.cols, w.vals.astype(np.float64))
    A.solve_raw(dev(w.b.astype(np.float64)), 1e-8, 2000)
    assert A.last_path()["path"] == "single_kernel" and A.diagonals() == 0

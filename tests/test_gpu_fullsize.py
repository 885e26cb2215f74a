"""Full-size parity: the workloads at their benchmark sizes, in the launch
configuration bench.py times, against reference values the CPU oracle wrote
(tests/golden/<workload>.json, produced by tests/golden/make_golden.py).

The oracle stores, per system, the iteration count, outcome, recursive
residual, the 2-norm, values at seeded sample indices and projections onto
seeded random vectors. A normwise relative error <= tol_x implies
|dx_i| <= tol_x ||x|| for every sample and |<dx, w>| <= tol_x ||x|| ||w|| for
every projection, which is what is asserted together with the norm itself.
"""
import json
import os

import numpy as np
import pytest
import torch

from differentiable_sparse_linear_csr_amd import SparseCSR, _lib
from workloads import make_workload

from gpu_util import dev, host

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
NAMES = ["diffusion3d_128", "knn_laplacian_2m", "batched_diffusion2d_512x32", "poisson2d_11548"]


def check_vector(v, ref, tol):
    v = v.astype(np.float64)
    norm = ref["norm"]
    assert abs(np.linalg.norm(v) - norm) <= tol * norm
    idx = np.random.default_rng(ref["sample_seed"]).integers(0, v.shape[0], len(ref["samples"]))
    assert np.all(np.abs(v[idx] - np.asarray(ref["samples"])) <= tol * norm)
    for k, pr in enumerate(ref["projections"]):
        w = np.random.default_rng(ref["sample_seed"] + 1000 * k).standard_normal(v.shape[0])
        assert abs(np.dot(w, v) - pr) <= tol * norm * np.linalg.norm(w)


# resident 0: the per-step kernels; 1: the automatic choice, which is the
# single-kernel solve where it applies (n <= 2^21, one system)
CASES = [(n, 0) for n in NAMES] + [("diffusion3d_128", 1), ("knn_laplacian_2m", 1)]


@pytest.mark.parametrize("name,resident", CASES)
def test_full_size_against_oracle_reference(name, resident):
    path = os.path.join(HERE, "golden", f"{name}.json")
    ref = json.load(open(path))
    print(f"full-size {name}: building inputs", flush=True)
    w = make_workload(name)
    assert ref["n"] == w.n and ref["nnz"] == w.nnz and ref["batch"] == w.batch
    if w.fmt == "coo":
        A = SparseCSR.from_coo(dev(w.rows), dev(w.cols), dev(w.vals), w.n)
    else:
        A = SparseCSR.from_csr(dev(w.row_ptr), dev(w.cols), dev(w.vals))
        assert A.row_index_dtype == torch.int64
    A.set_option(_lib.SLA_OPT_RESIDENT, resident)
    if resident == 1:
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
    print(f"full-size {name}: solving n={w.n} nnz={w.nnz} batch={w.batch}", flush=True)
    x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    if resident == 1:
        assert A.profile()["cg_resident"][0] == 1
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
    X = np.atleast_2d(host(x))
    tol_x = 1e-8 if w.dtype == "f64" else 1e-4
    for s, fr in enumerate(ref["forward"]):
        assert info.status[s] == fr["status"], (s, info.status[s], fr["status"])
        assert abs(info.iterations[s] - fr["iterations"]) <= 2, (s, info.iterations[s], fr["iterations"])
        if w.tol > 0:
            assert info.rel_residual[s] <= w.tol
        if info.iterations[s] == fr["iterations"]:
            # the recursive residual after the same number of steps depends on
            # the order of the row sums and of the p.q and r.r reductions (a
            # launch-shape choice): on the stencils the orders seen differ by
            # ~0.3%; on the kNN Laplacian (worse conditioned, reordered) the
            # single-kernel solve ends at 9.58e-9 against the oracle's 9.76e-9
            # after the same 276 steps (1.8%), both below the tolerance
            assert abs(info.rel_residual[s] - fr["rel_residual"]) <= 5e-2 * fr["rel_residual"]
        check_vector(X[s], fr, tol_x)
    if "adjoint" in ref:
        print(f"full-size {name}: adjoint", flush=True)
        gb, gv, ainfo = A.adjoint_raw(x, dev(w.g), w.tol, w.maxit)
        GB, GV = np.atleast_2d(host(gb)), np.atleast_2d(host(gv))
        tol_g = 1e-8 if w.dtype == "f64" else 1e-3
        for s, ar in enumerate(ref["adjoint"]):
            assert ainfo.status[s] == ar["status"]
            assert abs(ainfo.iterations[s] - ar["iterations"]) <= 2
            check_vector(GB[s], ar["lambda"], tol_g)
            check_vector(GV[s], ar["grad_vals"], tol_g)


def test_full_size_list_against_oracle_reference():
    """The 16-member list at its benchmark size, built as bench.py builds it
    (one block-diagonal handle), against each member's own oracle solve
    (tests/golden/list_diffusion2d_16.json). Both sides run the same
    recurrence from the same start and differ by rounding only, far below the
    tolerance-level error of either; 1e-6 bounds it with room."""
    from differentiable_sparse_linear_csr_amd import SparseTensorList
    name = "list_diffusion2d_16"
    ref = json.load(open(os.path.join(HERE, "golden", f"{name}.json")))
    print(f"full-size {name}: building inputs", flush=True)
    w = make_workload(name)
    assert ref["n"] == w.n and ref["members"] == len(w.extra["seg_rows"]) - 1
    A = SparseTensorList.from_block_diagonal_coo(dev(w.rows), dev(w.cols), dev(w.vals),
                                                 w.extra["seg_rows"])
    print(f"full-size {name}: solving n={w.n} nnz={w.nnz}", flush=True)
    x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    X = host(x)
    gb, gv, ainfo = A.adjoint_raw(x, dev(w.g), w.tol, w.maxit)
    GB, GV = host(gb), host(gv)
    k0 = 0
    for q, (fr, ar) in enumerate(zip(ref["forward"], ref["adjoint"])):
        r0, r1 = fr["rows"]
        assert info.status[q] == fr["status"] and ainfo.status[q] == ar["status"], q
        assert abs(info.iterations[q] - fr["iterations"]) <= 2, (q, info.iterations[q])
        assert abs(ainfo.iterations[q] - ar["iterations"]) <= 2, (q, ainfo.iterations[q])
        assert info.rel_residual[q] <= w.tol and ainfo.rel_residual[q] <= w.tol
        check_vector(X[r0:r1], fr, 1e-6)
        check_vector(GB[r0:r1], ar["lambda"], 1e-6)
        check_vector(GV[k0:k0 + ar["nnz"]], ar["grad_vals"], 1e-6)
        k0 += ar["nnz"]
    assert k0 == w.nnz

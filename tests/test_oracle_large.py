"""Pins for the oracle where the benchmark-size parity tests rely on it:

- its multi-threaded branch (loops over 65 536 rows or more run under
  OpenMP): SciPy's cg and scipy.sparse's product at those sizes, batched
  solves (whose per-system loops run on one thread) bitwise equal to single
  solves (whose loops run on all threads), and bitwise equal results from
  separate processes with 1 and with several threads;
- its fp32-storage reading (vectors and values stored in fp32, every
  product, sum and scalar formed in fp64, each stored value rounded once):
  iterate by iterate against the fp64 oracle (itself pinned by dense LU,
  eigenmodes and SciPy) on the same fp32-rounded inputs. One step moves the
  stored iterate by about one fp32 rounding of its entries, so after k steps
  the two stay within (1 + k/2) units of fp32 rounding (2^-24) normwise.
  Accumulating p.q or r.z in fp32 instead puts them 4 to 15 times past that
  bound (checked on a scratch copy of the oracle with those mistakes
  planted); accumulating a row of the product in fp32 is caught by the
  SpMV's own once-rounded pin.
"""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import scipy.sparse as sp
import scipy.sparse.linalg as spla

import oracle
from workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
U32 = 2.0 ** -24
PARALLEL_ROWS = 65536   # the oracle's threshold for its OpenMP loops


def csr_of(w, vals=None):
    out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals if vals is None else vals)
    return out["row_ptr"], out["col"], out["vals"]


def scipy_cg(rp, col, val, b, tol, maxit):
    n = rp.shape[0] - 1
    A = sp.csr_matrix((val, col, rp), shape=(n, n))
    dinv = 1.0 / A.diagonal()
    M = spla.LinearOperator((n, n), matvec=lambda y: dinv * y)
    count = [0]

    def cb(_):
        count[0] += 1

    x, info = spla.cg(A, b, rtol=tol, atol=0.0, maxiter=maxit, M=M, callback=cb)
    return count[0], x


LARGE = [("diffusion3d_128", 48, 1e-10), ("knn_laplacian_2m", 100000, 1e-8)]


@pytest.mark.parametrize("name,size,tol", LARGE)
def test_large_systems_against_scipy(name, size, tol):
    w = make_workload(name, size=size)
    assert w.n >= PARALLEL_ROWS
    rp, col, val = csr_of(w)
    A = sp.csr_matrix((val, col, rp), shape=(w.n, w.n))
    # the product: componentwise against scipy.sparse, |dy_i| <= (len_i + 2) u sum |a x|
    x = np.random.default_rng(5).standard_normal(w.n)
    y = oracle.spmv(rp, col, val, x)
    ys = A @ x
    bound = (np.diff(rp) + 2) * 2.0 ** -53 * (abs(A) @ np.abs(x))
    assert np.all(np.abs(y - ys) <= bound)
    # the solve: iteration count within one of SciPy's cg, same solution
    xo, it, rel, oc = oracle.pcg(rp, col, val, w.b, tol, 20000)
    it_sp, x_sp = scipy_cg(rp, col, val, w.b, tol, 20000)
    assert oc == oracle.CONVERGED and rel <= tol
    assert abs(it - it_sp) <= 1, (it, it_sp)
    assert np.linalg.norm(xo - x_sp) / np.linalg.norm(x_sp) <= 1e-6
    # and the true residual of the oracle's x
    assert np.linalg.norm(w.b - A @ xo) / np.linalg.norm(w.b) <= 10 * tol


def test_parallel_loops_match_single_thread_loops_bitwise():
    """A batch runs one system per thread with every per-system loop on that
    one thread; a single solve runs its row loops on all threads. At 110 592
    rows the two must agree bit for bit, in fp64 and fp32 storage, forward
    and adjoint."""
    if oracle.num_threads() < 2:
        pytest.skip("one host thread: the parallel loops do not split")
    w = make_workload("diffusion3d_128", size=48)
    g = np.random.default_rng(2).standard_normal(w.n)
    for dtype in (np.float64, np.float32):
        v = w.vals.astype(dtype)
        rp, col, val = csr_of(w, v)
        b, gg = w.b.astype(dtype), g.astype(dtype)
        B2 = np.stack([val, val])
        X, its, rels, ocs = oracle.pcg(rp, col, B2, np.stack([b, b]), 1e-6, 300)
        x, it, rel, oc = oracle.pcg(rp, col, val, b, 1e-6, 300)
        for s in range(2):
            assert X[s].tobytes() == x.tobytes() and its[s] == it and rels[s] == rel
        L, GV, *_ = oracle.adjoint(rp, col, B2, X, np.stack([gg, gg]), 1e-6, 300)
        lam, gv, *_ = oracle.adjoint(rp, col, val, x, gg, 1e-6, 300)
        assert L[0].tobytes() == lam.tobytes() and GV[1].tobytes() == gv.tobytes()
        Y = oracle.spmv(rp, col, B2, np.stack([b, b]))
        assert Y[0].tobytes() == oracle.spmv(rp, col, val, b).tobytes()


_CHILD = r"""
import hashlib, json, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle
from workloads import make_workload, convdiff2d_coo, rotating_flow
h = {"threads": oracle.num_threads()}
w = make_workload("knn_laplacian_2m", size=100000)
ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
rp, col, val = ref["row_ptr"], ref["col"], ref["vals"]
x, it, rel, oc = oracle.pcg(rp, col, val, w.b, w.tol, 2000)
lam, gv, it2, *_ = oracle.adjoint(rp, col, val, x, w.g, w.tol, 2000)
y = oracle.spmv(rp, col, val, w.b)
h["pcg"] = [hashlib.sha256(x.tobytes()).hexdigest(), it, rel.hex()]
h["adjoint"] = [hashlib.sha256(lam.tobytes() + gv.tobytes()).hexdigest(), it2]
h["spmv"] = hashlib.sha256(y.tobytes()).hexdigest()
r, c, v = convdiff2d_coo(300, *rotating_flow(300, 4.0))
ref = oracle.coo_to_csr(300 * 300, r, c, v)
bb = np.random.default_rng(3).standard_normal(300 * 300)
xb, itb, relb, _ = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], bb, 1e-8, 300)
h["bicgstab"] = [hashlib.sha256(xb.tobytes()).hexdigest(), itb, relb.hex()]
print(json.dumps(h))
"""


def test_results_do_not_depend_on_the_thread_count():
    """The same oracle calls in separate processes with OMP_NUM_THREADS = 1 and
    = 4 (loops over 100 000 and 90 000 rows): bitwise equal results."""
    oracle.build(force=False)
    outs = []
    for threads in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=threads)
        res = subprocess.run([sys.executable, "-c", _CHILD, ROOT], env=env, capture_output=True,
                             text=True, timeout=600)
        assert res.returncode == 0, res.stderr
        outs.append(json.loads(res.stdout.strip().splitlines()[-1]))
    assert outs[0]["threads"] == 1 and outs[1]["threads"] == 4
    for key in ("pcg", "adjoint", "spmv", "bicgstab"):
        assert outs[0][key] == outs[1][key], key


FP32_CASES = [("poisson2d_64", None), ("batched_diffusion2d_512x32", 48),
              ("knn_laplacian_2m", 5000), ("diffusion3d_128", 16)]


def fp32_inputs(name, size):
    w = make_workload(name, size=size, batch=1 if name.startswith("batched") else None)
    v32 = np.atleast_2d(w.vals)[0].astype(np.float32)
    b32 = np.atleast_2d(w.b)[0].astype(np.float32)
    g32 = np.atleast_2d(w.g)[0].astype(np.float32)
    return w, v32, b32, g32


@pytest.mark.parametrize("name,size", FP32_CASES)
def test_fp32_storage_iterates_track_fp64(name, size):
    w, v32, b32, _ = fp32_inputs(name, size)
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v32)
    ref64 = oracle.coo_to_csr(w.n, w.rows, w.cols, v32.astype(np.float64))
    b64 = b32.astype(np.float64)
    for k in range(1, 11):
        x32, it32, rel32, oc32 = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b32, 0.0, k)
        x64, it64, rel64, _ = oracle.pcg(ref64["row_ptr"], ref64["col"], ref64["vals"], b64, 0.0, k)
        assert x32.dtype == np.float32 and it32 == it64 == k and oc32 == oracle.MAXIT
        e = np.linalg.norm(x32.astype(np.float64) - x64) / np.linalg.norm(x64)
        bound = (1 + 0.5 * k) * U32
        assert e <= bound, (k, e / U32)
        assert abs(rel32 - rel64) <= bound * rel64, (k, abs(rel32 - rel64) / rel64 / U32)


@pytest.mark.parametrize("name,size", FP32_CASES)
def test_fp32_adjoint_iterates_track_fp64(name, size):
    """The fp32-storage adjoint (its solve on A^T and grad_vals rounded once
    from the fp64 product) against the fp64 adjoint on the same fp32 inputs,
    the forward x given as the same fp32 vector to both."""
    w, v32, b32, g32 = fp32_inputs(name, size)
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v32)
    ref64 = oracle.coo_to_csr(w.n, w.rows, w.cols, v32.astype(np.float64))
    x32, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b32, 1e-5, 5000)
    for k in (1, 2, 5, 10):
        lam32, gv32, it32, rel32, _ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], x32,
                                                     g32, 0.0, k)
        lam64, gv64, it64, rel64, _ = oracle.adjoint(ref64["row_ptr"], ref64["col"],
                                                     ref64["vals"], x32.astype(np.float64),
                                                     g32.astype(np.float64), 0.0, k)
        assert lam32.dtype == np.float32 and gv32.dtype == np.float32 and it32 == it64 == k
        bound = (1 + 0.5 * k) * U32
        el = np.linalg.norm(lam32 - lam64) / np.linalg.norm(lam64)
        eg = np.linalg.norm(gv32 - gv64) / np.linalg.norm(gv64)
        assert el <= bound, (k, el / U32)
        assert eg <= bound + U32, (k, eg / U32)

"""GPU SpMV versus the oracle: normwise relative error <= 1e-12 (fp64) and
<= 1e-5 (fp32), plus a componentwise rounding bound per row; irregular,
empty and long rows (short tiles, sub-wave groups, workgroup-per-row),
batched value sets, the workloads' matrices."""
import numpy as np
import pytest

import oracle
from workloads import adversarial, make_workload

from gpu_util import coo_handle, csr_handle, dev, host, rel

pytestmark = pytest.mark.gpu


def check(A, rows_np, cols_np, vals_np, n, x_np, tol):
    ref = oracle.coo_to_csr(n, rows_np, cols_np, vals_np)
    y_ref = oracle.spmv(ref["row_ptr"], ref["col"], ref["vals"], x_np)
    y = host(A.matvec(dev(x_np)))
    assert rel(y, y_ref) <= tol, rel(y, y_ref)
    # componentwise: |dy_i| <= (len_i + 2) u sum_k |a_ik x_k|
    V = np.atleast_2d(ref["vals"]).astype(np.float64)
    X = np.atleast_2d(x_np).astype(np.float64)
    Y = np.atleast_2d(y).astype(np.float64)
    Yr = np.atleast_2d(y_ref).astype(np.float64)
    rp, col = ref["row_ptr"], ref["col"]
    lens = np.diff(rp)
    rowid = np.repeat(np.arange(n), lens)
    u = np.finfo(np.float32 if vals_np.dtype == np.float32 else np.float64).eps
    for s in range(V.shape[0]):
        absum = np.bincount(rowid, weights=np.abs(V[s] * X[s][col]), minlength=n)
        bound = (lens + 2) * u * absum + (2 * u * np.abs(Yr[s]) if u > 1e-10 else 0) + 1e-300
        assert np.all(np.abs(Y[s] - Yr[s]) <= bound)


@pytest.mark.parametrize("dtype,tol", [(np.float64, 1e-12), (np.float32, 1e-5)])
def test_irregular_rows(dtype, tol):
    n = 120000
    lengths = np.random.default_rng(0).integers(0, 12, n)
    lengths[[5, 6, 7]] = 0
    for i, L in zip([100, 2000, 3000, 4000, 5000, 6000, 7000, 8000],
                    [63, 64, 65, 511, 512, 513, 4096, 100000]):
        lengths[i] = L
    lengths[9000:9300] = 300         # a run of medium rows (few rows per tile)
    print(f"spmv irregular n={n} nnz={lengths.sum()} {np.dtype(dtype).name}", flush=True)
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=1)
    v = v.astype(dtype)
    A = coo_handle(n, r, c, v)
    x = np.random.default_rng(2).standard_normal(n).astype(dtype)
    check(A, r, c, v, n, x, tol)


@pytest.mark.parametrize("name,size", [("poisson2d_64", None), ("diffusion3d_128", 30),
                                       ("knn_laplacian_2m", 30000)])
def test_workload_matrices(name, size):
    w = make_workload(name, size=size)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    check(A, w.rows, w.cols, w.vals, w.n, w.b, 1e-12)


def test_csr_int64_row_ptr():
    w = make_workload("poisson2d_11548", size=300)
    A = csr_handle(w.row_ptr, w.cols, w.vals)
    rows = np.repeat(np.arange(w.n), np.diff(w.row_ptr))
    check(A, rows, w.cols, w.vals, w.n, w.b, 1e-12)


@pytest.mark.parametrize("B", [2, 3, 32])
def test_batched(B):
    w = make_workload("batched_diffusion2d_512x32", size=70, batch=B)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    check(A, w.rows, w.cols, w.vals, w.n, w.b, 1e-5)
    v64 = w.vals.astype(np.float64)
    A = coo_handle(w.n, w.rows, w.cols, v64)
    check(A, w.rows, w.cols, v64, w.n, w.b.astype(np.float64), 1e-12)


@pytest.mark.parametrize("dtype,B", [(np.float32, 4), (np.float32, 8), (np.float32, 12),
                                     (np.float32, 256), (np.float64, 2), (np.float64, 16),
                                     (np.float64, 256)])
def test_batched_irregular(dtype, B):
    # empty, short and long rows (past the batched kernels' prefetch window and
    # the long-row limit) with B value sets; a ragged last workgroup
    n = 2003
    lengths = np.random.default_rng(3).integers(0, 12, n)
    lengths[[3, 4, n - 1]] = 0
    lengths[10], lengths[500], lengths[n - 2] = 40, 700, 9
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=3)
    V = np.random.default_rng(4).standard_normal((B, v.shape[0])).astype(dtype)
    A = coo_handle(n, r, c, V)
    x = np.random.default_rng(5).standard_normal((B, n)).astype(dtype)
    check(A, r, c, V, n, x, 1e-12 if dtype == np.float64 else 1e-5)


@pytest.mark.parametrize("D", [1000, 65000, 65535, 65536, 70000])
def test_column_span_around_16_bits(D):
    # rows hold columns i and i + D (and i - D): tiles whose columns span less
    # than 2^16 read 16-bit tile-relative indices, the others 32-bit ones
    n = 140000
    i = np.arange(n)
    rows = np.concatenate([i, i[i + D < n], i[i - D >= 0]])
    cols = np.concatenate([i, (i + D)[i + D < n], (i - D)[i - D >= 0]])
    order = np.lexsort((cols, rows))
    rows, cols = rows[order], cols[order]
    vals = np.random.default_rng(D).standard_normal(rows.shape[0])
    A = coo_handle(n, rows, cols, vals)
    x = np.random.default_rng(D + 1).standard_normal(n)
    check(A, rows, cols, vals, n, x, 1e-12)


def test_deterministic_bitwise():
    n = 50000
    r, c, v = adversarial.random_spd_coo(n, 12.0, 3, max_row=20000)
    A = coo_handle(n, r, c, v)
    x = dev(np.random.default_rng(5).standard_normal(n))
    y1 = host(A.matvec(x))
    y2 = host(A.matvec(x))
    assert y1.tobytes() == y2.tobytes()

"""GPU SpMV versus the oracle: normwise relative error <= 1e-12 (fp64) and
<= 1e-5 (fp32), plus a componentwise rounding bound per row; irregular,
empty and long rows (short tiles, sub-wave groups, workgroup-per-row),
batched value sets, the workloads' matrices."""
import numpy as np
import pytest

import oracle
from differentiable_sparse_linear_csr_amd import _lib
from workloads import adversarial, make_workload, poisson2d_coo

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


@pytest.mark.parametrize("name,size", [("poisson2d_11548", 4100), ("diffusion3d_128", 110),
                                       ("convdiff2d_1448", 1030)])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_band_aligned_tiles(name, size, dtype):
    """Stencil matrices of over 2^20 rows whose grid stride is 4096 rows or
    more (the 2D and 3D ones here) get band-aligned tiles (tile j + L is tile
    j moved by the stride) walked by columns; the smaller stride keeps the
    usual tiles. The product, and 30 PCG steps or 12 BiCGStab steps on the
    per-step kernels (tol 0), against the oracle."""
    w = make_workload(name, size=size)
    assert w.n >= 1 << 20
    if w.fmt == "csr":
        rows = np.repeat(np.arange(w.n), np.diff(w.row_ptr))
        r, c = rows, w.cols
    else:
        r, c = w.rows, w.cols
    v = w.vals.astype(dtype)
    print(f"band-aligned tiles: {name} n={w.n} {np.dtype(dtype).name}", flush=True)
    A = coo_handle(w.n, r, c, v)
    A.set_option(_lib.SLA_OPT_SPMV_DIA, 0)   # the tiles (stencils are also held by diagonals)
    x = np.random.default_rng(5).standard_normal(w.n).astype(dtype)
    check(A, r, c, v, w.n, x, 1e-12 if dtype == np.float64 else 1e-5)
    ref = oracle.coo_to_csr(w.n, r, c, v)
    b = w.b.astype(dtype)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    if w.extra.get("method") == "bicgstab":
        xg, info = A.solve_raw(dev(b), 0.0, 12, method="bicgstab")
        xo, *_ = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, 12)
        tol = 1e-9 if dtype == np.float64 else 1e-4
    else:
        xg, info = A.solve_raw(dev(b), 0.0, 30)
        xo, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, 30)
        tol = 1e-12 if dtype == np.float64 else 1e-5
    assert rel(host(xg), xo) <= tol, rel(host(xg), xo)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_band_aligned_tiles_bicgstab(dtype):
    """BiCGStab's two fused SpMVs on band-aligned tiles (the 4100^2 Poisson
    matrix, one panel per XCD): 12 steps (tol 0) against the oracle's."""
    w = make_workload("poisson2d_11548", size=4100)
    rows = np.repeat(np.arange(w.n), np.diff(w.row_ptr))
    v = w.vals.astype(dtype)
    b = w.b.astype(dtype)
    print(f"band-aligned bicgstab n={w.n} {np.dtype(dtype).name}", flush=True)
    A = coo_handle(w.n, rows, w.cols, v)
    A.set_option(_lib.SLA_OPT_SPMV_DIA, 0)   # the band tiles, not the diagonals
    ref = oracle.coo_to_csr(w.n, rows, w.cols, v)
    xg, info = A.solve_raw(dev(b), 0.0, 12, method="bicgstab")
    xo, *_ = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, 12)
    tol = 1e-9 if dtype == np.float64 else 1e-4
    assert rel(host(xg), xo) <= tol, rel(host(xg), xo)


def banded_irregular(n, seed):
    """Rows of 3 to 7 entries (one row in 50 empty) at columns within 2000 of
    the diagonal: every SpMV tile small and narrow, row lengths ragged."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(3, 8, n)
    lens[rng.random(n) < 0.02] = 0
    rows = np.repeat(np.arange(n), lens)
    off = rng.integers(-2000, 2001, rows.size)
    cols = np.clip(rows + off, 0, n - 1)
    key = np.unique(rows * n + cols)
    rows, cols = key // n, key % n
    vals = rng.standard_normal(rows.size)
    return rows, cols, vals


@pytest.mark.parametrize("case", ["poisson2d_1100", "diffusion3d_40", "banded_irregular", "tiny"])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_ring_pipeline_matches_one_tile_ahead(case, dtype):
    """SLA_OPT_SPMV_RING: the SpMV that keeps four tiles of entries and two
    of gathers in flight per wavefront (the default where every tile is
    small) against the one-tile-ahead kernel on the same handle: the same
    tiles and sums, so bitwise equal products; both against the oracle; and
    PCG (fused w.q) and BiCGStab (two fused dots) steps on the per-step
    kernels against the oracle's."""
    spd = True
    if case in ("poisson2d_1100", "diffusion3d_40"):
        w = (make_workload("poisson2d_11548", size=1100) if case == "poisson2d_1100"
             else make_workload("diffusion3d_128", size=40))
        n, c, v = w.n, w.cols, w.vals
        r = np.repeat(np.arange(n), np.diff(w.row_ptr)) if w.fmt == "csr" else w.rows
    elif case == "banded_irregular":
        n = 300000
        r, c, v = banded_irregular(n, 7)
        spd = False
    else:
        # fewer tiles than the ring holds: three wavefronts' rings never fill
        n = 10
        i = np.arange(n)
        r = np.concatenate([i, i[1:], i[:-1]])
        c = np.concatenate([i, i[:-1], i[1:]])
        v = np.concatenate([np.full(n, 2.0), np.full(n - 1, -1.0), np.full(n - 1, -1.0)])
    v = v.astype(dtype)
    print(f"ring SpMV: {case} n={n} nnz={v.size} {np.dtype(dtype).name}", flush=True)
    A = coo_handle(n, r, c, v)
    A.set_option(_lib.SLA_OPT_SPMV_DIA, 0)   # the tile kernels (stencils are also held by diagonals)
    lay = A.layout()
    assert lay["narrow_columns"] and lay["ring_tiles"], lay
    x = np.random.default_rng(11).standard_normal(n).astype(dtype)
    y_ring = host(A.matvec(dev(x)))
    A.set_option(_lib.SLA_OPT_SPMV_RING, 0)
    y_one = host(A.matvec(dev(x)))
    assert y_ring.tobytes() == y_one.tobytes()
    A.set_option(_lib.SLA_OPT_SPMV_RING, 1)
    check(A, r, c, v, n, x, 1e-12 if dtype == np.float64 else 1e-5)
    if not spd:
        return
    ref = oracle.coo_to_csr(n, r, c, v)
    b = np.random.default_rng(12).standard_normal(n).astype(dtype)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    steps, bsteps = (25, 8) if n > 1000 else (4, 3)   # short of exact convergence
    xg, _ = A.solve_raw(dev(b), 0.0, steps)
    xo, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, steps)
    tol = 1e-11 if dtype == np.float64 else 1e-4
    assert rel(host(xg), xo) <= tol, rel(host(xg), xo)
    xg, _ = A.solve_raw(dev(b), 0.0, bsteps, method="bicgstab")
    xo, *_ = oracle.bicgstab(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, bsteps)
    tol = 1e-9 if dtype == np.float64 else 1e-4
    assert rel(host(xg), xo) <= tol, rel(host(xg), xo)


@pytest.mark.parametrize("name,size,m", [("poisson2d_64", None, 5), ("poisson2d_11548", 1101, 5),
                                         ("diffusion3d_128", 45, 7), ("poisson2d_11548", 4100, 5)])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_spmv_by_diagonals(name, size, m, dtype):
    """Stencils (5 and 7 diagonals; 1101^2 and 45^3 rows, ragged against the
    kernel's 1024-row groups; 4100^2 past 2^24 rows) also held by diagonals:
    the per-step SpMV reads them (one row per lane) against the oracle and
    the row tiles (SLA_OPT_SPMV_DIA 0), 30 per-step PCG steps against the
    oracle, and new values after create reach the diagonals."""
    w = make_workload(name, size=size)
    n = w.n
    r = np.repeat(np.arange(n), np.diff(w.row_ptr)) if w.fmt == "csr" else w.rows
    v = w.vals.astype(dtype)
    print(f"SpMV by diagonals: {name} n={n} {np.dtype(dtype).name}", flush=True)
    A = coo_handle(n, r, w.cols, v)
    assert A.step_diagonals() == m
    x = np.random.default_rng(5).standard_normal(n).astype(dtype)
    tol = 1e-12 if dtype == np.float64 else 1e-5
    check(A, r, w.cols, v, n, x, tol)
    y1 = host(A.matvec(dev(x)))
    A.set_option(_lib.SLA_OPT_SPMV_DIA, 0)
    assert A.step_diagonals() == 0
    y0 = host(A.matvec(dev(x)))
    assert rel(y1, y0) <= tol
    A.set_option(_lib.SLA_OPT_SPMV_DIA, 1)
    # new values (scaled rows keep the pattern): the diagonals follow
    v2 = (v * (1.0 + 0.5 * (r % 7 == 3))).astype(dtype)
    A.set_values(dev(v2))
    check(A, r, w.cols, v2, n, x, tol)
    ref = oracle.coo_to_csr(n, r, w.cols, v)
    A.set_values(dev(v))
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    b = w.b.astype(dtype)
    xg, info = A.solve_raw(dev(b), 0.0, 30)
    xo, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, 0.0, 30)
    assert rel(host(xg), xo) <= (1e-12 if dtype == np.float64 else 1e-5), rel(host(xg), xo)


def test_diagonals_only_for_fitting_patterns():
    """Patterns that are not held by diagonals: a nine-point stencil, a
    tridiagonal matrix with one far pair (5 offsets, mostly empty
    diagonals), an irregular pattern, a batch."""
    N = 30
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    idx = (i * N + j).ravel()
    rows, cols = [idx], [idx]
    for di in (-1, 0, 1):
        for dj in (-1, 0, 1):
            if di or dj:
                ok = ((i + di >= 0) & (i + di < N) & (j + dj >= 0) & (j + dj < N)).ravel()
                rows.append(idx[ok])
                cols.append(((i + di) * N + (j + dj)).ravel()[ok])
    r9, c9 = np.concatenate(rows), np.concatenate(cols)
    assert coo_handle(N * N, r9, c9, np.ones(r9.size)).step_diagonals() == 0
    n = 5000
    k = np.arange(n)
    r = np.concatenate([k, k[1:], k[:-1], [0, n - 1]])
    c = np.concatenate([k, k[:-1], k[1:], [n - 1, 0]])
    assert coo_handle(n, r, c, np.ones(r.size)).step_diagonals() == 0
    r, c, v = adversarial.random_spd_coo(3000, 6.0, seed=2)
    assert coo_handle(3000, r, c, v).step_diagonals() == 0
    rp, cp, vp = poisson2d_coo(20)
    V = np.stack([vp, 2 * vp]).astype(np.float32)
    assert coo_handle(400, rp, cp, V).step_diagonals() == 0

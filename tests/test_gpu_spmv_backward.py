"""GPU backward of y = A x (sla_spmv_backward) against the oracle's
spmv_backward: A^T g normwise within 1e-12 (fp64) / 1e-5 (fp32) like the
forward SpMV, grad_vals[k] = g[row k] x[col k] bit-exact in fp64 (one rounded
product, the same on both sides) and within one fp32 rounding otherwise.
Covers unsymmetric irregular patterns with empty and long rows, batches (B a
multiple of the 16-byte system block, 1, 2, 3 and 8 blocks, or not: blocks of
one system), the
reordered solver, the symmetric-flag shortcut, new values after the first
backward, and autograd through SparseCSR.mv with duplicated COO input."""
import numpy as np
import pytest
import torch

import oracle
from differentiable_sparse_linear_csr_amd import SparseCSR
from workloads import adversarial, make_workload

from gpu_util import dev, host, rel

pytestmark = pytest.mark.gpu


def handle(n, r, c, v, **kw):
    return SparseCSR.from_coo(dev(r, torch.int64), dev(c, torch.int64), dev(v), n, **kw)


def check(A, r, c, V, n, X, G, dtype):
    ref = oracle.coo_to_csr(n, r, c, V)
    gx_o, gv_o = oracle.spmv_backward(ref["row_ptr"], ref["col"], ref["vals"], X, G)
    gx, gv = A.matvec_backward_raw(dev(X), dev(G))
    gx, gv = np.atleast_2d(host(gx)), np.atleast_2d(host(gv))
    gx_o, gv_o = np.atleast_2d(gx_o), np.atleast_2d(gv_o)
    tol = 1e-12 if dtype == np.float64 else 1e-5
    for s in range(gx.shape[0]):
        assert rel(gx[s], gx_o[s]) <= tol, (s, rel(gx[s], gx_o[s]))
        if dtype == np.float64:
            assert np.array_equal(gv[s], gv_o[s])
        else:
            assert np.all(np.abs(gv[s] - gv_o[s]) <= 2 ** -23 * np.abs(gv_o[s]))


@pytest.mark.parametrize("dtype,B", [(np.float64, 1), (np.float32, 1), (np.float64, 3),
                                     (np.float32, 8), (np.float64, 2), (np.float32, 4),
                                     (np.float64, 4), (np.float64, 6), (np.float32, 12),
                                     (np.float32, 32), (np.float32, 3), (np.float64, 5)])
def test_unsymmetric_irregular(dtype, B):
    n = 40009
    lengths = np.random.default_rng(5).integers(0, 12, n)
    lengths[[1, 2, n - 1]] = 0
    lengths[100], lengths[200] = 700, 129
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=6)
    V = np.random.default_rng(7).standard_normal((B, v.shape[0])).astype(dtype)
    X = np.random.default_rng(8).standard_normal((B, n)).astype(dtype)
    G = np.random.default_rng(9).standard_normal((B, n)).astype(dtype)
    if B == 1:
        V, X, G = V[0], X[0], G[0]
    print(f"spmv backward n={n} nnz={v.shape[0]} B={B} {np.dtype(dtype).name}", flush=True)
    for reorder in (False, True):
        A = handle(n, r, c, V, reorder=reorder)
        assert A.layout()["reordered"] == reorder
        check(A, r, c, V, n, X, G, dtype)


def test_workload_matrices_and_symmetric_shortcut():
    for name, size in [("knn_laplacian_2m", 70000), ("diffusion3d_128", 30)]:
        w = make_workload(name, size=size)
        x = np.random.default_rng(10).standard_normal(w.n)
        g = np.random.default_rng(11).standard_normal(w.n)
        for sym in (False, True):
            A = handle(w.n, w.rows, w.cols, w.vals, check_symmetric=sym)
            check(A, w.rows, w.cols, w.vals, w.n, x, g, np.float64)
    # a batch: grad_y goes to the internal layout once for A^T g and the value
    # gradient, also when A^T is the handle itself
    w = make_workload("batched_diffusion2d_512x32", size=40, batch=8)
    X = np.random.default_rng(12).standard_normal((8, w.n)).astype(np.float32)
    G = np.random.default_rng(13).standard_normal((8, w.n)).astype(np.float32)
    for sym in (False, True):
        A = handle(w.n, w.rows, w.cols, w.vals, check_symmetric=sym)
        check(A, w.rows, w.cols, w.vals, w.n, X, G, np.float32)
        gx, _ = A.matvec_backward_raw(dev(X), dev(G), want_vals=False)
        gx2, _ = A.matvec_backward_raw(dev(X), dev(G))
        assert host(gx).tobytes() == host(gx2).tobytes()


@pytest.mark.parametrize("reorder", [False, True])
def test_new_values_reach_the_transpose(reorder):
    # reordered: the backward runs on the inner handle's transpose
    n = 30000
    lengths = np.random.default_rng(12).integers(1, 9, n)
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=13)
    A = handle(n, r, c, v, reorder=reorder)
    assert A.layout()["reordered"] == reorder
    x = np.random.default_rng(14).standard_normal(n)
    g = np.random.default_rng(15).standard_normal(n)
    check(A, r, c, v, n, x, g, np.float64)            # builds A^T
    v2 = np.random.default_rng(16).standard_normal(v.shape[0])
    A.set_values(dev(v2))
    check(A, r, c, v2, n, x, g, np.float64)           # refreshed values


def test_autograd_through_mv_with_duplicates():
    n = 5000
    lengths = np.random.default_rng(17).integers(0, 10, n)
    r, c, v = adversarial.rows_of_lengths(lengths, n, seed=18)
    r, c, v = adversarial.split_duplicates(r, c, v, seed=19, frac=0.3)   # also shuffles
    A = handle(n, r, c, v)
    vals = dev(v).requires_grad_(True)
    x = dev(np.random.default_rng(20).standard_normal(n)).requires_grad_(True)
    w = dev(np.random.default_rng(21).standard_normal(n))
    loss = (A.mv(x, vals) * w).sum()
    gvals, gx = torch.autograd.grad(loss, [vals, x])
    ref = oracle.coo_to_csr(n, r, c, v)
    gx_o, gv_o = oracle.spmv_backward(ref["row_ptr"], ref["col"], ref["vals"], host(x), host(w))
    assert rel(host(gx), gx_o) <= 1e-12
    # every input entry receives the gradient of the CSR entry it merged into
    assert np.array_equal(host(gvals), gv_o[ref["slot"]])


@pytest.mark.parametrize("case", ["poisson2d_1100", "diffusion3d_40", "banded_irregular",
                                  "banded_long_rows", "tiny"])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_ring_gradient_matches_tile_kernel(case, dtype):
    """The value gradient in the ring form (single system, every tile small
    and narrow: four tiles of entries and two of gathers in flight per
    wavefront, whole 4-entry groups stored at once) against the
    one-tile-per-wavefront kernel (SLA_OPT_SPMV_RING off) on the same
    handle, bit for bit, and against the oracle; also into an output that
    starts 8 bytes past a 16-byte boundary (every group stored entry by
    entry)."""
    from differentiable_sparse_linear_csr_amd import _lib
    from differentiable_sparse_linear_csr_amd.sparse import _ptr, _stream
    from test_gpu_spmv import banded_irregular
    if case in ("poisson2d_1100", "diffusion3d_40"):
        w = (make_workload("poisson2d_11548", size=1100) if case == "poisson2d_1100"
             else make_workload("diffusion3d_128", size=40))
        n, c, v = w.n, w.cols, w.vals
        r = np.repeat(np.arange(n), np.diff(w.row_ptr)) if w.fmt == "csr" else w.rows
    elif case == "banded_irregular":
        n = 300000
        r, c, v = banded_irregular(n, 7)
    elif case == "banded_long_rows":
        # two rows past the tile limit (one workgroup each) among ring tiles
        n = 200000
        r, c, v = banded_irregular(n, 8)
        rng = np.random.default_rng(9)
        extra = []
        for row, m in ((1234, 200), (150001, 129)):
            cols = np.setdiff1d(np.unique(np.clip(row + rng.integers(-1500, 1501, 3 * m), 0,
                                                  n - 1)), c[r == row])[:m]
            extra.append((np.full(cols.size, row), cols, rng.standard_normal(cols.size)))
        r = np.concatenate([r] + [e[0] for e in extra])
        c = np.concatenate([c] + [e[1] for e in extra])
        v = np.concatenate([v] + [e[2] for e in extra])
        order = np.lexsort((c, r))
        r, c, v = r[order], c[order], v[order]
    else:
        n = 10
        i = np.arange(n)
        r = np.concatenate([i, i[1:], i[:-1]])
        c = np.concatenate([i, i[:-1], i[1:]])
        v = np.concatenate([np.full(n, 2.0), np.full(n - 1, -1.0), np.full(n - 1, -1.0)])
    v = v.astype(dtype)
    print(f"ring gradient: {case} n={n} nnz={v.size} {np.dtype(dtype).name}", flush=True)
    A = handle(n, r, c, v)
    lay = A.layout()
    assert lay["narrow_columns"] and lay["ring_tiles"], lay
    x = np.random.default_rng(31).standard_normal(n).astype(dtype)
    g = np.random.default_rng(32).standard_normal(n).astype(dtype)
    _, gv_ring = A.matvec_backward_raw(dev(x), dev(g), want_x=False)
    # the same gradient into an output 8 bytes off a 16-byte boundary
    buf = torch.zeros(A.nnz + 2, dtype=gv_ring.dtype, device=gv_ring.device)
    off = 1 if dtype == np.float64 else 2
    gv_off = buf[off:off + A.nnz]
    assert gv_off.data_ptr() % 16 == 8
    xd, gd = dev(x), dev(g)
    _lib.check(_lib.load().sla_spmv_backward(A._h, _ptr(xd), _ptr(gd), None, _ptr(gv_off),
                                             _stream(xd.device)))
    A.set_option(_lib.SLA_OPT_SPMV_RING, 0)
    _, gv_tile = A.matvec_backward_raw(dev(x), dev(g), want_x=False)
    A.set_option(_lib.SLA_OPT_SPMV_RING, 1)
    assert host(gv_ring).tobytes() == host(gv_tile).tobytes()
    assert host(gv_off).tobytes() == host(gv_tile).tobytes()
    # nothing written outside the output
    assert host(buf[:off]).tobytes() == bytes(off * buf.element_size())
    assert host(buf[off + A.nnz:]).tobytes() == bytes((2 - off) * buf.element_size())
    check(A, r, c, v, n, x, g, dtype)


@pytest.mark.parametrize("dtype,B", [(np.float64, 1), (np.float32, 1), (np.float64, 2),
                                     (np.float32, 4)])
def test_degenerate_patterns(dtype, B):
    """One entry (n = 1), an empty matrix (nnz = 0: A^T g = 0 and no value
    gradient), and a 900-row matrix whose only entries are in rows 2, 4 and
    a 700-entry row 6 (one long row beside short tiles, most rows empty),
    single and batched (one 16-byte block of systems)."""
    rng = np.random.default_rng(40)
    z = np.zeros(0, np.int64)
    lengths = np.array([0, 0, 3, 0, 1, 0, 700, 0, 0])
    r9, c9, v9 = adversarial.rows_of_lengths(lengths, 900, seed=3)
    cases = [(1, np.array([0]), np.array([0]), np.array([2.0])), (5, z, z, np.zeros(0)),
             (900, r9, c9, v9)]
    for n, r, c, v in cases:
        print(f"degenerate backward n={n} nnz={v.size} B={B} {np.dtype(dtype).name}", flush=True)
        V = np.stack([v * (1.0 + s) for s in range(B)]).astype(dtype) if B > 1 else v.astype(dtype)
        X = rng.standard_normal((B, n)).astype(dtype)
        G = rng.standard_normal((B, n)).astype(dtype)
        if B == 1:
            X, G = X[0], G[0]
        A = handle(n, r, c, V)
        ref = oracle.coo_to_csr(n, r, c, V)
        gx_o, gv_o = oracle.spmv_backward(ref["row_ptr"], ref["col"], ref["vals"], X, G)
        gx, gv = A.matvec_backward_raw(dev(X), dev(G))
        gx, gv = host(gx), host(gv)
        assert gv.shape == gv_o.shape
        if v.size == 0:
            assert not np.any(gx)
            continue
        tol = 1e-12 if dtype == np.float64 else 1e-5
        for s in range(B):
            a, o = np.atleast_2d(gx)[s], np.atleast_2d(gx_o)[s]
            assert np.linalg.norm(a - o) <= tol * np.linalg.norm(o), s
            ga, go = np.atleast_2d(gv)[s], np.atleast_2d(gv_o)[s]
            if dtype == np.float64:
                assert np.array_equal(ga, go)
            else:
                assert np.all(np.abs(ga - go) <= 2 ** -23 * np.abs(go))


def test_options_with_the_transpose():
    """Options set on A after A^T is built (they are passed on to it) and
    before (A^T starts with them): A^T g stays bitwise what the ring form
    gives (the one-tile-ahead form has the same tiles and sums) and matches
    the oracle."""
    from differentiable_sparse_linear_csr_amd import _lib
    w = make_workload("poisson2d_11548", size=300)
    n = w.n
    r = np.repeat(np.arange(n), np.diff(w.row_ptr))
    rng = np.random.default_rng(50)
    v = w.vals * (1.0 + 0.1 * rng.random(w.vals.size))     # unsymmetric values
    A = handle(n, r, w.cols, v)
    x, g = dev(rng.standard_normal(n)), dev(rng.standard_normal(n))
    gx_ring, _ = A.matvec_backward_raw(x, g, want_vals=False)     # builds A^T
    A.set_option(_lib.SLA_OPT_SPMV_RING, 0)
    gx_one, _ = A.matvec_backward_raw(x, g, want_vals=False)
    A.set_option(_lib.SLA_OPT_SPMV_RING, 1)
    assert host(gx_one).tobytes() == host(gx_ring).tobytes()
    B = handle(n, r, w.cols, v)
    B.set_option(_lib.SLA_OPT_SPMV_RING, 0)                       # before A^T exists
    B.set_option(_lib.SLA_OPT_CHECK_INTERVAL, 3)
    gx_b, _ = B.matvec_backward_raw(x, g, want_vals=False)
    assert host(gx_b).tobytes() == host(gx_ring).tobytes()
    ref = oracle.coo_to_csr(n, r, w.cols, v)
    gx_o, _ = oracle.spmv_backward(ref["row_ptr"], ref["col"], ref["vals"], host(x), host(g))
    assert rel(host(gx_ring), gx_o) <= 1e-12


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_band_aligned_tiles(dtype):
    """A 4100^2 Poisson matrix (16.8M rows, grid stride 4100) gets
    band-aligned tiles, whose SpMV and value-gradient kernels walk one panel
    per XCD (one band of rows after the other): A^T g and g_i x_j against the
    oracle, from the CSR input the 133M-DOF workload uses."""
    w = make_workload("poisson2d_11548", size=4100)
    assert w.n >= 1 << 20
    rows = np.repeat(np.arange(w.n), np.diff(w.row_ptr))
    v = w.vals.astype(dtype)
    print(f"band-aligned backward n={w.n} {np.dtype(dtype).name}", flush=True)
    A = SparseCSR.from_csr(dev(w.row_ptr, torch.int64), dev(w.cols, torch.int32), dev(v))
    x = np.random.default_rng(14).standard_normal(w.n).astype(dtype)
    g = np.random.default_rng(15).standard_normal(w.n).astype(dtype)
    check(A, rows, w.cols, v, w.n, x, g, dtype)

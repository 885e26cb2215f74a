"""Pins for the oracle's COO -> CSR assembly and CSR validation (CPU only).

The pages never spell out the storage format; the reading pinned here is the
standard COO semantics (SparseTensor built from row/col/value triples, torch-sla
API section): stable (row, col) order, duplicates summed in input order, slot
map from input entry to CSR position.
"""
import numpy as np
import pytest
import scipy.sparse as sp

import oracle
from workloads import adversarial, make_workload


def brute_force_dense(n, rows, cols, vals):
    """Dense accumulation in input order: first value at a position, then += ."""
    V = np.atleast_2d(vals)
    D = np.zeros((V.shape[0], n, n), V.dtype)
    seen = np.zeros((n, n), bool)
    for e in range(rows.shape[0]):
        r, c = int(rows[e]), int(cols[e])
        if not seen[r, c]:
            D[:, r, c] = V[:, e]
            seen[r, c] = True
        else:
            D[:, r, c] = D[:, r, c] + V[:, e]
    return D, seen


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_assembly_matches_dense_accumulation_bitwise(dtype, seed):
    n = 37
    r, c, v = adversarial.random_spd_coo(n, 4.0, seed)
    rng = np.random.default_rng(100 + seed)
    # order-sensitive duplicate parts: huge +/- pairs around a small value
    v = v.astype(dtype)
    rd, cd, vd = adversarial.split_duplicates(r, c, v, seed=seed, frac=0.5)
    k = rng.integers(0, rd.shape[0], 5)
    rd = np.concatenate([rd, rd[k], rd[k]])
    cd = np.concatenate([cd, cd[k], cd[k]])
    vd = np.concatenate([vd, np.full(5, 1e16, dtype), np.full(5, -1e16, dtype)])
    perm = rng.permutation(rd.shape[0])
    rd, cd, vd = rd[perm], cd[perm], vd[perm]

    out = oracle.coo_to_csr(n, rd, cd, vd)
    D, seen = brute_force_dense(n, rd, cd, vd)
    # pattern: row-major positions of the dense mask
    pr, pc = np.nonzero(seen)
    assert out["nnz"] == pr.shape[0]
    assert np.array_equal(np.diff(out["row_ptr"]), np.bincount(pr, minlength=n))
    assert np.array_equal(out["col"], pc)
    got = out["vals"]
    assert got.dtype == dtype
    assert np.array_equal(got.view(np.uint8), D[0][pr, pc].view(np.uint8))  # bit-exact
    # slot map: every input entry points at its own (row, col)
    rows_of_slot = np.repeat(np.arange(n), np.diff(out["row_ptr"]))
    assert np.array_equal(rows_of_slot[out["slot"]], rd)
    assert np.array_equal(out["col"][out["slot"]], cd)


def test_summation_order_is_input_order():
    # (1e16 + 1) - 1e16 = 0 in fp64, while (1e16 - 1e16) + 1 = 1
    rows = np.array([0, 0, 0, 1])
    cols = np.array([0, 0, 0, 1])
    a = oracle.coo_to_csr(2, rows, cols, np.array([1e16, 1.0, -1e16, 2.0]))
    b = oracle.coo_to_csr(2, rows, cols, np.array([1e16, -1e16, 1.0, 2.0]))
    assert a["vals"][0] == 0.0 and b["vals"][0] == 1.0


def test_batched_assembly_shares_permutation():
    n = 20
    r, c, v = adversarial.random_spd_coo(n, 3.0, 7)
    V = np.stack([v, 2 * v + 1, -v])
    rd, cd, Vd = adversarial.split_duplicates(r, c, V, seed=3)
    out = oracle.coo_to_csr(n, rd, cd, Vd)
    for s in range(3):
        single = oracle.coo_to_csr(n, rd, cd, Vd[s])
        assert np.array_equal(single["vals"], out["vals"][s])
        assert np.array_equal(single["col"], out["col"])
        assert np.array_equal(single["slot"], out["slot"])


def test_pattern_matches_scipy_sum_duplicates():
    n = 50
    r, c, v = adversarial.random_spd_coo(n, 5.0, 11)
    rng = np.random.default_rng(5)
    vi = rng.integers(-8, 9, r.shape[0]).astype(np.float64)  # exact under any summation order
    rd, cd, vd = adversarial.split_duplicates(r, c, vi, seed=2)
    vd = np.round(vd)  # integers: any order gives the same sum
    out = oracle.coo_to_csr(n, rd, cd, vd)
    S = sp.coo_matrix((vd, (rd, cd)), shape=(n, n))
    S.sum_duplicates()
    S = S.tocsr()
    S.sort_indices()
    # scipy drops nothing here (no explicit zeros are removed by sum_duplicates)
    assert np.array_equal(out["row_ptr"], S.indptr)
    assert np.array_equal(out["col"], S.indices)
    assert np.array_equal(out["vals"], S.data)


def test_invariants_on_generators():
    for name, size in [("poisson2d_64", None), ("diffusion3d_128", 9), ("knn_laplacian_2m", 3000),
                       ("batched_diffusion2d_512x32", 12)]:
        w = make_workload(name, size=size, batch=3 if name.startswith("batched") else None)
        out = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
        rp, col = out["row_ptr"], out["col"]
        assert rp[0] == 0 and rp[-1] == out["nnz"] == w.nnz  # generators emit no duplicates
        assert np.all(np.diff(rp) >= 0)
        for i in range(0, w.n, max(1, w.n // 50)):
            seg = col[rp[i]:rp[i + 1]]
            assert np.all(np.diff(seg) > 0)
        assert np.array_equal(out["slot"], np.arange(w.nnz))  # already sorted input
        assert oracle.check_csr(w.n, rp, col) == oracle.OK


def test_index_range_rejected():
    with pytest.raises(oracle.OracleError) as e:
        oracle.coo_to_csr(3, np.array([0, 3]), np.array([0, 1]), np.array([1.0, 2.0]))
    assert e.value.code == oracle.ERR_INDEX_RANGE
    with pytest.raises(oracle.OracleError) as e:
        oracle.coo_to_csr(3, np.array([0, 1]), np.array([-1, 1]), np.array([1.0, 2.0]))
    assert e.value.code == oracle.ERR_INDEX_RANGE


def test_check_csr_detects_malformed_input():
    rp = np.array([0, 2, 3, 5])
    col = np.array([0, 2, 1, 0, 2])
    assert oracle.check_csr(3, rp, col) == oracle.OK
    assert oracle.check_csr(3, rp, np.array([2, 0, 1, 0, 2])) == oracle.ERR_INVALID_CSR  # unsorted
    assert oracle.check_csr(3, rp, np.array([0, 0, 1, 0, 2])) == oracle.ERR_INVALID_CSR  # repeated
    assert oracle.check_csr(3, np.array([0, 3, 2, 5]), col) == oracle.ERR_INVALID_CSR  # decreasing
    assert oracle.check_csr(3, np.array([1, 2, 3, 5]), col) == oracle.ERR_INVALID_CSR  # rp[0] != 0
    assert oracle.check_csr(3, rp, np.array([0, 3, 1, 0, 2])) == oracle.ERR_INDEX_RANGE


def test_empty_and_single_entry():
    out = oracle.coo_to_csr(4, np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0))
    assert out["nnz"] == 0 and np.array_equal(out["row_ptr"], np.zeros(5))
    out = oracle.coo_to_csr(4, np.array([2]), np.array([1]), np.array([3.5]))
    assert np.array_equal(out["row_ptr"], [0, 0, 0, 1, 1]) and out["col"][0] == 1

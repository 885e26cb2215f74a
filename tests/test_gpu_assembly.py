"""GPU CSR assembly versus the oracle: bit-exact row_ptr, col_idx, values and
slot map, for sorted, shuffled and duplicated COO input, fp32/fp64, batched
value sets, int32/int64 indices; CSR input validation and adoption."""
import numpy as np
import pytest
import torch

import oracle
from differentiable_sparse_linear_csr_amd import _lib, SlaError, SparseCSR
from workloads import adversarial, make_workload

from gpu_util import bits_equal, coo_handle, dev, host

pytestmark = pytest.mark.gpu


def check_against_oracle(A: SparseCSR, n, rows, cols, vals):
    ref = oracle.coo_to_csr(n, rows, cols, vals)
    rp, col, v = A.csr()
    assert A.nnz == ref["nnz"]
    assert np.array_equal(host(rp).astype(np.int64), ref["row_ptr"])
    assert np.array_equal(host(col).astype(np.int64), ref["col"])
    assert bits_equal(host(v), ref["vals"])
    assert np.array_equal(host(A.slot()), ref["slot"])


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("idx", [torch.int32, torch.int64])
@pytest.mark.parametrize("case", ["sorted", "shuffled", "duplicates"])
def test_assembly_bit_exact(dtype, idx, case):
    print(f"assembly case={case} dtype={np.dtype(dtype).name} idx={idx}", flush=True)
    n = 3000
    r, c, v = adversarial.random_spd_coo(n, 9.0, 5, max_row=1500)
    v = v.astype(dtype)
    if case == "shuffled":
        r, c, v = adversarial.shuffled(r, c, v, seed=1)
    elif case == "duplicates":
        r, c, v = adversarial.split_duplicates(r, c, v, seed=2, frac=0.4)
        # order-sensitive duplicate sums
        k = np.arange(0, r.shape[0], 97)
        r = np.concatenate([r, r[k], r[k]])
        c = np.concatenate([c, c[k], c[k]])
        v = np.concatenate([v, np.full(k.shape, 1e7, dtype), np.full(k.shape, -1e7, dtype)])
        r, c, v = adversarial.shuffled(r, c, v, seed=3)
    A = coo_handle(n, r, c, v, idx=idx)
    check_against_oracle(A, n, r, c, v)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_batched_assembly_bit_exact(dtype):
    w = make_workload("batched_diffusion2d_512x32", size=40, batch=7)
    vals = w.vals.astype(dtype)
    r, c, V = adversarial.split_duplicates(w.rows.astype(np.int64), w.cols.astype(np.int64), vals,
                                           seed=4)
    A = coo_handle(w.n, r, c, V)
    assert A.batch == 7
    check_against_oracle(A, w.n, r, c, V)


def test_edge_cases():
    # n = 1; empty matrix; empty rows; one entry
    A = coo_handle(1, np.array([0]), np.array([0]), np.array([2.0]))
    check_against_oracle(A, 1, np.array([0]), np.array([0]), np.array([2.0]))
    z = np.zeros(0, np.int64)
    A = coo_handle(5, z, z, np.zeros(0))
    rp, col, v = A.csr()
    assert A.nnz == 0 and np.array_equal(host(rp), np.zeros(6))
    lengths = np.array([0, 0, 3, 0, 1, 0, 700, 0, 0])
    r, c, v = adversarial.rows_of_lengths(lengths, 900, seed=3)
    r, c, v = adversarial.shuffled(r, c, v, seed=9)
    A = coo_handle(900, r, c, v)
    check_against_oracle(A, 900, r, c, v)


def test_index_out_of_range_rejected():
    with pytest.raises(SlaError) as e:
        coo_handle(4, np.array([0, 4]), np.array([0, 1]), np.array([1.0, 1.0]))
    assert e.value.status == _lib.SLA_ERR_INDEX_RANGE
    with pytest.raises(SlaError) as e:
        coo_handle(4, np.array([0, 1]), np.array([0, -1]), np.array([1.0, 1.0]))
    assert e.value.status == _lib.SLA_ERR_INDEX_RANGE


@pytest.mark.parametrize("rp_dtype", [torch.int32, torch.int64])
def test_csr_input_adopted(rp_dtype):
    w = make_workload("poisson2d_11548", size=70)
    A = SparseCSR.from_csr(dev(w.row_ptr, rp_dtype), dev(w.cols, torch.int32), dev(w.vals))
    rp, col, v = A.csr()
    assert A.row_index_dtype == rp_dtype
    assert np.array_equal(host(rp).astype(np.int64), w.row_ptr)
    assert np.array_equal(host(col), w.cols)
    assert bits_equal(host(v), w.vals)
    assert np.array_equal(host(A.slot()), np.arange(w.nnz))


@pytest.mark.parametrize("bad", ["unsorted", "repeat", "decreasing", "start", "end", "range"])
def test_csr_input_validation(bad):
    rp = np.array([0, 2, 3, 5], np.int64)
    col = np.array([0, 2, 1, 0, 2], np.int32)
    expect = _lib.SLA_ERR_INVALID_CSR
    if bad == "unsorted":
        col = np.array([2, 0, 1, 0, 2], np.int32)
    elif bad == "repeat":
        col = np.array([0, 0, 1, 0, 2], np.int32)
    elif bad == "decreasing":
        rp = np.array([0, 3, 2, 5], np.int64)
    elif bad == "start":
        rp = np.array([1, 2, 3, 5], np.int64)
    elif bad == "end":
        rp = np.array([0, 2, 3, 4], np.int64)
    elif bad == "range":
        col = np.array([0, 3, 1, 0, 2], np.int32)
        expect = _lib.SLA_ERR_INDEX_RANGE
    with pytest.raises(SlaError) as e:
        SparseCSR.from_csr(dev(rp), dev(col), dev(np.ones(5)))
    assert e.value.status == expect


def test_symmetry_flag():
    w = make_workload("diffusion3d_128", size=8)
    coo_handle(w.n, w.rows, w.cols, w.vals, check_symmetric=True)
    v = w.vals.copy()
    k = int(np.nonzero(w.rows != w.cols)[0][3])
    v[k] = np.nextafter(v[k], 0.0)
    with pytest.raises(SlaError) as e:
        coo_handle(w.n, w.rows, w.cols, v, check_symmetric=True)
    assert e.value.status == _lib.SLA_ERR_NOT_SYMMETRIC


def test_set_values_and_gather():
    n = 500
    r, c, v = adversarial.random_spd_coo(n, 6.0, 8)
    r, c, v = adversarial.split_duplicates(r, c, v, seed=5)
    A = coo_handle(n, r, c, v)
    v2 = v * 3.0 - 0.25
    A.set_values(dev(v2))
    check_against_oracle(A, n, r, c, v2)
    ref = oracle.coo_to_csr(n, r, c, v2)
    g = A.gather_to_input(A.csr()[2])
    assert bits_equal(host(g), ref["vals"][ref["slot"]])

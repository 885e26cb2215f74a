"""GPU parity of segmented solves (SparseTensorList: systems with distinct
patterns solved together). Each member is compared with the oracle's PCG on
that member alone: outcome, iterations within +-2 (exact for immediate
convergence and breakdown), x within 1e-8 (fp32 storage 1e-4), and the
adjoint's lambda and value gradient likewise."""
import numpy as np
import pytest
import torch

import oracle
from differentiable_sparse_linear_csr_amd import SlaError, SparseTensorList, _lib
from workloads import adversarial, make_workload, poisson2d_coo

from gpu_util import dev, host, rel

pytestmark = pytest.mark.gpu


def members():
    out = []
    r, c, v = poisson2d_coo(30)
    out.append(("poisson30", 900, r, c, v))
    w = make_workload("diffusion3d_128", size=12)
    out.append(("diffusion12", w.n, w.rows, w.cols, w.vals))
    r, c, v = adversarial.random_spd_coo(3001, 8.0, 5, skew=False)
    out.append(("random3001", 3001, r, c, v))
    w = make_workload("knn_laplacian_2m", size=2500)
    out.append(("knn2500", w.n, w.rows, w.cols, w.vals))
    out.append(("one", 1, np.array([0]), np.array([0]), np.array([2.0])))
    r, c, v = poisson2d_coo(10)
    out.append(("zero_rhs", 100, r, c, v))
    out.append(("indefinite", 2, np.array([0, 0, 1, 1]), np.array([0, 1, 0, 1]),
                np.array([1.0, 2.0, 2.0, 1.0])))
    r, c, v = poisson2d_coo(70)
    out.append(("poisson70", 4900, r, c, v))
    return out


def build(ms, dtype):
    return SparseTensorList.from_coo_list([dev(m[2], torch.int64) for m in ms],
                                          [dev(m[3], torch.int64) for m in ms],
                                          [dev(m[4].astype(dtype)) for m in ms],
                                          [m[1] for m in ms])


def rhs(ms, dtype, seed):
    bs = []
    for q, m in enumerate(ms):
        b = np.random.default_rng(seed + q).standard_normal(m[1])
        if m[0] == "zero_rhs":
            b[:] = 0.0
        if m[0] == "indefinite":
            b = np.array([1.0, -1.0])
        bs.append(b.astype(dtype))
    return bs


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_members_match_their_own_solves(dtype):
    ms = members()
    A = build(ms, dtype)
    assert A.nseg == len(ms)
    bs = rhs(ms, dtype, 100)
    gs = rhs(ms, dtype, 200)
    tol = 1e-10 if dtype == np.float64 else 1e-5
    x, info = A.solve_raw(dev(np.concatenate(bs)), tol, 3000)
    gb, gv, ainfo = A.adjoint_raw(x, dev(np.concatenate(gs)), tol, 3000)
    X, GB, GV = host(x), host(gb), host(gv)
    xtol = 1e-8 if dtype == np.float64 else 1e-4
    gtol = 1e-8 if dtype == np.float64 else 1e-3
    o, ko = 0, 0
    for q, (name, n, r, c, v) in enumerate(ms):
        ref = oracle.coo_to_csr(n, r, c, v.astype(dtype))
        xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], bs[q], tol, 3000)
        assert info.status[q] == oco, (name, info.status[q], oco)
        assert abs(info.iterations[q] - ito) <= 2, (name, info.iterations[q], ito)
        if name in ("zero_rhs", "indefinite"):
            assert info.iterations[q] == ito and not X[o:o + n].any()
        else:
            assert rel(X[o:o + n], xo) <= xtol, (name, rel(X[o:o + n], xo))
            lam, gvo, ita, _, oca = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo,
                                                   gs[q], tol, 3000)
            assert ainfo.status[q] == oca and abs(ainfo.iterations[q] - ita) <= 2
            assert rel(GB[o:o + n], lam) <= gtol, name
            nnz = ref["col"].shape[0]
            assert rel(GV[ko:ko + nnz], gvo) <= gtol, name
        o += n
        ko += ref["col"].shape[0]


def test_autograd_through_list_solve():
    ms = [m for m in members() if m[0] in ("poisson30", "random3001", "diffusion12")]
    A = build(ms, np.float64)
    vals = dev(np.concatenate([m[4] for m in ms])).requires_grad_(True)
    bs = [dev(b).requires_grad_(True) for b in rhs(ms, np.float64, 300)]
    ws = [dev(np.random.default_rng(400 + q).standard_normal(m[1])) for q, m in enumerate(ms)]
    xs = A.solve(bs, values=vals)
    loss = sum((x * w).sum() for x, w in zip(xs, ws))
    grads = torch.autograd.grad(loss, [vals] + bs)
    gvals = A.split_values(grads[0])
    for q, (name, n, r, c, v) in enumerate(ms):
        ref = oracle.coo_to_csr(n, r, c, v)
        xo, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], host(bs[q]), 1e-10, 3000)
        lam, gvo, *_ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, host(ws[q]),
                                      1e-10, 3000)
        assert rel(host(grads[1 + q]), lam) <= 1e-8
        assert rel(host(gvals[q]), gvo[ref["slot"]]) <= 1e-8


def test_entry_outside_its_block_is_rejected():
    v = [dev(np.array([1.0, 1.0])), dev(np.array([1.0, 1.0]))]
    r = [dev(np.array([0, 1]), torch.int64), dev(np.array([0, 1]), torch.int64)]
    # member 1's column -2 lands (after its offset of 2) in member 0's block
    c = [dev(np.array([0, 1]), torch.int64), dev(np.array([-2, 1]), torch.int64)]
    with pytest.raises(SlaError) as e:
        SparseTensorList.from_coo_list(r, c, v, [2, 2])
    assert e.value.status == _lib.SLA_ERR_INDEX_RANGE
    # a column past the whole matrix is an index error too
    c = [dev(np.array([0, 1]), torch.int64), dev(np.array([0, 2]), torch.int64)]
    with pytest.raises(SlaError) as e:
        SparseTensorList.from_coo_list(r, c, v, [2, 2])
    assert e.value.status == _lib.SLA_ERR_INDEX_RANGE


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_list_ring_spmv_matches_one_tile_ahead(dtype):
    """A list of stencil members (every tile small and narrow, so the list's
    SpMV takes the ring form, reading the per-tile live flags as words and
    skipping finished members' tiles): the solve bitwise equal with the ring
    on and off (same tiles, same per-tile dots), and every member against
    its own oracle solve."""
    ms = [m for m in members() if m[0] in ("poisson30", "diffusion12", "poisson70", "one",
                                           "zero_rhs")]
    A = build(ms, dtype)
    lay = A.layout()
    assert lay["ring_tiles"], lay
    bs = rhs(ms, dtype, 300)
    tol = 1e-10 if dtype == np.float64 else 1e-5
    xs = []
    for ring in (1, 0):
        A.set_option(_lib.SLA_OPT_SPMV_RING, ring)
        x, info = A.solve_raw(dev(np.concatenate(bs)), tol, 3000)
        xs.append((host(x), list(info.iterations)))
    assert xs[0][0].tobytes() == xs[1][0].tobytes() and xs[0][1] == xs[1][1]
    X = xs[0][0]
    o = 0
    for q, (name, n, r, c, v) in enumerate(ms):
        ref = oracle.coo_to_csr(n, r, c, v.astype(dtype))
        xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], bs[q], tol, 3000)
        assert abs(xs[0][1][q] - ito) <= 2, (name, xs[0][1][q], ito)
        assert rel(X[o:o + n], xo) <= (1e-8 if dtype == np.float64 else 1e-4), name
        o += n

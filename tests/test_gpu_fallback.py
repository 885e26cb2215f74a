"""Bounded grid-wide waits that give up. The single-kernel solve and the fused
update + direction kernel wait for other workgroups; when a wait gives up
(on a shared GPU their workgroups may not all run at once) the solve runs
again from the start on kernels without such waits. Here the host forces
it: SLA_OPT_SPIN_LIMIT = 0 makes every wait that is not satisfied at its
first poll give up at once, so every kernel still exits normally. The
results must equal the oracle's, and sla_csr_get_last_path must say what
ran."""
import numpy as np
import pytest

import oracle
from differentiable_sparse_linear_csr_amd import _lib
from workloads import make_workload

from gpu_util import coo_handle, dev, host, rel

pytestmark = pytest.mark.gpu
DEFAULT_SPINS = 1 << 22


def reference(w, v, b, tol, g=None):
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, v)
    xo, ito, _, oco = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, tol, w.maxit)
    out = {"x": xo, "it": np.atleast_1d(ito), "oc": np.atleast_1d(oco)}
    if g is not None:
        lam, gv, ita, _, _ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], xo, g, tol,
                                            w.maxit)
        out.update(lam=lam, gv=gv, ita=np.atleast_1d(ita))
    return out


def check(x, info, R, xtol, B=1):
    X = np.atleast_2d(host(x))
    XO = np.atleast_2d(R["x"])
    for s in range(B):
        assert info.status[s] == R["oc"][s] == oracle.CONVERGED
        assert abs(info.iterations[s] - R["it"][s]) <= 2, (s, info.iterations[s], R["it"][s])
        assert rel(X[s], XO[s]) <= xtol, (s, rel(X[s], XO[s]))


@pytest.mark.parametrize("coop", [1, 0])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_single_kernel_wait_gives_up(dtype, coop):
    w = make_workload("diffusion3d_128", size=32)
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    g = np.random.default_rng(4).standard_normal(w.n).astype(dtype)
    tol = 1e-10 if dtype == np.float64 else 1e-5
    xtol = 1e-8 if dtype == np.float64 else 1e-4
    R = reference(w, v, b, tol, g)
    A = coo_handle(w.n, w.rows, w.cols, v)
    A.set_option(_lib.SLA_OPT_COOPERATIVE, coop)
    x, info = A.solve_raw(dev(b), tol, w.maxit)
    assert A.last_path() == {"path": "single_kernel", "cooperative_refused": False,
                             "wait_timed_out": False}
    check(x, info, R, xtol)
    print(f"single-kernel wait gives up: {np.dtype(dtype).name} cooperative={coop}", flush=True)
    A.set_option(_lib.SLA_OPT_SPIN_LIMIT, 0)
    x0, info0 = A.solve_raw(dev(b), tol, w.maxit)
    lp = A.last_path()
    assert lp["path"] == "per_step" and lp["wait_timed_out"], lp
    check(x0, info0, R, xtol)
    gb, gv, ainfo = A.adjoint_raw(x0, dev(g), tol, w.maxit)
    assert A.last_path()["path"] == "per_step"
    assert abs(ainfo.iterations[0] - R["ita"][0]) <= 2
    assert rel(host(gb), R["lam"]) <= xtol * 10 and rel(host(gv), R["gv"]) <= xtol * 10
    # back to the default: the single kernel again (the fused update stays
    # off on this handle until it is switched on)
    A.set_option(_lib.SLA_OPT_SPIN_LIMIT, DEFAULT_SPINS)
    x1, info1 = A.solve_raw(dev(b), tol, w.maxit)
    assert A.last_path() == {"path": "single_kernel", "cooperative_refused": False,
                             "wait_timed_out": False}
    assert host(x1).tobytes() == host(x).tobytes()


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_fused_update_wait_gives_up(dtype):
    """Per-step path (single kernel off): the fused update + direction kernel's
    broadcast wait gives up; the solve runs again with the update and the
    direction as two kernels, and the handle keeps to them until the fused
    form is switched on again."""
    w = make_workload("diffusion3d_128", size=40)
    v, b = w.vals.astype(dtype), w.b.astype(dtype)
    tol = 1e-10 if dtype == np.float64 else 1e-5
    xtol = 1e-8 if dtype == np.float64 else 1e-4
    R = reference(w, v, b, tol)
    A = coo_handle(w.n, w.rows, w.cols, v)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_FOLD_DIRECTION, 0)   # unfused: update, then direction

    def solve_profiled():
        A.profile_reset()
        A.set_option(_lib.SLA_OPT_PROFILE, 1)
        x, info = A.solve_raw(dev(b), tol, w.maxit)
        prof = A.profile()
        A.set_option(_lib.SLA_OPT_PROFILE, 0)
        return x, info, prof

    x, info, prof = solve_profiled()
    assert prof["direction"][0] == 0          # fused: no separate direction kernel
    assert A.last_path() == {"path": "per_step", "cooperative_refused": False,
                             "wait_timed_out": False}
    check(x, info, R, xtol)
    A.set_option(_lib.SLA_OPT_SPIN_LIMIT, 0)
    for graphs in (1, 0):
        # the default polled graphs, then kernels launched one by one
        A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 1)
        A.set_option(_lib.SLA_OPT_USE_GRAPH, graphs)
        x0, info0 = A.solve_raw(dev(b), tol, w.maxit)
        lp = A.last_path()
        assert lp["path"] == "per_step" and lp["wait_timed_out"], lp
        check(x0, info0, R, xtol)
    A.set_option(_lib.SLA_OPT_USE_GRAPH, 1)
    A.set_option(_lib.SLA_OPT_SPIN_LIMIT, DEFAULT_SPINS)
    x2, info2, prof2 = solve_profiled()
    assert prof2["direction"][0] > 0          # the handle kept the two kernels
    assert not A.last_path()["wait_timed_out"]
    check(x2, info2, R, xtol)
    A.set_option(_lib.SLA_OPT_FUSED_UPDATE, 1)
    x3, info3, prof3 = solve_profiled()
    assert prof3["direction"][0] == 0
    assert host(x3).tobytes() == host(x).tobytes()


def test_batched_fused_update_wait_gives_up():
    """A batch whose update fits one resident pass (fused, per-system beta
    broadcast): every system against its oracle solve after the fallback."""
    B = 4
    w = make_workload("batched_diffusion2d_512x32", size=40, batch=B)
    tol = 1e-10
    R = reference(w, w.vals, w.b, tol)
    A = coo_handle(w.n, w.rows, w.cols, w.vals)
    A.set_option(_lib.SLA_OPT_RESIDENT, 0)
    A.set_option(_lib.SLA_OPT_SPIN_LIMIT, 0)
    x, info = A.solve_raw(dev(w.b), tol, w.maxit)
    lp = A.last_path()
    assert lp["path"] == "per_step" and lp["wait_timed_out"], lp
    check(x, info, R, 1e-8, B)


def test_reordered_and_bicgstab_paths_are_recorded():
    from differentiable_sparse_linear_csr_amd import SparseCSR
    w = make_workload("knn_laplacian_2m", size=20000)
    A = SparseCSR.from_coo(dev(w.rows), dev(w.cols), dev(w.vals), w.n, reorder=True)
    assert A.layout()["reordered"]
    R = reference(w, w.vals, w.b, w.tol)
    x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    assert A.last_path()["path"] == "single_kernel"
    check(x, info, R, 100 * w.tol)
    A.set_option(_lib.SLA_OPT_SPIN_LIMIT, 0)
    x, info = A.solve_raw(dev(w.b), w.tol, w.maxit)
    lp = A.last_path()
    assert lp["path"] == "per_step" and lp["wait_timed_out"], lp
    check(x, info, R, 100 * w.tol)
    xb, ib = A.solve_raw(dev(w.b), w.tol, w.maxit, method="bicgstab")
    assert A.last_path() == {"path": "per_step", "cooperative_refused": False,
                             "wait_timed_out": False}
    assert ib.status[0] == oracle.CONVERGED

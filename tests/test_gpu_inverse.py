"""GPU inverse-conductivity demonstration (experiments section of the
torch-sla pages, Figure 3) against the host reference built on the oracle:
the gradient of the misfit with respect to kappa (batched PCG solve of the
four experiments, batched adjoint, PyTorch's chain through the assembly)
within 1e-8 relative (both solves to 1e-12) on a 24x24 grid and on the
benchmarked 128x128 grid, and 150 Adam steps taken on the
GPU and, with the reference gradient, on the host: the trajectories agree to
1e-6 and the misfit falls."""
import numpy as np
import pytest
import torch

from differentiable_sparse_linear_csr_amd.inverse import ConductivityRecovery

import inverse_reference as ref
from gpu_util import host, rel

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [24, 128])   # 128: the benchmarked grid
def test_gradient_matches_reference(N):
    rec = ConductivityRecovery(N, sources=4, tol=1e-12, device="cuda:0")
    k0 = np.random.default_rng(3).uniform(0.7, 1.3, N * N)
    with torch.no_grad():
        rec.kappa.copy_(torch.as_tensor(k0))
    L = rec.loss()
    (dk,) = torch.autograd.grad(L, [rec.kappa])
    G = ref.grid(N)
    F = ref.sources(G)
    U = ref.observations(G, F)
    assert rel(host(rec.u_obs), U) <= 1e-9
    Lr, dkr = ref.loss_and_grad(G, k0, F, U)
    assert abs(float(L.detach()) - Lr) <= 1e-8 * Lr
    assert rel(host(dk), dkr) <= 1e-8, rel(host(dk), dkr)


def test_adam_trajectory_matches_host():
    N, steps = 16, 150
    rec = ConductivityRecovery(N, sources=4, lr=0.03, total_steps=steps, tol=1e-12,
                               device="cuda:0")
    first = rec.step()
    for _ in range(steps - 1):
        last = rec.step()
    G = ref.grid(N)
    F = ref.sources(G)
    U = ref.observations(G, F)
    k = torch.ones(N * N, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([k], lr=0.03)
    sched = torch.optim.lr_scheduler.CosineAnnealingLR(opt, steps)
    for _ in range(steps):
        _, g = ref.loss_and_grad(G, k.detach().numpy(), F, U)
        opt.zero_grad()
        k.grad = torch.as_tensor(g)
        opt.step()
        sched.step()
    assert rel(host(rec.kappa), k.detach().numpy()) <= 1e-6
    assert last < 1e-2 * first
    rep = rec.report()
    assert rep["steps"] == steps and rep["misfit_rel"] < 0.1 * np.sqrt(first)

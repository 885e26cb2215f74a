"""Host checks of the inverse-conductivity demonstration (experiments section
of the torch-sla pages, Figure 3): the package's PyTorch assembly of A(kappa)
against the unit five-point Laplacian and against the test reference's
explicit assembly, and the reference gradient against central finite
differences of the loss through dense solves (which fixes the chain rule
through the assembly, independent of the adjoint)."""
import numpy as np
import torch

import oracle
from differentiable_sparse_linear_csr_amd.inverse import GridDiffusion
from workloads import poisson2d_coo

import inverse_reference as ref


def merged(n, r, c, v):
    out = oracle.coo_to_csr(n, r, c, v)
    return out["row_ptr"], out["col"], out["vals"]


def test_unit_conductivity_is_the_five_point_laplacian():
    N = 9
    g = GridDiffusion(N, "cpu")
    v = g.values(torch.ones(N * N, dtype=torch.float64)).numpy()
    a = merged(N * N, g.rows.numpy(), g.cols.numpy(), v)
    b = merged(N * N, *poisson2d_coo(N))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_package_assembly_matches_reference_assembly():
    N = 7
    G = ref.grid(N)
    k = np.random.default_rng(1).uniform(0.5, 1.5, N * N)
    g = GridDiffusion(N, "cpu")
    v = g.values(torch.as_tensor(k)).numpy()
    r2, c2, v2 = ref.coo(G, k)
    a = merged(N * N, g.rows.numpy(), g.cols.numpy(), v)
    b = merged(N * N, r2, c2, v2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.allclose(a[2], b[2], rtol=1e-15, atol=0)
    assert np.allclose(g.true_conductivity().numpy(), ref.true_kappa(G), rtol=1e-15)
    assert np.allclose(g.sources(4).numpy(), ref.sources(G), rtol=1e-14)


def test_reference_gradient_against_finite_differences():
    N = 5
    G = ref.grid(N)
    F = ref.sources(G)
    U = ref.observations(G, F)
    k = np.random.default_rng(2).uniform(0.7, 1.3, N * N)
    L, dk = ref.loss_and_grad(G, k, F, U)

    def dense_loss(kk):
        r, c, v = ref.coo(G, kk)
        A = np.zeros((N * N, N * N))
        np.add.at(A, (r, c), v)
        X = np.linalg.solve(A, F.T).T
        return float(((X - U) ** 2).sum() / (U * U).sum())

    assert abs(dense_loss(k) - L) <= 1e-10 * L
    h = 1e-6
    for i in (0, 3, 12, 24):
        e = np.zeros(N * N)
        e[i] = h
        fd = (dense_loss(k + e) - dense_loss(k - e)) / (2 * h)
        assert abs(fd - dk[i]) <= 1e-6 * np.abs(dk).max(), (i, fd, dk[i])

"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This package builds matrices (as COO triples or, for the largest grid, CSR
arrays produced in closed form from the stencil) and right-hand sides. It holds
none of the solver's arithmetic: no sorting or merging of entries, no matvec,
no Krylov step, no gradient. Every array is a plain numpy array on the host.
"""
from .generators import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_workload,
    poisson2d_coo,
    poisson2d_csr,
    diffusion2d_coo,
    diffusion3d_coo,
    convdiff2d_coo,
    rotating_flow,
    knn_laplacian_coo,
    normal_vector,
)
from . import adversarial  # noqa: F401

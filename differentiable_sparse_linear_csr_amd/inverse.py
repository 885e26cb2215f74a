"""Inverse conductivity recovery through the differentiable solve.

torch-sla's demonstration (experiments section, Figure 3 and its paragraph)
recovers the coefficient kappa of -div(kappa grad u) = f on a 2D grid from
observed solutions by running Adam on the data misfit, with A(kappa).solve(f)
inside the loop: 1500 steps, a true field with values in [0.5, 1.5], relative
errors of 2.3e-3 in kappa and 3.0e-5 in u. The pages give neither the grid,
nor the field, nor the sources, loss or step size; this module's choices:

- unit square, N x N interior nodes, spacing h = 1/(N+1), homogeneous
  Dirichlet boundary; five-point finite volumes with kappa at the nodes and
  the face coefficient between two nodes their arithmetic mean (a boundary
  face takes its node's kappa); rows scaled by h^2, so A(1) is the unit
  five-point Laplacian;
- true field kappa*(x, y) = 1 + 0.5 sin(2 pi x) sin(pi y), range [0.5, 1.5];
- S experiments (S = 4 by default): Gaussian sources of width 0.1 centred
  at (0.25, 0.25), (0.75, 0.25), (0.25, 0.75), (0.75, 0.75), times h^2 —
  one source leaves kappa unidentifiable where grad u vanishes; the S
  solves share A(kappa) and run as one batched solve;
- loss: sum_s ||u_s - u_obs,s||^2 / sum_s ||u_obs,s||^2 (relative misfit
  squared), kappa itself the parameter (start 1), Adam with step 0.03 and
  cosine decay over the run.

Only the solve (forward and adjoint) runs in the library's kernels; the
assembly of A's values from kappa is a few PyTorch elementwise operations
whose gradient PyTorch forms.
"""
from __future__ import annotations

import math
import time
from typing import Dict, List, Optional

import numpy as np
import torch

from .sparse import SparseCSR

SOURCE_CENTRES = [(0.25, 0.25), (0.75, 0.25), (0.25, 0.75), (0.75, 0.75)]
SOURCE_WIDTH = 0.1


class GridDiffusion:
    """Pattern and value assembly of A(kappa) on an N x N node grid.

    COO order: the N^2 diagonal entries, then entries (i, j) and then (j, i)
    of every interior face (i, j), horizontal faces first, each group in node
    order.
    """

    def __init__(self, N: int, device, dtype=torch.float64):
        self.N, self.n = N, N * N
        self.device, self.dtype = torch.device(device), dtype
        idx = np.arange(self.n).reshape(N, N)                        # [y, x]
        fi = np.concatenate([idx[:, :-1].ravel(), idx[:-1, :].ravel()])
        fj = np.concatenate([idx[:, 1:].ravel(), idx[1:, :].ravel()])
        y, x = np.divmod(np.arange(self.n), N)
        nbound = (x == 0).astype(np.float64) + (x == N - 1) + (y == 0) + (y == N - 1)
        rows = np.concatenate([np.arange(self.n), fi, fj])
        cols = np.concatenate([np.arange(self.n), fj, fi])
        t = lambda a, dt: torch.as_tensor(a, dtype=dt, device=self.device)
        self.rows, self.cols = t(rows, torch.int64), t(cols, torch.int64)
        self.fi, self.fj = t(fi, torch.int64), t(fj, torch.int64)
        self.nbound = t(nbound, dtype)
        self.h = 1.0 / (N + 1)
        self.xc = t((x + 1) * self.h, dtype)
        self.yc = t((y + 1) * self.h, dtype)

    def values(self, kappa: torch.Tensor) -> torch.Tensor:
        """COO values of A(kappa) (differentiable in kappa, shape [n])."""
        face = 0.5 * (kappa[self.fi] + kappa[self.fj])
        diag = kappa * self.nbound
        diag = diag.index_add(0, self.fi, face).index_add(0, self.fj, face)
        return torch.cat([diag, -face, -face])

    def true_conductivity(self) -> torch.Tensor:
        return 1.0 + 0.5 * torch.sin(2 * math.pi * self.xc) * torch.sin(math.pi * self.yc)

    def sources(self, S: int = 4) -> torch.Tensor:
        """[S, n] right-hand sides (Gaussian bumps times h^2)."""
        out = []
        for a, b in SOURCE_CENTRES[:S]:
            r2 = (self.xc - a) ** 2 + (self.yc - b) ** 2
            out.append(self.h ** 2 * torch.exp(-r2 / (2 * SOURCE_WIDTH ** 2)))
        return torch.stack(out)


class ConductivityRecovery:
    """The Adam loop of the demonstration; ``step()`` is one Adam step."""

    def __init__(self, N: int = 128, sources: int = 4, lr: float = 0.03, total_steps: int = 1500,
                 tol: float = 1e-10, maxit: int = 20000, device="cuda:0"):
        if not 1 <= sources <= len(SOURCE_CENTRES):
            raise ValueError(f"sources in [1, {len(SOURCE_CENTRES)}]")
        self.grid = g = GridDiffusion(N, device)
        self.S, self.tol, self.maxit = sources, tol, maxit
        self.F = g.sources(sources)
        self.kappa_true = g.true_conductivity()
        v_true = g.values(self.kappa_true)
        self.A = SparseCSR.from_coo(g.rows, g.cols, v_true.expand(sources, -1).contiguous(), g.n)
        with torch.no_grad():
            self.u_obs = self.A.solve(self.F, tol=tol, maxit=maxit)
            self.obs_norm2 = float((self.u_obs * self.u_obs).sum())
        self.kappa = torch.ones(g.n, dtype=g.dtype, device=g.device, requires_grad=True)
        self.opt = torch.optim.Adam([self.kappa], lr=lr)
        self.sched = torch.optim.lr_scheduler.CosineAnnealingLR(self.opt, total_steps)
        self.steps_done = 0
        self.iterations = 0      # PCG iterations (forward + adjoint), summed over sources

    def loss(self) -> torch.Tensor:
        vals = self.grid.values(self.kappa).expand(self.S, -1).contiguous()
        u = self.A.solve(self.F, values=vals, tol=self.tol, maxit=self.maxit)
        res = u - self.u_obs
        return (res * res).sum() / self.obs_norm2

    def step(self) -> float:
        self.opt.zero_grad()
        L = self.loss()
        L.backward()
        self.opt.step()
        self.sched.step()
        self.steps_done += 1
        self.iterations += sum(self.A.last_info.iterations) + sum(
            self.A.last_adjoint_info.iterations)
        return float(L.detach())

    def report(self) -> Dict[str, float]:
        with torch.no_grad():
            k, ks = self.kappa.detach(), self.kappa_true
            vals = self.grid.values(k).expand(self.S, -1).contiguous()
            u = self.A.solve(self.F, values=vals, tol=self.tol, maxit=self.maxit)
            misfit = math.sqrt(float(((u - self.u_obs) ** 2).sum()) / self.obs_norm2)
            return {"steps": self.steps_done,
                    "kappa_rel_error": float(torch.linalg.norm(k - ks) / torch.linalg.norm(ks)),
                    "misfit_rel": misfit,
                    "kappa_min": float(k.min()), "kappa_max": float(k.max())}


def recover(N: int = 128, steps: int = 1500, sources: int = 4, lr: float = 0.03,
            device="cuda:0", log_every: int = 0) -> Dict[str, object]:
    """Run the whole recovery; returns the final report, the loss history and
    the wall time per step."""
    rec = ConductivityRecovery(N, sources, lr, steps, device=device)
    history: List[float] = []
    torch.cuda.synchronize(device)
    t0 = time.perf_counter()
    for s in range(steps):
        history.append(rec.step())
        if log_every and (s % log_every == 0 or s == steps - 1):
            print(f"[recover] step {s} loss {history[-1]:.3e}", flush=True)
    torch.cuda.synchronize(device)
    dt = time.perf_counter() - t0
    out: Dict[str, object] = dict(rec.report())
    out.update({"ms_per_step": 1e3 * dt / max(steps, 1), "seconds": dt, "loss": history,
                "pcg_iterations": rec.iterations})
    return out

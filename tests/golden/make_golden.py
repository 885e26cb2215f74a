#!/usr/bin/env python3
"""Write the oracle's reference values for the full-size workloads.

Calls only the CPU oracle (``oracle/``) and the seeded generators
(``workloads/``); nothing here touches the GPU library. For each workload it
stores, for the forward solve and (where the workload has one) the adjoint:
iteration count, outcome, recursive relative residual, 2-norms, the values at
seeded sample indices, and projections onto seeded random vectors. The GPU
parity tests regenerate the same inputs and compare.

Usage: python tests/golden/make_golden.py diffusion3d_128 [more names ...]
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_workload  # noqa: E402

SAMPLES = 512
PROJECTIONS = 4
SAMPLE_SEED = 77


def sample_indices(m: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, m, SAMPLES)


def projection(v: np.ndarray, k: int, seed: int) -> float:
    w = np.random.default_rng(seed + 1000 * k).standard_normal(v.shape[0])
    return float(np.dot(w, v.astype(np.float64)))


def summarize(v: np.ndarray, seed: int) -> dict:
    v64 = v.astype(np.float64)
    idx = sample_indices(v.shape[0], seed)
    return {"norm": float(np.linalg.norm(v64)),
            "sample_seed": seed,
            "samples": [float(a) for a in v64[idx]],
            "projections": [projection(v64, k, seed) for k in range(PROJECTIONS)]}


def csr_of(w):
    if w.fmt == "csr":
        assert oracle.check_csr(w.n, w.row_ptr, w.cols) == oracle.OK
        return w.row_ptr.astype(np.int64), w.cols.astype(np.int64), w.vals
    ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
    return ref["row_ptr"], ref["col"], ref["vals"]


def list_members(w):
    """(row range, CSR, b, g) of each member of a list workload"""
    seg = w.extra["seg_rows"]
    out = []
    for q in range(len(seg) - 1):
        sel = (w.rows >= seg[q]) & (w.rows < seg[q + 1])
        ref = oracle.coo_to_csr(seg[q + 1] - seg[q], w.rows[sel] - seg[q], w.cols[sel] - seg[q],
                                w.vals[sel])
        out.append(((seg[q], seg[q + 1]), ref, w.b[seg[q]:seg[q + 1]], w.g[seg[q]:seg[q + 1]]))
    return out


def main_list(name):
    """A list of systems: every member solved alone (forward and adjoint)."""
    t0 = time.time()
    w = make_workload(name)
    rec = {"workload": name, "n": w.n, "nnz": int(w.nnz), "members": len(w.extra["seg_rows"]) - 1,
           "dtype": w.dtype, "tol": w.tol, "maxit": w.maxit,
           "written_by": "tests/golden/make_golden.py (CPU oracle)", "forward": [], "adjoint": []}
    for q, ((r0, r1), ref, b, g) in enumerate(list_members(w)):
        x, it, rel, oc = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], b, w.tol, w.maxit)
        d = {"rows": [int(r0), int(r1)], "iterations": int(it), "status": int(oc),
             "rel_residual": float(rel)}
        d.update(summarize(x, SAMPLE_SEED + q))
        rec["forward"].append(d)
        lam, gv, it2, rel2, oc2 = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], x, g, w.tol,
                                                 w.maxit)
        rec["adjoint"].append({"iterations": int(it2), "status": int(oc2), "rel_residual": float(rel2),
                               "nnz": int(ref["col"].shape[0]),
                               "lambda": summarize(lam, SAMPLE_SEED + 100 + q),
                               "grad_vals": summarize(gv, SAMPLE_SEED + 200 + q)})
        print(f"  member {q}: n={r1 - r0} iterations {it} / {it2} ({time.time() - t0:.0f} s)",
              flush=True)
    with open(os.path.join(HERE, f"{name}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def main(names):
    for name in names:
        t0 = time.time()
        if name.startswith("list_"):
            main_list(name)
            continue
        w = make_workload(name)
        rp, col, vals = csr_of(w)
        print(f"{name}: n={w.n} nnz={col.shape[0]} batch={w.batch} threads={oracle.num_threads()}",
              flush=True)
        x, it, rel, oc = oracle.pcg(rp, col, vals, w.b, w.tol, w.maxit)
        X = np.atleast_2d(x)
        rec = {"workload": name, "n": w.n, "nnz": int(col.shape[0]), "batch": w.batch,
               "dtype": w.dtype, "tol": w.tol, "maxit": w.maxit,
               "written_by": "tests/golden/make_golden.py (CPU oracle)",
               "forward": []}
        its, rels, ocs = np.atleast_1d(it), np.atleast_1d(rel), np.atleast_1d(oc)
        for s in range(w.batch):
            d = {"iterations": int(its[s]), "status": int(ocs[s]), "rel_residual": float(rels[s])}
            d.update(summarize(X[s], SAMPLE_SEED + s))
            rec["forward"].append(d)
        print(f"  forward: iterations {its.tolist()} ({time.time() - t0:.0f} s)", flush=True)
        if w.adjoint:
            lam, gv, it2, rel2, oc2 = oracle.adjoint(rp, col, vals, x, w.g, w.tol, w.maxit)
            L, GV = np.atleast_2d(lam), np.atleast_2d(gv)
            its2, rels2, ocs2 = np.atleast_1d(it2), np.atleast_1d(rel2), np.atleast_1d(oc2)
            rec["adjoint"] = []
            for s in range(w.batch):
                d = {"iterations": int(its2[s]), "status": int(ocs2[s]),
                     "rel_residual": float(rels2[s]),
                     "lambda": summarize(L[s], SAMPLE_SEED + 100 + s),
                     "grad_vals": summarize(GV[s], SAMPLE_SEED + 200 + s)}
                rec["adjoint"].append(d)
            print(f"  adjoint: iterations {its2.tolist()} ({time.time() - t0:.0f} s)", flush=True)
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])

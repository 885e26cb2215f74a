#!/usr/bin/env python3
"""Throughput of the differentiable Jacobi-PCG path on one MI355X.

A step is one pass of the whole hot path over the workload's matrix:
  sla_csr_set_values  (values in input order -> CSR values, Jacobi reciprocal)
  sla_pcg_solve       (Jacobi-PCG to the workload's tolerance / budget)
  sla_adjoint_backward(adjoint solve + value gradient), for workloads with one
The handle (pattern, tiles, workspace) is built once before timing, as the
pattern is shared by every step. Inputs are resident in HBM before timing.

value = PCG iterations (forward + adjoint) per second over the timed steps.

With no --workload, the run covers both points of the metric: the 2.1M-DOF
3D diffusion (the line's own figures) and then the 133M-DOF 2D Poisson share
(extra.dof_133m: 1 warm-up + 3 timed 500-iteration solves, its own roofline
and CPU baseline).

Printed as one JSON line. `roofline` covers the dominant kernel: its
algorithmic bytes per launch over its average launch duration, measured with
hipEvents on the stream it is launched on after the timed steps:
  - single system, per-step kernels: the SpMV tile kernel, 50 back-to-back
    sla_spmv launches between one event pair, the median of three such
    batches (the solve runs its fused form, which adds the p.q partials);
  - single system solved by the one-kernel path (the automatic choice
    wherever it applies, e.g. the default 2.1M-row workload): that kernel,
    one launch per solve, per-launch events (whole solves of milliseconds);
  - batch, or a matrix the library reordered for locality (sla_spmv then
    also transposes or permutes the vectors): the fused SpMV of the solve,
    per-launch events.
`traffic` is the HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
counters (profiles/), while the kernel source they were taken on is
unchanged. `cpu_baseline` times the CPU oracle on a bounded sample of the
same solve.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Jacobi-PCG iterations/sec and achieved HBM GB/s (% of peak) at 2M and 133M DOF"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "diffusion3d_128"
LARGE_WORKLOAD = "poisson2d_11548"
# sources of the kernel the roofline covers, per kernel tag (counter files are
# only used while these sources are unchanged)
KERNEL_SOURCES = {"spmv_dot": ["spmv.hip", "common.h"],
                  "cg_resident": ["resident.hip", "common.h"]}


def algorithmic_bytes(n, nnz, B, V, R):
    """Bytes one launch must move at minimum (each array touched once)."""
    spmv = V * nnz * B + 4 * nnz + R * (n + 1) + 2 * V * n * B   # vals, cols, row_ptr, p in, q out
    matrix = V * nnz * B + 4 * nnz + R * (n + 1)
    return {
        "spmv": spmv,
        "iter_3k": matrix + 13 * V * n * B,   # fused SpMV (2 vectors) + update (7) + direction (4)
        "iter_min": matrix + 7 * V * n * B,
        "grad": 4 * nnz + R * (n + 1) + V * nnz * B + 2 * V * n * B,
    }


def kernel_source_hash(tag: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[tag]:
        with open(os.path.join(ROOT, "differentiable_sparse_linear_csr_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, tag: str):
    """Per-launch HBM bytes of the roofline kernel from rocprofv3 counters, if
    they were taken on the current kernel source
    (profiles/<tag>_counters_<workload>.json), and where they come from."""
    rel = f"profiles/{tag}_counters_{workload}.json"
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(tag):
        return None, f"{rel} was taken on another kernel source: not used"
    return rec.get("hbm_bytes_per_launch"), (
        f"{rel}: rocprofv3 FETCH_SIZE + WRITE_SIZE per launch of this kernel in a separate run "
        f"of the same command, each scaled by the counter's reading for a 1 GiB device copy "
        f"(fetch x{rec['calibration']['fetch_factor']:.2f}, write "
        f"x{rec['calibration']['write_factor']:.2f}); not measured in this run")


def host_info() -> dict:
    """CPU model, NUMA nodes and the CPUs this process may run on."""
    import glob
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    numa = len(glob.glob("/sys/devices/system/node/node[0-9]*")) or None
    return {"cpu_model": model, "numa_nodes": numa, "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(w, budget_s: float, budget_1t_s: float = 0.0):
    """The oracle as it stands, on the host cores: iterations/s of the forward
    solve (Jacobi-PCG, or Jacobi-BiCGStab for a non-symmetric workload) on the
    same matrix and right-hand side, over a bounded number of iterations (the
    first ones of the same solve), with all threads and (budget_1t_s > 0)
    with one thread. For a workload whose step also runs the adjoint, the
    oracle's adjoint (the transposed solve, tol 0, for a bounded number of
    iterations, then the value gradient) is timed the same way after the
    forward sample, and value is forward + adjoint iterations over their
    summed time, as the GPU's value counts them."""
    import numpy as np
    import oracle

    threads = oracle.num_threads()
    bicg = w.extra.get("method") == "bicgstab"
    solve = oracle.bicgstab if bicg else oracle.pcg
    adjoint = oracle.bicgstab_adjoint if bicg else oracle.adjoint
    if "seg_rows" in w.extra:
        # every member is its own system: the oracle solves them one by one,
        # each for the same bounded number of iterations
        seg = w.extra["seg_rows"]
        members = []
        for q in range(len(seg) - 1):
            sel = (w.rows >= seg[q]) & (w.rows < seg[q + 1])
            ref = oracle.coo_to_csr(seg[q + 1] - seg[q], w.rows[sel] - seg[q], w.cols[sel] - seg[q],
                                    w.vals[sel])
            members.append((ref, ref["vals"], w.b[seg[q]:seg[q + 1]],
                            w.g[seg[q]:seg[q + 1]] if w.g is not None else None))
        what = f"iterations (tol 0) of each of the {len(members)} members of {w.name}, " \
               f"solved one by one"
        probe_iters = 2
    else:
        if w.fmt == "csr":
            ref = {"row_ptr": w.row_ptr.astype(np.int64), "col": w.cols.astype(np.int64)}
            vals = w.vals
        else:
            ref = oracle.coo_to_csr(w.n, w.rows, w.cols, w.vals)
            vals = ref["vals"]
        members = [(ref, vals, w.b, w.g)]
        what = f"iterations (tol 0) of {w.name} ({w.batch} system(s)), oracle CSR built from " \
               f"the same input"
        probe_iters = 5 if w.n * w.batch < (1 << 24) else 1
    xs = [None] * len(members)

    def run(iters):
        total = 0
        for q, (ref, vals, bq, _) in enumerate(members):
            xs[q], it, _, _ = solve(ref["row_ptr"], ref["col"], vals, bq, 0.0, iters)
            total += int(np.sum(it))
        return total

    def run_adj(iters):
        total = 0
        for q, (ref, vals, _, gq) in enumerate(members):
            _, _, it, _, _ = adjoint(ref["row_ptr"], ref["col"], vals, xs[q], gq, 0.0, iters)
            total += int(np.sum(it))
        return total

    def timed(fn, budget, probe):
        t0 = time.perf_counter()
        fn(probe)
        per = (time.perf_counter() - t0) / probe
        iters = int(max(1, min(w.maxit, budget / max(per, 1e-9))))
        t0 = time.perf_counter()
        it = fn(iters)
        dt = time.perf_counter() - t0
        return it, iters, dt

    name = "Jacobi-BiCGStab" if bicg else "Jacobi-PCG"
    with_adj = bool(w.adjoint) and w.g is not None
    it_f, iters_f, dt_f = timed(run, budget_s / 2 if with_adj else budget_s, probe_iters)
    out = {"value": round(it_f / dt_f, 3), "unit": "iterations/s", "cores": threads,
           "kind": "oracle",
           "sample": f"first {iters_f} {name} {what}; {dt_f:.1f} s on {threads} threads"}
    if with_adj:
        it_a, iters_a, dt_a = timed(run_adj, budget_s / 2, probe_iters)
        out["forward_value"] = out["value"]
        out["adjoint_value"] = round(it_a / dt_a, 3)
        out["value"] = round((it_f + it_a) / (dt_f + dt_a), 3)
        out["sample"] = (f"first {iters_f} forward {name} {what} ({dt_f:.1f} s), then the "
                         f"adjoint from the forward iterate: first {iters_a} transposed "
                         f"iterations and the value gradient ({dt_a:.1f} s); value = forward + "
                         f"adjoint iterations over both times, on {threads} threads")
    if budget_1t_s > 0:
        oracle.set_num_threads(1)
        try:
            it1, iters1, dt1 = timed(run, budget_1t_s, 1)
        finally:
            oracle.set_num_threads(threads)
        out["value_1_thread"] = round(it1 / dt1, 3)
        out["sample_1_thread"] = f"first {iters1} iterations of the same forward solve; {dt1:.1f} s"
    out.update(host_info())
    return out


def run_inverse(args, N: int = 128, S: int = 4) -> int:
    """The inverse-conductivity demonstration as a workload: a step is one Adam
    step (assembly of A(kappa), batched PCG of the S experiments, batched
    adjoint, chain to kappa, update). warmup + steps Adam steps run on one
    trajectory (cosine decay over all of them); value counts the PCG
    iterations (forward + adjoint, summed over experiments) of the timed steps."""
    import numpy as np
    import torch
    from differentiable_sparse_linear_csr_amd import _lib
    from differentiable_sparse_linear_csr_amd.inverse import ConductivityRecovery

    total = args.warmup + args.steps
    t_gen = time.perf_counter()
    rec = ConductivityRecovery(N, sources=S, total_steps=total, device="cuda:0")
    A = rec.A
    A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, args.check_interval)
    if args.ordinary_launch:
        A.set_option(_lib.SLA_OPT_COOPERATIVE, 0)
    print(f"[bench] inverse conductivity {N}x{N}, {S} experiments, {total} Adam steps "
          f"(set up in {time.perf_counter() - t_gen:.1f} s)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        rec.step()
    torch.cuda.synchronize()
    it0 = rec.iterations
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rec.step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    value = (rec.iterations - it0) / elapsed
    rep = rec.report()
    # profiled SpMV launches of one more solve (after the trajectory)
    A.profile_reset()
    A.set_option(_lib.SLA_OPT_PROFILE, 1)
    with torch.no_grad():
        _, pinfo = A.solve_raw(rec.F, rec.tol, rec.maxit)
    prof = A.profile()
    A.set_option(_lib.SLA_OPT_PROFILE, 0)
    n, nnz = rec.grid.n, A.nnz
    V, R = 8, (8 if A.row_index_dtype == torch.int64 else 4)
    ab = algorithmic_bytes(n, nnz, S, V, R)
    if prof["cg_resident"][0] > 0:
        # the batch as S groups of the single-kernel solve: per system
        # iteration its matrix, the p gathers and the p store; b, dinv read
        # and x written once per system
        launches, total_ms = prof["cg_resident"]
        avg_ms = total_ms / launches
        one = algorithmic_bytes(n, nnz, 1, V, R)["spmv"]
        bytes_launch = sum(pinfo.iterations) * one / launches + 3 * V * n * S
        kernel = "k_cg_resident (whole batched solve per launch; per-launch events)"
    else:
        launches, total_ms = prof["spmv_dot"]
        avg_ms = total_ms / max(launches, 1)
        bytes_launch = ab["spmv"]
        kernel = "k_spmv_bvec (fused q = A p, p.q partials, alpha; per-launch events)"
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "iterations/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / max(args.steps, 1) * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"inverse_conductivity_{N}",
                   "description": f"Adam recovery of kappa in -div(kappa grad u) = f_s, {N}x{N} "
                                  f"grid, {S} Gaussian sources solved as one batch",
                   "n": n, "nnz": nnz, "batch": S, "tol": rec.tol, "maxit": rec.maxit,
                   "step": "assemble A(kappa) + pcg_solve (batch) + adjoint_backward + Adam",
                   "adam_steps_total": total, "check_interval": args.check_interval},
        "roofline": {"kernel": kernel,
                     "bound": "hbm", "achieved": round(bytes_launch / (avg_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(bytes_launch / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": round(bytes_launch),
                     "avg_launch_ms": round(avg_ms, 5), "launches_timed": launches},
        "extra": {"recovery": rep,
                  "pages_figure": "1500 Adam steps, kappa error 2.3e-3, misfit 3.0e-5, "
                                  "32 ms/step on RTX PRO 6000 (grid not stated)",
                  "kernel_avg_ms": {k: round(v[1] / max(v[0], 1), 5) for k, v in prof.items()
                                    if v[0]}},
    }
    if not args.no_cpu_baseline:
        # the oracle's batched PCG on the same systems (true kappa, the S sources)
        class W:
            pass
        w = W()
        g = rec.grid
        w.name, w.n, w.batch, w.fmt, w.maxit, w.extra = f"inverse_conductivity_{N}", n, S, "coo", \
            rec.maxit, {}
        w.rows, w.cols = g.rows.cpu().numpy(), g.cols.cpu().numpy()
        w.vals = np.ascontiguousarray(
            g.values(rec.kappa_true).expand(S, -1).detach().cpu().numpy())
        w.b = rec.F.cpu().numpy()
        # the step's adjoint too: tol-0 iterations cost the same whatever the
        # upstream gradient, so a seeded normal one stands in for the misfit's
        w.adjoint = True
        w.g = np.random.default_rng(7).standard_normal(w.b.shape).astype(w.b.dtype)
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def measure(args, name: str, steps: int, warmup: int, cpu_budget: float,
            cpu_1t_budget: float) -> dict:
    """One workload: handle built once, `warmup` untimed and `steps` timed
    steps, the roofline kernel's launches timed on its stream, and the CPU
    oracle's rate (cpu_budget seconds of work with all threads, cpu_1t_budget
    with one; 0 skips it). Returns the JSON record."""
    import numpy as np
    import torch
    import differentiable_sparse_linear_csr_amd as sla
    from differentiable_sparse_linear_csr_amd import _lib
    from workloads import make_workload

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    w = make_workload(name)
    print(f"[bench] workload {w.name}: n={w.n} nnz={w.nnz} batch={w.batch} dtype={w.dtype} "
          f"(generated in {time.perf_counter() - t_gen:.1f} s)", file=sys.stderr, flush=True)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    cols = d(w.cols)
    vals = d(w.vals)
    b = d(w.b)
    g = d(w.g) if w.adjoint else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if "seg_rows" in w.extra:
        A = sla.SparseTensorList.from_block_diagonal_coo(d(w.rows), cols, vals, w.extra["seg_rows"])
    elif w.fmt == "coo":
        A = sla.SparseCSR.from_coo(d(w.rows), cols, vals, w.n)
    else:
        A = sla.SparseCSR.from_csr(d(w.row_ptr), cols, vals)
    torch.cuda.synchronize()
    create_ms = (time.perf_counter() - t0) * 1e3
    layout = A.layout()
    A.set_option(_lib.SLA_OPT_CHECK_INTERVAL, args.check_interval)
    if args.ordinary_launch:
        A.set_option(_lib.SLA_OPT_COOPERATIVE, 0)
    x = torch.empty_like(b)

    method = w.extra.get("method", "cg")

    # how each solve ran (single kernel or per-step, and whether it fell
    # back), counted over the timed steps
    path_counts = {}
    counting = [False]

    def note_path():
        if not counting[0] or not hasattr(A, "last_path"):
            return
        lp = A.last_path()
        key = lp["path"] + ("+cooperative_refused" if lp["cooperative_refused"] else "") + \
            ("+wait_timed_out" if lp["wait_timed_out"] else "")
        path_counts[key] = path_counts.get(key, 0) + 1

    def step():
        A.set_values(vals)
        _, info = A.solve_raw(b, w.tol, w.maxit, out=x, method=method)
        note_path()
        its = list(info.iterations)
        if w.adjoint:
            _, _, ainfo = A.adjoint_raw(x, g, w.tol, w.maxit, method=method)
            note_path()
            its = [i + j for i, j in zip(its, ainfo.iterations)]
        return its, info

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    counting[0] = True
    t0 = time.perf_counter()
    total_its = 0
    for _ in range(steps):
        its, info = step()
        total_its += sum(its)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    counting[0] = False
    value = total_its / elapsed
    ms_per_step = elapsed / steps * 1e3
    fwd_its = info.iterations

    # profiled step: hipEvents around every kernel launch, on the launch stream
    A.profile_reset()
    A.set_option(_lib.SLA_OPT_PROFILE, 1)
    prof_its = sum(step()[0])
    prof = A.profile()
    A.set_option(_lib.SLA_OPT_PROFILE, 0)
    # the same SpMV kernel launched back to back, one event pair around all of
    # them on the launch stream: its average duration without per-launch
    # event overhead (the figure rocprofv3's kernel trace reports)
    stream = torch.cuda.current_stream()
    y = A.matvec(b)
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    batches = []
    for _ in range(3):   # the median of three batches (a batch now and then runs slow)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            A.matvec(b)
        e1.record(stream)
        torch.cuda.synchronize()
        batches.append(e0.elapsed_time(e1) / reps)
    b2b_ms = sorted(batches)[1]
    # the matvec backward (A^T g and the value gradient), timed the same way;
    # the first call builds A^T's pattern (a device sort), outside the timed
    # region
    gy = torch.ones_like(b)
    t_tr = time.perf_counter()
    A.matvec_backward_raw(b, gy)
    torch.cuda.synchronize()
    transpose_build_ms = (time.perf_counter() - t_tr) * 1e3
    e0.record(stream)
    for _ in range(10):
        A.matvec_backward_raw(b, gy)
    e1.record(stream)
    torch.cuda.synchronize()
    bwd_ms = e0.elapsed_time(e1) / 10

    V = 8 if w.dtype == "f64" else 4
    R = 8 if A.row_index_dtype == torch.int64 else 4
    ab = algorithmic_bytes(w.n, w.nnz, w.batch, V, R)
    # whole-job bytes per second of the iterations the steps performed: a
    # list's member iteration moves that member's bytes only
    if method == "bicgstab":
        # two SpMVs (matrix twice, one gather and one store each, the fused
        # dot partner read) and 25 vector passes in the five kernels (dir 6,
        # SpMVs 3 + 3, half 5, update 8)
        mat = ab["iter_3k"] - 13 * V * w.n * w.batch
        bicg_iter = 2 * mat + 25 * V * w.n * w.batch
        job_bps = {"iter_3k": bicg_iter / w.batch * value, "iter_min": bicg_iter / w.batch * value}
    elif "seg_rows" in w.extra:
        seg = w.extra["seg_rows"]
        seg_nnz = np.bincount(np.searchsorted(seg, w.rows, side="right") - 1,
                              minlength=len(seg) - 1)
        per_step = {k: sum(i * algorithmic_bytes(seg[q + 1] - seg[q], int(seg_nnz[q]), 1, V, R)[k]
                           for q, i in enumerate(its)) for k in ("iter_3k", "iter_min")}
        job_bps = {k: v * steps / elapsed for k, v in per_step.items()}
    else:
        # value counts system-iterations; one batched iteration moves ab[k]
        # for all B systems
        job_bps = {k: ab[k] / w.batch * value for k in ("iter_3k", "iter_min")}
    res_launches, res_ms = prof["cg_resident"]
    ndiag = A.diagonals()
    sdiag = A.step_diagonals()
    layout["diagonals"] = ndiag
    layout["step_diagonals"] = sdiag
    # what the single-kernel solve reads per iteration: the matrix as held
    # (by diagonals: their values, no column indices) and p gathered and stored
    moved_iter = (ndiag * w.n * V + 2 * V * w.n) if ndiag > 0 else ab["spmv"] / w.batch
    if res_launches > 0:
        # whole solves in one cooperative kernel: per iteration the matrix, the
        # p gathers and the p store (x, r, p, dinv stay on chip); plus b and
        # dinv read and x written once per solve
        launches, total_ms = res_launches, res_ms
        avg_ms = total_ms / launches
        bytes_launch = prof_its / launches * ab["spmv"] + 3 * V * w.n * w.batch
        moved_launch = prof_its / launches * moved_iter * w.batch + 3 * V * w.n * w.batch
        per_iter_ms = total_ms / max(prof_its, 1)
        kernel = "k_cg_resident (whole solve per launch: SpMV, p.q, update, r.z/r.r, direction)"
    elif w.batch == 1 and not layout["reordered"]:
        # the SpMV tile kernel (the solve runs its fused form, which adds the
        # p.q partials): back-to-back launches of sla_spmv
        launches, avg_ms = reps, b2b_ms
        bytes_launch = ab["spmv"]
        # iterations: one direction-kernel launch each (two SpMVs in BiCGStab)
        n_it = max(prof["direction"][0] if method == "bicgstab" else prof["spmv_dot"][0], 1)
        per_iter_ms = sum(prof[k][1] for k in ("spmv_dot", "update", "direction")) / n_it
        kernel = ((f"k_spmv_dia (the matrix held by {sdiag} diagonals)" if sdiag > 0 else
                   "k_spmv_tile_ring" if layout.get("ring_tiles") else "k_spmv_tile")
                  + " (q = A p; 50 back-to-back sla_spmv launches, median of 3 batches)")
        if sdiag > 0:
            moved_launch = sdiag * w.n * V + 2 * V * w.n
    else:
        # batched, or reordered: sla_spmv also transposes or permutes x and y,
        # so the fused SpMV of the solve is timed per launch (events around
        # each launch)
        launches, total_ms = prof["spmv_dot"]
        avg_ms = total_ms / max(launches, 1)
        bytes_launch = ab["spmv"]
        per_iter_ms = sum(prof[k][1] for k in ("spmv_dot", "update", "direction")) / max(launches, 1)
        kernel = ("k_spmv_bvec (fused q = A p, p.q partials, alpha; per-launch events)" if w.batch > 1
                  else "k_spmv_tile on P A P^T (fused q = A p, p.q partials; per-launch events)")
    achieved = bytes_launch / (avg_ms * 1e-3) / 1e9
    traffic, traffic_src = load_traffic(w.name, "cg_resident" if res_launches > 0 else "spmv_dot")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "iterations/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "n": w.n, "nnz": w.nnz, "batch": w.batch,
            "row_ptr": "int64" if R == 8 else "int32", "col_idx": "int32",
            "tol": w.tol, "maxit": w.maxit,
            "step": ("set_values + bicgstab_solve" + (" + bicgstab_adjoint" if w.adjoint else "")
                     if method == "bicgstab" else
                     "set_values + pcg_solve" + (" + adjoint_backward" if w.adjoint else "")),
            "forward_iterations": fwd_its,
            "check_interval": args.check_interval,
        },
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "algorithmic_bytes_per_launch": round(bytes_launch),
            "avg_launch_ms": round(avg_ms, 5),
            "launches_timed": launches,
        },
        "extra": {
            "create_ms": round(create_ms, 2),
            # whole-job figures: every second of the timed steps counted
            "iteration_ms": round(1e3 / value, 5),
            "iteration_model": ("BiCGStab: 2 matrix reads + 25 vector passes per iteration"
                                if method == "bicgstab" else
                                ("PCG in one kernel: the matrix"
                                 + (f" (held by {ndiag} diagonals: their values, no column "
                                    f"indices)" if ndiag > 0 else "")
                                 + ", p gathered and p stored per iteration (x, r, p, dinv stay "
                                 "on chip) = 'moved'; 3k/min: what the per-step kernels would "
                                 "move for the same iterations")
                                if res_launches > 0 else
                                "PCG: matrix + 13 vector passes (3k) / + 7 (min) per iteration"),
            "iteration_gbps_3k": round(job_bps["iter_3k"] / 1e9, 1),
            "iteration_frac_3k": round(job_bps["iter_3k"] / 1e9 / HBM_PEAK_GBS, 4),
            "iteration_gbps_min": round(job_bps["iter_min"] / 1e9, 1),
            **({"iteration_gbps_moved": round(moved_iter * value / 1e9, 1),
                "iteration_frac_moved": round(moved_iter * value / 1e9 / HBM_PEAK_GBS, 4)}
               if res_launches > 0 else {}),
            # the kernels of one iteration alone (per-launch events, which add
            # a few microseconds of event overhead per launch)
            "iteration_kernels_ms": round(per_iter_ms, 5),
            "path": "single cooperative kernel" if res_launches > 0 else "per-step kernels",
            # solves (forward and adjoint) of the timed steps by the path they took
            "solve_paths": path_counts or None,
            "spmv_ms": round(b2b_ms, 5),
            "spmv_gflops": round(2 * w.nnz * w.batch / (b2b_ms * 1e-3) / 1e9, 1),
            "spmv_gbps": round(ab["spmv"] / (b2b_ms * 1e-3) / 1e9, 1),
            # matvec backward: A^T g (SpMV bytes) + grad_vals (gradient bytes)
            "spmv_backward_first_call_ms": round(transpose_build_ms, 1),
            "spmv_backward_ms": round(bwd_ms, 5) if bwd_ms else None,
            "spmv_backward_gbps": (round((ab["spmv"] + ab["grad"]) / (bwd_ms * 1e-3) / 1e9, 1)
                                   if bwd_ms else None),
            "kernel_avg_ms": {k: round(v[1] / max(v[0], 1), 5) for k, v in prof.items() if v[0]},
            "handle_bytes": A.memory_bytes(),
            "layout": layout,
        },
    }
    if (res_launches > 0 and ndiag > 0) or (res_launches == 0 and sdiag > 0
                                             and w.batch == 1 and not layout["reordered"]):
        out["roofline"]["bytes_moved_per_launch"] = round(moved_launch)
        out["roofline"]["frac_on_moved"] = round(
            moved_launch / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        out["roofline"]["held_by_diagonals"] = (
            f"the kernel holds the matrix by {max(ndiag, sdiag)} diagonals and reads no column "
            f"indices: "
            f"'achieved' counts the CSR algorithmic bytes (values, column indices, row "
            f"pointers, p in and q out per iteration), bytes_moved_per_launch what it reads "
            f"and writes")
    matrix_mb = (ab["spmv"] - 2 * V * w.n * w.batch) / 1e6
    if matrix_mb < 256.0:
        out["roofline"]["note"] = (
            f"the matrix ({matrix_mb:.0f} MB as counted here) fits the 256 MB Infinity Cache, "
            f"which can serve it from one iteration to the next: 'achieved' and 'traffic' count "
            f"bytes the L2 reads from the Infinity Cache or HBM"
            + ("; extra.dof_133m is the point whose matrix cannot stay there"
               if name == DEFAULT_WORKLOAD else ""))
    if cpu_budget > 0:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, cpu_budget, cpu_1t_budget)
    else:
        out["cpu_baseline"] = None
    del A, cols, vals, b, g, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help=f"one workload only (default: {DEFAULT_WORKLOAD}, then {LARGE_WORKLOAD} "
                         f"as extra.dof_133m)")
    ap.add_argument("--check-interval", type=int, default=16)
    ap.add_argument("--ordinary-launch", action="store_true",
                    help="start the single-kernel solve with an ordinary launch instead of "
                         "a cooperative one (for profilers that cannot follow cooperative "
                         "launches); same kernel, same grid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--cpu-budget-1t", type=float, default=5.0,
                    help="seconds of oracle work on one thread")
    ap.add_argument("--large-steps", type=int, default=3,
                    help=f"timed steps of {LARGE_WORKLOAD} in the default run")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the measurement, copy a buffer of this size 3 times with a plain "
                         "device copy kernel (reference for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library's path runs on a single MI355X "
              "(sharding across GPUs is designed, not built). Use --gpus 1.",
              file=sys.stderr)
        return 2

    if args.workload == "inverse_conductivity_128":
        return run_inverse(args)

    import torch

    cpu = 0.0 if args.no_cpu_baseline else args.cpu_budget
    cpu1 = 0.0 if args.no_cpu_baseline else args.cpu_budget_1t
    if args.workload is not None:
        out = measure(args, args.workload, args.steps, args.warmup, cpu, cpu1)
    else:
        out = measure(args, DEFAULT_WORKLOAD, args.steps, args.warmup, cpu, cpu1)
        # the metric's second point: one GPU's share of the 400M-DOF solve
        big = measure(args, LARGE_WORKLOAD, args.large_steps, 1, 0.0 if cpu == 0 else 10.0,
                      0.0 if cpu1 == 0 else 8.0)
        out["extra"]["dof_133m"] = {
            "workload": big["config"]["workload"], "n": big["config"]["n"],
            "nnz": big["config"]["nnz"], "value": big["value"], "unit": big["unit"],
            "steps": big["steps"], "warmup": big["warmup"], "ms_per_step": big["ms_per_step"],
            "step": big["config"]["step"], "tol": big["config"]["tol"],
            "maxit": big["config"]["maxit"], "roofline": big["roofline"],
            **{k: big["extra"][k] for k in ("path", "solve_paths", "iteration_ms", "iteration_gbps_3k",
                                            "iteration_frac_3k", "iteration_kernels_ms",
                                            "spmv_ms", "spmv_gbps", "spmv_backward_first_call_ms",
                                            "spmv_backward_ms", "spmv_backward_gbps",
                                            "kernel_avg_ms")},
            "cpu_baseline": big["cpu_baseline"]}
    print(json.dumps(out), flush=True)
    if args.calibrate_copy_mib > 0:
        src = torch.ones(args.calibrate_copy_mib << 17, dtype=torch.float64, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration: copied {args.calibrate_copy_mib} MiB x3", file=sys.stderr)
    return 0



if __name__ == "__main__":
    sys.exit(main())

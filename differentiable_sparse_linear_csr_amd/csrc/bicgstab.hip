// Jacobi-preconditioned BiCGStab for one general (non-symmetric) system, and
// the host driver that replays blocks of its iterations as hipGraphs.
//
// torch-sla's pytorch-native backend offers BiCGStab next to CG (backend
// list of the API section); its distributed section says BiCGStab follows the
// CG template with more inner products. The pages print no recurrence; this
// is van der Vorst's preconditioned BiCGStab with M = diag(A) on the right,
// x0 = 0 and shadow residual r^ = b:
//   p = r (first) or r + beta (p - omega v);  p^ = M^-1 p;  v = A p^
//   alpha = rho / r^.v;  s = r - alpha v       (half step: ||s|| <= tol ||b||)
//   s^ = M^-1 s;  t = A s^;  omega = t.s / t.t
//   x += alpha p^ + omega s^;  r = s - omega t;  rho' = r^.r;
//   beta = (rho'/rho)(alpha/omega)
// Breakdown is an exact zero (or a non-finite value) of r^.v, t.t, omega or
// rho'; one at omega keeps the half step as the iterate.
//
// One iteration is five kernels, all on one system:
//   dir     p and p^ = dinv p                          (reads r, p, v, dinv)
//   SpMV    v = A p^ with the r^.v partials fused       (gathers p^, reads r^)
//   half    alpha; s = r - alpha v written over r, s^ = dinv s, ||s||^2; the
//           last workgroup takes the half-step test
//   SpMV    t = A s^ with t.s and t.t partials fused    (gathers s^, reads s)
//   update  omega; x and r; r^.r and r.r; the last workgroup takes the stopping
//           test, the budget and beta
// Every workgroup that needs a step size sums the previous kernel's
// per-workgroup partials itself, in the same fixed order, so the scalars are
// identical everywhere and no kernel ends with a grid-wide wait. The status
// lives on the device; finished solves make every kernel a no-op, so the host
// polls every k iterations without changing the iterate or the count.
#include "common.h"

namespace sla {

void launch_spmv_dots(Handle &h, const void *x, void *y, const void *w, int ndot, double *spart,
                      const int32_t *status, hipStream_t s);
int64_t spmv_grid(const Handle &h);

namespace {

constexpr int kBiGroups = 2;  // 16-byte groups per lane and pass

// Scalars of the solve (one system)
struct BiState {
    double bb;      // ||b||^2
    double rho;     // r^.r of the current residual
    double alpha, omega, beta;
    double rr;      // ||r||^2 of the last residual formed
    double ss;      // ||s||^2 of the current half step
    int32_t iter;   // iterations started
    int32_t status; // kRunning or an sla_outcome
    int32_t half;   // 1: the update kernel still has to apply the final half step
    int32_t pad;
};

int64_t bi_grid(int64_t n, int W) {
    const int64_t per = (int64_t)kBlock * kBiGroups * W;
    int64_t g = (n + per - 1) / per;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g < 1) g = 1;
    return g;
}

// sum over j < m of part[j * C + c], in an order that depends only on m
// (identical in every workgroup); result in every thread
__device__ __forceinline__ double sum_parts(const double *__restrict__ part, int64_t m, int C,
                                            int c, double *lds4) {
    double a = 0.0;
    for (int64_t j = threadIdx.x; j < m; j += 4 * kBlock) {
        double v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t jj = j + (int64_t)u * kBlock;
            v4[u] = jj < m ? part[jj * C + c] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) a += v4[u];
    }
    return block_sum(a, lds4);
}

// x = 0, r = r^ = b; ||b||^2; the last workgroup sets up the scalars
template <typename T>
__global__ __launch_bounds__(kBlock) void k_bi_init(int64_t n, const T *__restrict__ b,
                                                    T *__restrict__ x, T *__restrict__ r,
                                                    T *__restrict__ rh, Red red,
                                                    Ctl *__restrict__ ctl,
                                                    BiState *__restrict__ st,
                                                    int32_t *__restrict__ h_running) {
    __shared__ double lds4[kWaves];
    __shared__ double tmp[kBlock];
    __shared__ double tot[1];
    double sbb = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const T bv = b[i];
        x[i] = (T)0;
        r[i] = bv;
        rh[i] = bv;
        sbb += (double)bv * (double)bv;
    }
    sbb = block_sum(sbb, lds4);
    if (threadIdx.x == 0) store_partial(red.part + blockIdx.x, sbb);
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 1, tmp, tot) &&
        threadIdx.x == 0) {
        BiState s{};
        s.bb = tot[0];
        s.rho = tot[0];
        s.rr = tot[0];
        if (s.bb == 0.0) s.status = SLA_CONVERGED;
        else if (ctl->maxit <= 0) s.status = SLA_MAXIT;
        else s.status = kRunning;
        *st = s;
        publish_running(ctl, h_running, s.status == kRunning ? 1 : 0);
    }
}

// p = r (first iteration) or r + beta (p - omega v); p^ = dinv p
template <typename T>
__global__ __launch_bounds__(kBlock) void k_bi_dir(int64_t n, const T *__restrict__ r,
                                                   T *__restrict__ p, T *__restrict__ ph,
                                                   const T *__restrict__ v,
                                                   const T *__restrict__ dinv,
                                                   const BiState *__restrict__ st) {
    constexpr int W = VecW<T>::W;
    if (st->status != kRunning) return;
    const bool first = st->iter == 0;
    const double beta = st->beta, omega = st->omega;
    auto row = [&](T rv, T &pv, T vv, T dv, T &phv) {
        pv = first ? rv : (T)((double)rv + beta * ((double)pv - omega * (double)vv));
        phv = (T)((double)dv * (double)pv);
    };
    const int tid = threadIdx.x;
    const int64_t ng = n / W;
    const int64_t per_pass = (int64_t)kBlock * kBiGroups;
    for (int64_t g0 = (int64_t)blockIdx.x * per_pass; g0 < ng; g0 += (int64_t)gridDim.x * per_pass) {
        T rv[kBiGroups][W], pv[kBiGroups][W], vv[kBiGroups][W], dv[kBiGroups][W],
            hv[kBiGroups][W];
#pragma unroll
        for (int u = 0; u < kBiGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
                vload(r + g * W, rv[u]);
                vload(dinv + g * W, dv[u]);
                if (!first) {
                    vload(p + g * W, pv[u]);
                    vload(v + g * W, vv[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kBiGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
#pragma unroll
                for (int k = 0; k < W; ++k) row(rv[u][k], pv[u][k], vv[u][k], dv[u][k], hv[u][k]);
                vstore(p + g * W, pv[u]);
                vstore(ph + g * W, hv[u]);
            }
        }
    }
    if (blockIdx.x == 0 && tid < n - ng * W) {
        const int64_t i = ng * W + tid;
        T pi = first ? (T)0 : p[i], vi = first ? (T)0 : v[i], hi;
        row(r[i], pi, vi, dinv[i], hi);
        p[i] = pi;
        ph[i] = hi;
    }
}

// alpha = rho / r^.v (from the SpMV's partials); s = r - alpha v over r,
// s^ = dinv s, partials of ||s||^2; the last workgroup counts the iteration
// and takes the half-step test
template <typename T>
__global__ __launch_bounds__(kBlock) void k_bi_half(int64_t n, T *__restrict__ r,
                                                    const T *__restrict__ v,
                                                    const T *__restrict__ dinv,
                                                    T *__restrict__ sh,
                                                    const double *__restrict__ spart,
                                                    int64_t spart_n, Red red,
                                                    Ctl *__restrict__ ctl,
                                                    BiState *__restrict__ st,
                                                    int32_t *__restrict__ h_running) {
    constexpr int W = VecW<T>::W;
    __shared__ double lds4[kWaves];
    __shared__ double tmp[kBlock];
    __shared__ double tot[1];
    if (st->status != kRunning) return;
    const int tid = threadIdx.x;
    const int64_t ngl = n / W;
    const int64_t per_pass = (int64_t)kBlock * kBiGroups;
    T rv[kBiGroups][W], vv[kBiGroups][W], dv[kBiGroups][W], hv[kBiGroups][W];
    auto load = [&](int64_t g0) {
#pragma unroll
        for (int u = 0; u < kBiGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ngl) {
                vload(r + g * W, rv[u]);
                vload(v + g * W, vv[u]);
                vload(dinv + g * W, dv[u]);
            }
        }
    };
    // the first pass's rows are loaded before the SpMV's partials are read,
    // so the two latencies overlap
    int64_t g0 = (int64_t)blockIdx.x * per_pass;
    load(g0);
    const double sigma = sum_parts(spart, spart_n, 1, 0, lds4);
    const bool bad = sigma == 0.0 || !isfinite(sigma);
    const double alpha = bad ? 0.0 : st->rho / sigma;
    double sss = 0.0;
    auto row = [&](T &rv, T vv, T dv, T &shv) {
        rv = (T)((double)rv - alpha * (double)vv);
        shv = (T)((double)dv * (double)rv);
        sss += (double)rv * (double)rv;
    };
    const int64_t ng = bad ? 0 : ngl;   // breakdown: r stays as it is
    for (; g0 < ng; g0 += (int64_t)gridDim.x * per_pass) {
#pragma unroll
        for (int u = 0; u < kBiGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
#pragma unroll
                for (int k = 0; k < W; ++k) row(rv[u][k], vv[u][k], dv[u][k], hv[u][k]);
                vstore(r + g * W, rv[u]);
                vstore(sh + g * W, hv[u]);
            }
        }
        if (g0 + (int64_t)gridDim.x * per_pass < ng) load(g0 + (int64_t)gridDim.x * per_pass);
    }
    if (!bad && blockIdx.x == 0 && tid < n - (n / W) * W) {
        const int64_t i = (n / W) * W + tid;
        T ri = r[i], hi;
        row(ri, v[i], dinv[i], hi);
        r[i] = ri;
        sh[i] = hi;
    }
    sss = block_sum(sss, lds4);
    if (tid == 0) store_partial(red.part + blockIdx.x, sss);
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 1, tmp, tot) && tid == 0) {
        BiState &s = *st;
        s.iter += 1;
        if (bad) {
            s.status = SLA_BREAKDOWN;            // x and r untouched
            publish_running(ctl, h_running, 0);
            return;
        }
        const double ss = tot[0];
        s.alpha = alpha;
        s.ss = ss;
        if (!isfinite(ss)) {
            s.status = SLA_BREAKDOWN;            // x untouched
            publish_running(ctl, h_running, 0);
        } else if (sqrt(ss) <= ctl->tol * sqrt(s.bb)) {
            s.status = SLA_CONVERGED;            // the update kernel adds alpha p^ to x
            s.half = 1;
            s.rr = ss;
            publish_running(ctl, h_running, 0);
        }
    }
}

// omega = t.s / t.t (from the SpMV's partials); x += alpha p^ + omega s^,
// r = s - omega t (s is in r); partials of r^.r and r.r. After a half step
// that ends the solve (converged, or a breakdown at omega) only x += alpha p^.
// The last workgroup takes the stopping test, the budget and beta.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_bi_update(int64_t n, T *__restrict__ x,
                                                      T *__restrict__ r,
                                                      const T *__restrict__ rh,
                                                      const T *__restrict__ ph,
                                                      const T *__restrict__ sh,
                                                      const T *__restrict__ t,
                                                      const double *__restrict__ spart,
                                                      int64_t spart_n, Red red,
                                                      Ctl *__restrict__ ctl,
                                                      BiState *__restrict__ st,
                                                      int32_t *__restrict__ h_running) {
    constexpr int W = VecW<T>::W;
    __shared__ double lds4[kWaves];
    __shared__ double tmp[kBlock];
    __shared__ double tot[2];
    if (st->status != kRunning && st->half == 0) return;
    const bool half = st->half != 0;
    const int tid = threadIdx.x;
    const int64_t ng = n / W;
    const int64_t per_pass = (int64_t)kBlock * kBiGroups;
    T xv[kBiGroups][W], rv[kBiGroups][W], rhv[kBiGroups][W], phv[kBiGroups][W],
        shv[kBiGroups][W], tv[kBiGroups][W];
    // a half step needs x and p^ only; otherwise all six (a breakdown at
    // omega, known only after the partials, then ignores four of them)
    auto load = [&](int64_t g0) {
#pragma unroll
        for (int u = 0; u < kBiGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
                vload(x + g * W, xv[u]);
                vload(ph + g * W, phv[u]);
                if (!half) {
                    vload(r + g * W, rv[u]);
                    vload(rh + g * W, rhv[u]);
                    vload(sh + g * W, shv[u]);
                    vload(t + g * W, tv[u]);
                }
            }
        }
    };
    int64_t g0 = (int64_t)blockIdx.x * per_pass;
    load(g0);   // overlaps the reading of the SpMV's partials
    double omega = 0.0;
    bool obad = false;
    if (!half) {
        const double ts = sum_parts(spart, spart_n, 2, 0, lds4);
        const double tt = sum_parts(spart, spart_n, 2, 1, lds4);
        omega = tt == 0.0 ? 0.0 : ts / tt;
        obad = tt == 0.0 || !isfinite(tt) || !isfinite(omega) || omega == 0.0;
    }
    const bool full = !half && !obad;
    const double alpha = st->alpha;
    double srh = 0.0, srr = 0.0;
    auto row = [&](T &xv, T &rv, T rhv, T phv, T shv, T tv) {
        if (full) {
            xv = (T)(((double)xv + alpha * (double)phv) + omega * (double)shv);
            rv = (T)((double)rv - omega * (double)tv);
            srh += (double)rhv * (double)rv;
            srr += (double)rv * (double)rv;
        } else {
            xv = (T)((double)xv + alpha * (double)phv);
        }
    };
    for (; g0 < ng; g0 += (int64_t)gridDim.x * per_pass) {
#pragma unroll
        for (int u = 0; u < kBiGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
#pragma unroll
                for (int k = 0; k < W; ++k)
                    row(xv[u][k], rv[u][k], rhv[u][k], phv[u][k], shv[u][k], tv[u][k]);
                vstore(x + g * W, xv[u]);
                if (full) vstore(r + g * W, rv[u]);
            }
        }
        if (g0 + (int64_t)gridDim.x * per_pass < ng) load(g0 + (int64_t)gridDim.x * per_pass);
    }
    if (blockIdx.x == 0 && tid < n - ng * W) {
        const int64_t i = ng * W + tid;
        T xi = x[i], ri = full ? r[i] : (T)0;
        row(xi, ri, full ? rh[i] : (T)0, ph[i], full ? sh[i] : (T)0, full ? t[i] : (T)0);
        x[i] = xi;
        if (full) r[i] = ri;
    }
    srh = block_sum(srh, lds4);
    srr = block_sum(srr, lds4);
    if (tid == 0) {
        store_partial(red.part + (int64_t)blockIdx.x * 2, srh);
        store_partial(red.part + (int64_t)blockIdx.x * 2 + 1, srr);
    }
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2, tmp, tot) && tid == 0) {
        BiState &s = *st;
        int running = 0;
        if (half) {
            s.half = 0;                          // status was set by the half-step kernel
        } else if (obad) {
            s.status = SLA_BREAKDOWN;            // the half step is the iterate
            s.rr = s.ss;
        } else {
            const double rhor = tot[0], rr = tot[1];
            s.omega = omega;
            s.rr = rr;
            if (sqrt(rr) <= ctl->tol * sqrt(s.bb)) {
                s.status = SLA_CONVERGED;
            } else if (!isfinite(rr)) {
                s.status = SLA_BREAKDOWN;
            } else if (s.iter >= ctl->maxit) {
                s.status = SLA_MAXIT;
            } else if (rhor == 0.0 || !isfinite(rhor)) {
                s.status = SLA_BREAKDOWN;
            } else {
                s.beta = (rhor / s.rho) * (alpha / omega);
                s.rho = rhor;
                running = 1;
            }
        }
        publish_running(ctl, h_running, running);
    }
}

// workspace of the solver, allocated at the first BiCGStab call on a handle
void ensure_workspace(Handle &h, hipStream_t s) {
    if (h.bi_state) return;
    const size_t vec = (size_t)h.n * h.vbytes;
    for (void *&v : h.bi_vec) v = dalloc(h, vec);
    h.bi_part = (double *)dalloc(h, sizeof(double) * 2 * kMaxGrid);
    h.bi_gpart = (double *)dalloc(h, sizeof(double) * 2 * kGroups);
    h.bi_spart2 = (double *)dalloc(h, sizeof(double) * 2 * std::max(kMaxGrid, kDiaGridMax));
    h.bi_sync = (uint32_t *)dalloc(h, sizeof(uint32_t) * 3 * kCountersPerKind);
    SLA_HIP(hipMemsetAsync(h.bi_sync, 0, sizeof(uint32_t) * 3 * kCountersPerKind, s));
    h.bi_state = dalloc(h, sizeof(BiState));
    SLA_HIP(hipMemsetAsync(h.bi_state, 0, sizeof(BiState), s));
}

template <typename T>
void iter_t(Handle &h, hipStream_t s, Launcher *lp) {
    constexpr int W = VecW<T>::W;
    const unsigned g = (unsigned)bi_grid(h.n, W);
    T *rh = (T *)h.bi_vec[0], *ph = (T *)h.bi_vec[1], *sh = (T *)h.bi_vec[2],
      *t = (T *)h.bi_vec[3];
    T *v = (T *)h.q;
    BiState *st = (BiState *)h.bi_state;
    const int32_t *status = &st->status;
    const int64_t sg = spmv_blocks(h);
    hipEvent_t a = nullptr;
    if (lp) lp->begin(SLA_KERNEL_DIRECTION, &a);
    hipLaunchKernelGGL(k_bi_dir<T>, dim3(g), dim3(kBlock), 0, s, h.n, (const T *)h.r, (T *)h.p, ph,
                       (const T *)v, (const T *)h.dinv, (const BiState *)st);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_DIRECTION, a);
    if (lp) lp->begin(SLA_KERNEL_SPMV_DOT, &a);
    launch_spmv_dots(h, ph, v, rh, 1, h.spart, status, s);
    if (lp) lp->end(SLA_KERNEL_SPMV_DOT, a);
    if (lp) lp->begin(SLA_KERNEL_UPDATE, &a);
    const Red red_half{h.bi_part, h.bi_gpart, h.bi_sync};
    hipLaunchKernelGGL(k_bi_half<T>, dim3(g), dim3(kBlock), 0, s, h.n, (T *)h.r, (const T *)v,
                       (const T *)h.dinv, sh, (const double *)h.spart, sg, red_half, h.ctl, st,
                       h.d_running);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_UPDATE, a);
    if (lp) lp->begin(SLA_KERNEL_SPMV_DOT, &a);
    launch_spmv_dots(h, sh, t, h.r, 2, h.bi_spart2, status, s);
    if (lp) lp->end(SLA_KERNEL_SPMV_DOT, a);
    if (lp) lp->begin(SLA_KERNEL_UPDATE, &a);
    const Red red_upd{h.bi_part, h.bi_gpart, h.bi_sync + kCountersPerKind};
    hipLaunchKernelGGL(k_bi_update<T>, dim3(g), dim3(kBlock), 0, s, h.n, (T *)h.x, (T *)h.r,
                       (const T *)rh, (const T *)ph, (const T *)sh, (const T *)t,
                       (const double *)h.bi_spart2, sg, red_upd, h.ctl, st, h.d_running);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_UPDATE, a);
}

void iter_kernels(Handle &h, hipStream_t s, Launcher *lp) {
    if (h.vt == SLA_F64) iter_t<double>(h, s, lp);
    else iter_t<float>(h, s, lp);
}

void ensure_graph(Handle &h) {
    if (h.bi_graph && h.bi_graph_k == h.check_k) return;
    if (h.bi_graph) {
        SLA_HIP(hipGraphExecDestroy(h.bi_graph));
        h.bi_graph = nullptr;
    }
    hipGraph_t g = nullptr;
    SLA_HIP(hipStreamBeginCapture(h.cap_stream, hipStreamCaptureModeThreadLocal));
    try {
        for (int k = 0; k < h.check_k; ++k) iter_kernels(h, h.cap_stream, nullptr);
    } catch (...) {
        hipGraph_t junk = nullptr;
        (void)hipStreamEndCapture(h.cap_stream, &junk);
        if (junk) (void)hipGraphDestroy(junk);
        throw;
    }
    SLA_HIP(hipStreamEndCapture(h.cap_stream, &g));
    hipGraphExec_t ex = nullptr;
    const hipError_t e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    SLA_HIP(e);
    h.bi_graph = ex;
    h.bi_graph_k = h.check_k;
}

}  // namespace

// Solve A x = b (one system, B = 1, not segmented; the caller checks). b and
// x are device vectors of n elements; x may be null with keep_internal, in
// which case the solution stays in h.x.
void bicgstab(Handle &h, const void *b, void *x, double tol, int32_t maxit, sla_info *info,
              hipStream_t s, bool keep_internal) {
    ensure_workspace(h, s);
    Launcher L{h, s, h.profile};
    Launcher *lp = h.profile ? &L : nullptr;
    h.h_ctl->tol = tol;
    h.h_ctl->maxit = maxit;
    h.h_ctl->n_running = 0;
    h.h_ctl->epoch = ++h.epoch;
    h.h_ctl->error = 0;
    h.h_ctl->spin_limit = h.spin_limit;
    SLA_HIP(hipMemcpyAsync(h.ctl, h.h_ctl, sizeof(Ctl), hipMemcpyHostToDevice, s));
    h.last_path = kPathPerStep;   // its own kernels, none of which waits on another workgroup
    h.last_fallback = 0;
    {
        int64_t g = (h.n + kBlock - 1) / kBlock;
        if (g > kMaxGrid) g = kMaxGrid;
        hipEvent_t a = nullptr;
        if (lp) lp->begin(SLA_KERNEL_INIT, &a);
        const Red red{h.bi_part, h.bi_gpart, h.bi_sync + 2 * kCountersPerKind};
        if (h.vt == SLA_F64)
            hipLaunchKernelGGL(k_bi_init<double>, dim3((unsigned)g), dim3(kBlock), 0, s, h.n,
                               (const double *)b, (double *)h.x, (double *)h.r,
                               (double *)h.bi_vec[0], red, h.ctl, (BiState *)h.bi_state,
                               h.d_running);
        else
            hipLaunchKernelGGL(k_bi_init<float>, dim3((unsigned)g), dim3(kBlock), 0, s, h.n,
                               (const float *)b, (float *)h.x, (float *)h.r, (float *)h.bi_vec[0],
                               red, h.ctl, (BiState *)h.bi_state, h.d_running);
        SLA_HIP(hipGetLastError());
        if (lp) lp->end(SLA_KERNEL_INIT, a);
    }
    const bool graph = h.use_graph && !h.profile;
    if (graph) ensure_graph(h);
    const int64_t k = h.check_k;
    const int64_t max_chunks = maxit <= 0 ? 0 : (maxit + k - 1) / k;
    for (int64_t ch = 0; ch < max_chunks; ++ch) {
        if (graph) {
            SLA_HIP(hipGraphLaunch(h.bi_graph, s));
        } else {
            for (int64_t j = 0; j < k; ++j) iter_kernels(h, s, lp);
        }
        SLA_HIP(hipEventRecord(h.ev[ch & 1], s));
        // poll the block before this one while this one runs
        if (ch >= 1) {
            SLA_HIP(hipEventSynchronize(h.ev[(ch - 1) & 1]));
            if (__atomic_load_n(h.h_running, __ATOMIC_ACQUIRE) == 0) break;
        }
    }
    if (!keep_internal)
        SLA_HIP(hipMemcpyAsync(x, h.x, (size_t)h.n * h.vbytes, hipMemcpyDeviceToDevice, s));
    BiState hs{};
    SLA_HIP(hipMemcpyAsync(&hs, h.bi_state, sizeof(BiState), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    if (h.profile) flush_profile(h);
    info[0].iterations = hs.iter;
    info[0].status = hs.status == kRunning ? SLA_MAXIT : hs.status;
    info[0].rel_residual = hs.bb == 0.0 ? 0.0 : sqrt(hs.rr / hs.bb);
}

}  // namespace sla

// Jacobi-preconditioned CG on the device, its adjoint value gradient, and the
// host driver that replays blocks of iterations as hipGraphs.
//
// torch-sla's pytorch-native backend runs CG with Jacobi preconditioning with
// every tensor on the device (backend list; distributed-CG paragraph: one
// SpMV and the two inner products <r,r>, <p,Ap> per iteration; Table 3 and
// Table 4 text). Backward solves A^T lambda = dL/dx and forms -lambda_i x_j
// on the stored entries (adjoint paragraph of the distributed section). The
// recurrence itself is not printed there; this is textbook PCG from x0 = 0:
//   r = b, z = D^-1 r, p = z, rho = r.z
//   q = A p, alpha = rho / p.q, x += alpha p, r -= alpha q,
//   converged when ||r|| <= tol ||b||, else rho' = r.z', beta = rho'/rho,
//   p = z' + beta p.
// One iteration is three kernels: the fused SpMV (q and the p.q partials,
// alpha), the fused update (x, r, and the r.z / r.r partials, the test, beta)
// and the direction update. Each system's status lives on the device; kernels
// leave finished systems untouched, so the host can poll every k iterations
// without changing the iterate or the count.
#include <atomic>

#include "common.h"

namespace sla {

void launch_spmv_dot(Handle &h, hipStream_t s);
int64_t spmv_grid(const Handle &h);
void launch_spmv_plain(Handle &h, const void *x, void *y, hipStream_t s);

namespace {

constexpr int kVecItems = 4;  // rows per lane and pass (loads issued together)
constexpr int kVecGroups = 2;  // 16-byte groups per lane and pass

int64_t vec_grid(int64_t n, int B) {
    const int64_t rows = (int64_t)(kBlock / B) * kVecItems;
    int64_t g = (n + rows - 1) / rows;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g < 1) g = 1;
    return g;
}

// r = b, x = 0, p = z = dinv r (and z into z_out unless null); partials of
// b.b and r.z; last block sets up the per-system scalars and status.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_init(int64_t n, int B, const T *__restrict__ b_in,
                                                 T *__restrict__ x, T *__restrict__ r,
                                                 T *__restrict__ p, const T *__restrict__ dinv,
                                                 T *__restrict__ z_out, Red red,
                                                 Ctl *__restrict__ ctl, SysState *__restrict__ st,
                                                 int32_t *__restrict__ h_running) {
    __shared__ double tmp[kBlock];
    __shared__ double blk[kMaxBatch];
    __shared__ double tot[2 * kMaxBatch];
    const Lanes L(B);
    double sbb = 0.0, srz = 0.0;
    if (L.on) {
        const int64_t step = (int64_t)gridDim.x * L.J * kVecItems;
        for (int64_t base = (int64_t)blockIdx.x * L.J * kVecItems + L.jr; base < n; base += step) {
            T bv[kVecItems], dv[kVecItems];
#pragma unroll
            for (int u = 0; u < kVecItems; ++u) {
                const int64_t i = base + (int64_t)u * L.J;
                const int64_t f = i * B + L.b;
                bv[u] = i < n ? b_in[f] : (T)0;
                dv[u] = i < n ? dinv[f] : (T)0;
            }
#pragma unroll
            for (int u = 0; u < kVecItems; ++u) {
                const int64_t i = base + (int64_t)u * L.J;
                if (i >= n) break;
                const int64_t f = i * B + L.b;
                const double z = (double)dv[u] * (double)bv[u];
                x[f] = (T)0;
                r[f] = bv[u];
                p[f] = (T)z;
                if (z_out) z_out[f] = (T)z;
                sbb += (double)bv[u] * (double)bv[u];
                srz += (double)bv[u] * z;
            }
        }
    }
    block_sum_per_system(sbb, L, tmp, blk);
    if (threadIdx.x < B)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + threadIdx.x, blk[threadIdx.x]);
    __syncthreads();
    block_sum_per_system(srz, L, tmp, blk);
    if (threadIdx.x < B)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + B + threadIdx.x, blk[threadIdx.x]);
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2 * B, tmp, tot)) {
        // one thread per system
        const int32_t maxit = ctl->maxit;
        int running = 0;
        for (int b = threadIdx.x; b < B; b += kBlock) {
            SysState s;
            s.bb = tot[b];
            s.rho = tot[B + b];
            s.alpha = 0.0;
            s.alpha2 = 0.0;
            s.beta = 0.0;
            s.rr = s.bb;
            s.iter = 0;
            if (s.bb == 0.0) s.status = SLA_CONVERGED;
            else if (maxit <= 0) s.status = SLA_MAXIT;
            else s.status = kRunning;
            running += s.status == kRunning;
            st[b] = s;
        }
        running = block_count(running);
        if (threadIdx.x == 0) publish_running(ctl, h_running, running);
    }
}

// Last block of an update (every thread of it calls this, one thread per
// system): r.z and r.r per system in tot[0..2B); applies the stopping test,
// the iteration budget and beta, then publishes the number still running.
__device__ __forceinline__ void finish_update(const double *tot, int B, Ctl *ctl, SysState *st,
                                              int32_t *h_running) {
    const double tol = ctl->tol;
    const int32_t maxit = ctl->maxit;
    int running = 0;
    for (int b = threadIdx.x; b < B; b += kBlock) {
        SysState &s = st[b];
        if (s.status != kRunning) continue;
        const double rz = tot[b], rr = tot[B + b];
        s.rr = rr;
        s.iter += 1;
        if (sqrt(rr) <= tol * sqrt(s.bb)) {
            s.status = SLA_CONVERGED;
        } else if (s.iter >= maxit) {
            s.status = SLA_MAXIT;
        } else {
            s.beta = rz / s.rho;
            s.rho = rz;
            ++running;
        }
    }
    running = block_count(running);
    if (threadIdx.x == 0) publish_running(ctl, h_running, running);
}

// The same for the batched kernels whose SpMV left only group sums of p.q
// (sigma[b], summed by every block of the update): the breakdown test on
// sigma, alpha kept in the state (the folded solve applies it to x later),
// then the stopping test, budget and beta of every system that stepped.
__device__ __forceinline__ void finish_update_sigma(const double *tot, const double *sigma, int B,
                                                    Ctl *ctl, SysState *st, int32_t *h_running) {
    const double tol = ctl->tol;
    const int32_t maxit = ctl->maxit;
    int running = 0;
    for (int b = threadIdx.x; b < B; b += kBlock) {
        SysState &s = st[b];
        if (s.status != kRunning) continue;
        s.iter += 1;
        const double sg = sigma[b];
        if (!(sg > 0.0) || !isfinite(sg)) {
            s.status = SLA_BREAKDOWN;   // x, r untouched; rr keeps the last residual
            s.alpha = 0.0;
            continue;
        }
        s.alpha = s.rho / sg;
        const double rz = tot[b], rr = tot[B + b];
        s.rr = rr;
        if (sqrt(rr) <= tol * sqrt(s.bb)) {
            s.status = SLA_CONVERGED;
        } else if (s.iter >= maxit) {
            s.status = SLA_MAXIT;
        } else {
            s.beta = rz / s.rho;
            s.rho = rz;
            ++running;
        }
    }
    running = block_count(running);
    if (threadIdx.x == 0) publish_running(ctl, h_running, running);
}

// x += alpha p, r -= alpha q; partials of r.z and r.r with z = dinv r; the
// last block applies the stopping test, the iteration budget and beta.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_update(int64_t n, int B, T *__restrict__ x,
                                                   T *__restrict__ r, const T *__restrict__ p,
                                                   const T *__restrict__ q,
                                                   const T *__restrict__ dinv, Red red,
                                                   Ctl *__restrict__ ctl,
                                                   SysState *__restrict__ st,
                                                   int32_t *__restrict__ h_running) {
    __shared__ double tmp[kBlock];
    __shared__ double blk[kMaxBatch];
    __shared__ double tot[2 * kMaxBatch];
    if (ctl->n_running == 0) return;
    const Lanes L(B);
    const bool active = L.on && st[L.b].status == kRunning;
    const double alpha = L.on ? st[L.b].alpha : 0.0;
    double srz = 0.0, srr = 0.0;
    if (active) {
        // pass base (uniform, 64-bit) + per-lane 32-bit offsets
        const int64_t rows_pass = (int64_t)L.J * kVecItems;
        for (int64_t r0 = (int64_t)blockIdx.x * rows_pass; r0 < n; r0 += (int64_t)gridDim.x * rows_pass) {
            const int64_t fb = r0 * B;
            T *xb = x + fb;
            T *rb = r + fb;
            const T *pb = p + fb;
            const T *qb = q + fb;
            const T *db = dinv + fb;
            const int64_t left = n - r0;
            T xv[kVecItems], pv[kVecItems], rv[kVecItems], qv[kVecItems], dv[kVecItems];
#pragma unroll
            for (int u = 0; u < kVecItems; ++u) {
                const int ii = u * L.J + L.jr;
                const int o = ii * B + L.b;
                const bool in = ii < left;
                xv[u] = in ? xb[o] : (T)0;
                pv[u] = in ? pb[o] : (T)0;
                rv[u] = in ? rb[o] : (T)0;
                qv[u] = in ? qb[o] : (T)0;
                dv[u] = in ? db[o] : (T)0;
            }
#pragma unroll
            for (int u = 0; u < kVecItems; ++u) {
                const int ii = u * L.J + L.jr;
                if (ii >= left) break;
                const int o = ii * B + L.b;
                const T xn = (T)((double)xv[u] + alpha * (double)pv[u]);
                const T rn = (T)((double)rv[u] - alpha * (double)qv[u]);
                xb[o] = xn;
                rb[o] = rn;
                const double z = (double)dv[u] * (double)rn;
                srz += (double)rn * z;
                srr += (double)rn * (double)rn;
            }
        }
    }
    block_sum_per_system(srz, L, tmp, blk);
    if (threadIdx.x < B)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + threadIdx.x, blk[threadIdx.x]);
    __syncthreads();
    block_sum_per_system(srr, L, tmp, blk);
    if (threadIdx.x < B)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + B + threadIdx.x, blk[threadIdx.x]);
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2 * B, tmp, tot))
        finish_update(tot, B, ctl, st, h_running);
}

// Batched (B > 1) update and direction with 16-byte accesses, for Q = B / W a
// power of two (W = 16 / sizeof(T)): chunk c of W consecutive values of the
// [n][B] layout holds systems (c % Q) * W .. + W - 1 of row c / Q, and since
// the chunk stride of every lane is a multiple of kBlock, lane t always holds
// systems (t % Q) * W + w. Systems that are not running keep their values
// (the stored chunk carries the old bits for them).
// FOLD (folded batched solve): x and p are not touched; z = dinv r is stored
// in x's place (the z buffer), and the last block counts the update in
// ctl->fold_iter.
//
// The SpMV before it left group sums of p.q (sg, for an SpMV of sg_blocks
// blocks): every block finishes that sum (group order) and forms alpha per
// system; a system whose p.q is not > 0 or not finite breaks down here.
template <typename T, bool FOLD = false>
__global__ __launch_bounds__(kBlock) void k_update_bv(int64_t nc, int B, T *__restrict__ x,
                                                      T *__restrict__ r, const T *__restrict__ p,
                                                      const T *__restrict__ q,
                                                      const T *__restrict__ dinv,
                                                      const double *__restrict__ sg,
                                                      int64_t sg_blocks, Red red,
                                                      Ctl *__restrict__ ctl,
                                                      SysState *__restrict__ st,
                                                      int32_t *__restrict__ h_running) {
    constexpr int W = VecW<T>::W;
    __shared__ double tmp[4 * kMaxBatch];
    __shared__ double blk[kMaxBatch];
    __shared__ double tot[2 * kMaxBatch];
    __shared__ double sigma[kMaxBatch];
    if (ctl->n_running == 0) return;
    const int Q = B / W;
    const int t = threadIdx.x;
    const int s0 = (t & (Q - 1)) * W;
    // the first pass's rows are requested before the sum of the SpMV's group
    // rows, so that their latency overlaps it
    bool any_run = false;
#pragma unroll
    for (int w = 0; w < W; ++w) any_run |= st[s0 + w].status == kRunning;
    const int64_t per_pass = (int64_t)kBlock * kVecGroups;
    T xv[kVecGroups][W], pv[kVecGroups][W], rv[kVecGroups][W], qv[kVecGroups][W],
        dv[kVecGroups][W];
    auto load_pass = [&](int64_t c0) {
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t c = c0 + u * kBlock + t;
            if (c < nc) {
                // FOLD: xv carries z (x's own bits for stopped systems)
                vload(x + c * W, xv[u]);
                if (!FOLD) vload(p + c * W, pv[u]);
                vload(r + c * W, rv[u]);
                vload(q + c * W, qv[u]);
                vload(dinv + c * W, dv[u]);
            }
        }
    };
    int64_t c0 = (int64_t)blockIdx.x * per_pass;
    if (any_run && c0 < nc) load_pass(c0);
    group_total(sg, sg_blocks, B, tmp, sigma);
    bool act[W];
    double alpha[W];
    bool any = false;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const double sw = sigma[s0 + w];
        act[w] = st[s0 + w].status == kRunning && sw > 0.0 && isfinite(sw);
        alpha[w] = act[w] ? st[s0 + w].rho / sw : 0.0;
        any |= act[w];
    }
    double srz[W], srr[W];
#pragma unroll
    for (int w = 0; w < W; ++w) srz[w] = srr[w] = 0.0;
    auto process_pass = [&](int64_t c0) {
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t c = c0 + u * kBlock + t;
            if (c >= nc) continue;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                if (!act[w]) continue;
                if (!FOLD) xv[u][w] = (T)((double)xv[u][w] + alpha[w] * (double)pv[u][w]);
                rv[u][w] = (T)((double)rv[u][w] - alpha[w] * (double)qv[u][w]);
                const double z = (double)dv[u][w] * (double)rv[u][w];
                if (FOLD) xv[u][w] = (T)z;
                srz[w] += (double)rv[u][w] * z;
                srr[w] += (double)rv[u][w] * (double)rv[u][w];
            }
            vstore(x + c * W, xv[u]);
            vstore(r + c * W, rv[u]);
        }
    };
    if (any) {
        if (c0 < nc) process_pass(c0);
        for (c0 += (int64_t)gridDim.x * per_pass; c0 < nc; c0 += (int64_t)gridDim.x * per_pass) {
            load_pass(c0);
            process_pass(c0);
        }
    }
    block_sum_systems<W>(srz, Q, tmp, blk);
    for (int s = t; s < B; s += kBlock)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + s, blk[s]);
    block_sum_systems<W>(srr, Q, tmp, blk);
    for (int s = t; s < B; s += kBlock)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + B + s, blk[s]);
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2 * B, tmp, tot)) {
        finish_update_sigma(tot, sigma, B, ctl, st, h_running);
        if (FOLD && t == 0) ctl->fold_iter += 1;
    }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_direction_bv(int64_t nc, int B,
                                                         const T *__restrict__ r,
                                                         T *__restrict__ p,
                                                         const T *__restrict__ dinv,
                                                         const Ctl *__restrict__ ctl,
                                                         const SysState *__restrict__ st) {
    constexpr int W = VecW<T>::W;
    if (ctl->n_running == 0) return;
    const int Q = B / W;
    const int t = threadIdx.x;
    const int s0 = (t & (Q - 1)) * W;
    bool act[W];
    double beta[W];
    bool any = false;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        act[w] = st[s0 + w].status == kRunning;
        beta[w] = act[w] ? st[s0 + w].beta : 0.0;
        any |= act[w];
    }
    if (!any) return;
    const int64_t per_pass = (int64_t)kBlock * kVecGroups;
    for (int64_t c0 = (int64_t)blockIdx.x * per_pass; c0 < nc; c0 += (int64_t)gridDim.x * per_pass) {
        T rv[kVecGroups][W], pv[kVecGroups][W], dv[kVecGroups][W];
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t c = c0 + u * kBlock + t;
            if (c < nc) {
                vload(r + c * W, rv[u]);
                vload(p + c * W, pv[u]);
                vload(dinv + c * W, dv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t c = c0 + u * kBlock + t;
            if (c >= nc) continue;
#pragma unroll
            for (int w = 0; w < W; ++w)
                if (act[w])
                    pv[u][w] = (T)((double)dv[u][w] * (double)rv[u][w] + beta[w] * (double)pv[u][w]);
            vstore(p + c * W, pv[u]);
        }
    }
}

// Batched update and direction in one kernel (bv layout, Q = B / W a power of
// two), for grids that are resident at once: one pass of kFusedGroups
// 16-byte chunks per lane. After the per-system reductions the last
// workgroup publishes every system's beta and whether it still runs
// (device-scope stores, then a generation word one above the one every
// workgroup read at its start); the others wait for it (bounded; a timeout is
// reported through ctl->error) and write p = z + beta p for their chunks from
// registers, which saves reading r, p and dinv again and a launch.
constexpr int kBvFusedGroups = 4;

// Entry check of the kernels of a fused step: nothing to do once no system
// runs, or once a bounded wait of this solve has given up (ctl->error is
// sticky). In the second case the first workgroup publishes "none running",
// so the host stops launching and re-runs the solve on kernels without
// grid-wide waits.
__device__ __forceinline__ bool fused_step_idle(Ctl *ctl, int32_t *h_running) {
    if (__hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        if (blockIdx.x == 0 && threadIdx.x == 0) publish_running(ctl, h_running, 0);
        return true;
    }
    return ctl->n_running == 0;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_update_dir_bv(int64_t nc, int B, T *__restrict__ x,
                                                          T *__restrict__ r, T *__restrict__ p,
                                                          const T *__restrict__ q,
                                                          const T *__restrict__ dinv,
                                                          const double *__restrict__ sg,
                                                          int64_t sg_blocks, Red red,
                                                          Ctl *__restrict__ ctl,
                                                          SysState *__restrict__ st,
                                                          int32_t *__restrict__ h_running,
                                                          Bcast *__restrict__ bc,
                                                          double *__restrict__ bcv) {
    constexpr int W = VecW<T>::W;
    constexpr int U = kBvFusedGroups;
    __shared__ double tmp[4 * kMaxBatch];
    __shared__ double blk[kMaxBatch];
    __shared__ double tot[2 * kMaxBatch];
    __shared__ double sigma[kMaxBatch];
    __shared__ int s_ok;
    if (fused_step_idle(ctl, h_running)) return;
    const uint64_t gen =
        __hip_atomic_load(&bc->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    const int Q = B / W;
    const int t = threadIdx.x;
    const int s0 = (t & (Q - 1)) * W;
    // this workgroup's rows first, so that their latency overlaps the sum of
    // the SpMV's group rows (sigma = p.q per system, group order)
    const int64_t c0 = (int64_t)blockIdx.x * kBlock * U;
    T xv[U][W], pv[U][W], rv[U][W], qv[U][W], dv[U][W];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kBlock + t;
        if (c < nc) {
            vload(x + c * W, xv[u]);
            vload(p + c * W, pv[u]);
            vload(r + c * W, rv[u]);
            vload(q + c * W, qv[u]);
            vload(dinv + c * W, dv[u]);
        }
    }
    group_total(sg, sg_blocks, B, tmp, sigma);
    bool act[W];
    double alpha[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const double sw = sigma[s0 + w];
        act[w] = st[s0 + w].status == kRunning && sw > 0.0 && isfinite(sw);
        alpha[w] = act[w] ? st[s0 + w].rho / sw : 0.0;
    }
    double srz[W], srr[W];
#pragma unroll
    for (int w = 0; w < W; ++w) srz[w] = srr[w] = 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kBlock + t;
        if (c >= nc) continue;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            if (!act[w]) continue;
            xv[u][w] = (T)((double)xv[u][w] + alpha[w] * (double)pv[u][w]);
            rv[u][w] = (T)((double)rv[u][w] - alpha[w] * (double)qv[u][w]);
            const double z = (double)dv[u][w] * (double)rv[u][w];
            srz[w] += (double)rv[u][w] * z;
            srr[w] += (double)rv[u][w] * (double)rv[u][w];
        }
        vstore(x + c * W, xv[u]);
        vstore(r + c * W, rv[u]);
    }
    block_sum_systems<W>(srz, Q, tmp, blk);
    for (int s = t; s < B; s += kBlock)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + s, blk[s]);
    block_sum_systems<W>(srr, Q, tmp, blk);
    for (int s = t; s < B; s += kBlock)
        store_partial(red.part + (int64_t)blockIdx.x * 2 * B + B + s, blk[s]);
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2 * B, tmp, tot)) {
        // the stopping test, budget and beta of every system (as in
        // finish_update), one thread per system, then the broadcast
        const double tol = ctl->tol;
        int running = 0;
        for (int b = t; b < B; b += kBlock) {
            SysState &sy = st[b];
            int run = 0;
            const double sgb = sigma[b];
            if (sy.status == kRunning && !(sgb > 0.0 && isfinite(sgb))) {
                sy.iter += 1;
                sy.status = SLA_BREAKDOWN;   // x, r untouched; rr keeps the last residual
                sy.alpha = 0.0;
            } else if (sy.status == kRunning) {
                const double rz = tot[b], rr = tot[B + b];
                sy.alpha = sy.rho / sgb;
                sy.rr = rr;
                sy.iter += 1;
                if (sqrt(rr) <= tol * sqrt(sy.bb)) {
                    sy.status = SLA_CONVERGED;
                } else if (sy.iter >= ctl->maxit) {
                    sy.status = SLA_MAXIT;
                } else {
                    sy.beta = rz / sy.rho;
                    sy.rho = rz;
                    run = 1;
                }
            }
            store_partial(bcv + 2 * b, sy.beta);
            store_partial(bcv + 2 * b + 1, run ? 1.0 : 0.0);
            running += run;
        }
        tmp[t] = (double)running;
        __syncthreads();
        if (t == 0) {
            int total = 0;
            const int nt = B < kBlock ? B : kBlock;
            for (int j = 0; j < nt; ++j) total += (int)tmp[j];
            publish_running(ctl, h_running, total);
        }
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t == 0) __hip_atomic_store(&bc->gen, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (t == 0) {
        const uint32_t limit = ctl->spin_limit;
        uint32_t spins = 0;
        int ok = 1;
        while (__hip_atomic_load(&bc->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gen) {
            if (++spins > limit) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) {
            __hip_atomic_store(&ctl->error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            publish_running(ctl, h_running, 0);
        }
        s_ok = ok;
    }
    __syncthreads();
    if (!s_ok) return;
    double beta[W];
    bool run[W];
#pragma unroll
    for (int w = 0; w < W; ++w) {
        beta[w] = load_partial(bcv + 2 * (s0 + w));
        run[w] = act[w] && load_partial(bcv + 2 * (s0 + w) + 1) != 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * kBlock + t;
        if (c >= nc) continue;
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (run[w])
                pv[u][w] = (T)((double)dv[u][w] * (double)rv[u][w] + beta[w] * (double)pv[u][w]);
        vstore(p + c * W, pv[u]);
    }
}

template <typename T>
bool bv_ok(const Handle &h) {
    constexpr int W = VecW<T>::W;
    if (h.B < 2 || h.B % W) return false;
    const int Q = h.B / W;
    return (Q & (Q - 1)) == 0 && Q <= kBlock;
}

// at most the workgroups resident at once: a larger grid would run a second,
// partial round
int64_t bv_grid(int64_t nc, int64_t resident) {
    const int64_t per = (int64_t)kBlock * kVecGroups;
    int64_t g = (nc + per - 1) / per;
    if (g > resident) g = resident;
    if (g < 1) g = 1;
    return g;
}

// Single-system (B = 1) forms of the update and direction kernels: every
// array access is 16 bytes per lane (W = 16 / sizeof(T) consecutive rows), so
// each memory instruction moves twice (fp64) or four times (fp32) the data of
// the per-row forms; rows past the last full group are done by block 0.

//
// FOLD (direction folded into the SpMV, see FoldArgs): x and p are not
// touched here; z = dinv r is stored into x's place (the z buffer), and the
// step alpha is kept in the system state for the next SpMV (or the final
// x update) to apply to x.
template <typename T, bool NT, bool FOLD = false>
__global__ __launch_bounds__(kBlock) void k_update1(int64_t n, T *__restrict__ x,
                                                    T *__restrict__ r, const T *__restrict__ p,
                                                    const T *__restrict__ q,
                                                    const T *__restrict__ dinv,
                                                    const double *__restrict__ spart,
                                                    int64_t spart_n, Red red,
                                                    Ctl *__restrict__ ctl,
                                                    SysState *__restrict__ st,
                                                    int32_t *__restrict__ h_running) {
    constexpr int W = VecW<T>::W;
    __shared__ double lds4[kWaves];
    __shared__ double tmp[kBlock];
    __shared__ double tot[2];
    if (ctl->n_running == 0) return;  // one system: running or not
    const int tid = threadIdx.x;
    // sigma = p.q from the SpMV's per-workgroup partials, summed by every
    // workgroup in the same order (identical in all of them)
    double sg = 0.0;
    for (int64_t j = tid; j < spart_n; j += 4 * kBlock) {
        double v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v4[u] = j + u * kBlock < spart_n ? spart[j + u * kBlock] : 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u) sg += v4[u];
    }
    const double sigma = block_sum(sg, lds4);
    const bool breakdown = !(sigma > 0.0) || !isfinite(sigma);
    const double alpha = breakdown ? 0.0 : st[0].rho / sigma;
    double srz = 0.0, srr = 0.0;
    // FOLD: xv carries z out instead of x
    auto row = [&](T &xv, T &rv, T pv, T qv, T dv) {
        if (!FOLD) xv = (T)((double)xv + alpha * (double)pv);
        rv = (T)((double)rv - alpha * (double)qv);
        const double z = (double)dv * (double)rv;
        if (FOLD) xv = (T)z;
        srz += (double)rv * z;
        srr += (double)rv * (double)rv;
    };
    const int64_t ng = breakdown ? 0 : n / W;   // breakdown: x and r stay as they are
    const int64_t per_pass = (int64_t)kBlock * kVecGroups;
    for (int64_t g0 = (int64_t)blockIdx.x * per_pass; g0 < ng; g0 += (int64_t)gridDim.x * per_pass) {
        T xv[kVecGroups][W], pv[kVecGroups][W], rv[kVecGroups][W], qv[kVecGroups][W],
            dv[kVecGroups][W];
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
                if (!FOLD) {
                    vload_h<NT>(x + g * W, xv[u]);
                    vload_h<NT>(p + g * W, pv[u]);
                }
                vload_h<NT>(r + g * W, rv[u]);
                vload_h<NT>(q + g * W, qv[u]);
                vload_h<NT>(dinv + g * W, dv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
#pragma unroll
                for (int k = 0; k < W; ++k) row(xv[u][k], rv[u][k], pv[u][k], qv[u][k], dv[u][k]);
                vstore_h<NT>(x + g * W, xv[u]);
                vstore_h<NT>(r + g * W, rv[u]);
            }
        }
    }
    if (!breakdown && blockIdx.x == 0 && tid < n - ng * W) {
        const int64_t i = ng * W + tid;
        T xi = FOLD ? (T)0 : x[i], ri = r[i];
        row(xi, ri, FOLD ? (T)0 : p[i], q[i], dinv[i]);
        x[i] = xi;
        r[i] = ri;
    }
    srz = block_sum(srz, lds4);
    srr = block_sum(srr, lds4);
    if (tid == 0) {
        store_partial(red.part + (int64_t)blockIdx.x * 2, srz);
        store_partial(red.part + (int64_t)blockIdx.x * 2 + 1, srr);
    }
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2, tmp, tot)) {
        if (tid == 0) {
            SysState &sy = st[0];
            const double rz = tot[0], rr = tot[1];
            int running = 0;
            sy.iter += 1;
            if (FOLD) {
                // x += alpha p is applied later (0 at breakdown), together
                // with the step before where that one is still pending
                sy.alpha2 = sy.alpha;
                sy.alpha = alpha;
            }
            if (breakdown) {
                sy.status = SLA_BREAKDOWN;  // x, r untouched; rr keeps the last residual
            } else {
                sy.rr = rr;
            }
            if (breakdown) {
                // nothing more: the solve ends here
            } else if (sqrt(rr) <= ctl->tol * sqrt(sy.bb)) {
                sy.status = SLA_CONVERGED;
            } else if (sy.iter >= ctl->maxit) {
                sy.status = SLA_MAXIT;
            } else {
                sy.beta = rz / sy.rho;
                sy.rho = rz;
                running = 1;
            }
            publish_running(ctl, h_running, running);
        }
    }
}

// Single system, update and direction in one kernel: every workgroup does
// one pass of kFusedGroups 16-byte groups per lane, keeps r, p and dinv of
// its rows in registers, and waits for the last workgroup of the r.z / r.r
// reduction to broadcast beta (and whether the system still runs); then it
// writes p = z + beta p for the same rows. This saves reading r, p and dinv
// a second time. All workgroups must be resident at once (the grid is at
// most the occupancy-API count, launched on an otherwise idle stream); the
// wait is bounded and a timeout is reported through ctl->error.
constexpr int kFusedGroups = 4;

template <typename T>
__global__ __launch_bounds__(kBlock) void k_update_dir1(int64_t n, T *__restrict__ x,
                                                        T *__restrict__ r, T *__restrict__ p,
                                                        const T *__restrict__ q,
                                                        const T *__restrict__ dinv,
                                                        const double *__restrict__ spart,
                                                        int64_t spart_n, Red red,
                                                        Ctl *__restrict__ ctl,
                                                        SysState *__restrict__ st,
                                                        int32_t *__restrict__ h_running,
                                                        Bcast *__restrict__ bc) {
    constexpr int W = VecW<T>::W;
    __shared__ double lds4[kWaves];
    __shared__ double tmp[kBlock];
    __shared__ double tot[2];
    __shared__ double s_beta;
    __shared__ int s_run;
    if (fused_step_idle(ctl, h_running)) return;  // one system: running or not
    const int tid = threadIdx.x;
    const uint64_t gen = ((uint64_t)ctl->epoch << 32) | (uint32_t)(st[0].iter + 1);
    // this workgroup's rows are loaded first, so their latency overlaps the
    // reading of the SpMV's partials below
    const int64_t ngl = n / W;
    const int64_t g0 = (int64_t)blockIdx.x * kBlock * kFusedGroups;
    T xv[kFusedGroups][W], pv[kFusedGroups][W], rv[kFusedGroups][W], qv[kFusedGroups][W],
        dv[kFusedGroups][W];
#pragma unroll
    for (int u = 0; u < kFusedGroups; ++u) {
        const int64_t g = g0 + u * kBlock + tid;
        if (g < ngl) {
            vload(x + g * W, xv[u]);
            vload(p + g * W, pv[u]);
            vload(r + g * W, rv[u]);
            vload(q + g * W, qv[u]);
            vload(dinv + g * W, dv[u]);
        }
    }
    double sg = 0.0;
    for (int64_t j = tid; j < spart_n; j += 4 * kBlock) {
        double v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v4[u] = j + u * kBlock < spart_n ? spart[j + u * kBlock] : 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u) sg += v4[u];
    }
    const double sigma = block_sum(sg, lds4);
    const bool breakdown = !(sigma > 0.0) || !isfinite(sigma);
    const double alpha = breakdown ? 0.0 : st[0].rho / sigma;
    double srz = 0.0, srr = 0.0;
    const int64_t ng = breakdown ? 0 : ngl;   // breakdown: x and r stay as they are
    auto row = [&](T &xe, T &re, T pe, T qe, T de) {
        xe = (T)((double)xe + alpha * (double)pe);
        re = (T)((double)re - alpha * (double)qe);
        const double z = (double)de * (double)re;
        srz += (double)re * z;
        srr += (double)re * (double)re;
    };
#pragma unroll
    for (int u = 0; u < kFusedGroups; ++u) {
        const int64_t g = g0 + u * kBlock + tid;
        if (g < ng) {
#pragma unroll
            for (int k = 0; k < W; ++k) row(xv[u][k], rv[u][k], pv[u][k], qv[u][k], dv[u][k]);
            vstore(x + g * W, xv[u]);
            vstore(r + g * W, rv[u]);
        }
    }
    // rows past the last whole group: workgroup 0, one per lane
    const bool tail = !breakdown && blockIdx.x == 0 && tid < n - ng * W;
    T xt = (T)0, rt = (T)0, pt = (T)0, dt = (T)0;
    if (tail) {
        const int64_t i = ng * W + tid;
        xt = x[i];
        rt = r[i];
        pt = p[i];
        dt = dinv[i];
        row(xt, rt, pt, q[i], dt);
        x[i] = xt;
        r[i] = rt;
    }
    srz = block_sum(srz, lds4);
    srr = block_sum(srr, lds4);
    if (tid == 0) {
        store_partial(red.part + (int64_t)blockIdx.x * 2, srz);
        store_partial(red.part + (int64_t)blockIdx.x * 2 + 1, srr);
    }
    if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, 2, tmp, tot)) {
        if (tid == 0) {
            SysState &sy = st[0];
            const double rz = tot[0], rr = tot[1];
            int running = 0;
            sy.iter += 1;
            if (breakdown) {
                sy.status = SLA_BREAKDOWN;  // x, r untouched; rr keeps the last residual
            } else {
                sy.rr = rr;
                if (sqrt(rr) <= ctl->tol * sqrt(sy.bb)) {
                    sy.status = SLA_CONVERGED;
                } else if (sy.iter >= ctl->maxit) {
                    sy.status = SLA_MAXIT;
                } else {
                    sy.beta = rz / sy.rho;
                    sy.rho = rz;
                    running = 1;
                }
            }
            publish_running(ctl, h_running, running);
            __hip_atomic_store(&bc->beta, sy.beta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&bc->running, running, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __hip_atomic_store(&bc->gen, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid == 0) {
        const uint32_t limit = ctl->spin_limit;
        uint32_t spins = 0;
        bool ok = true;
        while (__hip_atomic_load(&bc->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != gen) {
            if (++spins > limit) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (ok) {
            s_beta = __hip_atomic_load(&bc->beta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_run = __hip_atomic_load(&bc->running, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_store(&ctl->error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            publish_running(ctl, h_running, 0);
            s_run = 0;
        }
    }
    __syncthreads();
    if (!s_run) return;
    const double beta = s_beta;
#pragma unroll
    for (int u = 0; u < kFusedGroups; ++u) {
        const int64_t g = g0 + u * kBlock + tid;
        if (g < ng) {
#pragma unroll
            for (int k = 0; k < W; ++k)
                pv[u][k] = (T)((double)dv[u][k] * (double)rv[u][k] + beta * (double)pv[u][k]);
            vstore(p + g * W, pv[u]);
        }
    }
    if (tail) p[ng * W + tid] = (T)((double)dt * (double)rt + beta * (double)pt);
}

template <typename T, bool NT>
__global__ __launch_bounds__(kBlock) void k_direction1(int64_t n, const T *__restrict__ r,
                                                       T *__restrict__ p,
                                                       const T *__restrict__ dinv,
                                                       const Ctl *__restrict__ ctl,
                                                       const SysState *__restrict__ st) {
    constexpr int W = VecW<T>::W;
    if (ctl->n_running == 0) return;
    const double beta = st[0].beta;
    const int tid = threadIdx.x;
    const int64_t ng = n / W;
    const int64_t per_pass = (int64_t)kBlock * kVecGroups;
    for (int64_t g0 = (int64_t)blockIdx.x * per_pass; g0 < ng; g0 += (int64_t)gridDim.x * per_pass) {
        T rv[kVecGroups][W], pv[kVecGroups][W], dv[kVecGroups][W];
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
                vload_h<NT>(r + g * W, rv[u]);
                vload_h<NT>(p + g * W, pv[u]);
                vload_h<NT>(dinv + g * W, dv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
#pragma unroll
                for (int k = 0; k < W; ++k)
                    pv[u][k] = (T)((double)dv[u][k] * (double)rv[u][k] + beta * (double)pv[u][k]);
                vstore_h<NT>(p + g * W, pv[u]);
            }
        }
    }
    if (blockIdx.x == 0 && tid < n - ng * W) {
        const int64_t i = ng * W + tid;
        p[i] = (T)((double)dinv[i] * (double)r[i] + beta * (double)p[i]);
    }
}

// End of a single-system folded solve: the steps no SpMV applied to x, in
// their order: for an odd count K of updates (the last SpMV skipped x),
// alpha2 p_(K-1) (in p[(K - 1) & 1]), then the last update's alpha p_K (the
// direction the last SpMV formed, p[K & 1]).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_fold_finish(int64_t n, T *__restrict__ x,
                                                        const T *__restrict__ p0,
                                                        const T *__restrict__ p1,
                                                        const SysState *__restrict__ st) {
    constexpr int W = VecW<T>::W;
    // pending: alpha p_K (K = st.iter, its direction in p[K & 1]) and, for
    // an odd K (the last SpMV did not update x), alpha2 p_(K-1) before it
    const int32_t K = st[0].iter;
    const double alpha = st[0].alpha, alpha2 = (K & 1) ? st[0].alpha2 : 0.0;
    if (alpha == 0.0 && alpha2 == 0.0) return;
    const T *p = (K & 1) ? p1 : p0;
    const T *pp = (K & 1) ? p0 : p1;
    auto upd = [&](T xv, T pv, T ppv) {
        if (alpha2 != 0.0) xv = (T)((double)xv + alpha2 * (double)ppv);
        if (alpha != 0.0) xv = (T)((double)xv + alpha * (double)pv);
        return xv;
    };
    const int tid = threadIdx.x;
    const int64_t ng = n / W;
    const int64_t per_pass = (int64_t)kBlock * kVecGroups;
    for (int64_t g0 = (int64_t)blockIdx.x * per_pass; g0 < ng; g0 += (int64_t)gridDim.x * per_pass) {
        T xv[kVecGroups][W], pv[kVecGroups][W], ppv[kVecGroups][W];
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
                vload(x + g * W, xv[u]);
                vload(p + g * W, pv[u]);
                if (alpha2 != 0.0) {
                    vload(pp + g * W, ppv[u]);
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) ppv[u][k] = (T)0;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kVecGroups; ++u) {
            const int64_t g = g0 + u * kBlock + tid;
            if (g < ng) {
#pragma unroll
                for (int k = 0; k < W; ++k) xv[u][k] = upd(xv[u][k], pv[u][k], ppv[u][k]);
                vstore(x + g * W, xv[u]);
            }
        }
    }
    if (blockIdx.x == 0 && tid < n - ng * W) {
        const int64_t i = ng * W + tid;
        x[i] = upd(x[i], p[i], alpha2 != 0.0 ? pp[i] : (T)0);
    }
}

// The same for a folded batch ([n][B], 16-byte groups of W systems): each
// system's last step x += alpha_b p, p = the newest direction buffer
// (p[fold_iter & 1]; stopped systems carried their last direction into it).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_fold_finish_bv(int64_t nc, int B, T *__restrict__ x,
                                                           const T *__restrict__ p0,
                                                           const T *__restrict__ p1,
                                                           const Ctl *__restrict__ ctl,
                                                           const SysState *__restrict__ st) {
    constexpr int W = VecW<T>::W;
    const int Q = B / W;
    const int t = threadIdx.x;
    const int s0 = (t & (Q - 1)) * W;
    double alpha[W];
    bool any = false;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        alpha[w] = st[s0 + w].alpha;
        any |= alpha[w] != 0.0;
    }
    if (!any) return;
    const T *p = (ctl->fold_iter & 1) ? p1 : p0;
    for (int64_t c = (int64_t)blockIdx.x * kBlock + t; c < nc; c += (int64_t)gridDim.x * kBlock) {
        T xv[W], pv[W];
        vload(x + c * W, xv);
        vload(p + c * W, pv);
#pragma unroll
        for (int w = 0; w < W; ++w)
            if (alpha[w] != 0.0) xv[w] = (T)((double)xv[w] + alpha[w] * (double)pv[w]);
        vstore(x + c * W, xv);
    }
}

// grid of the fused update + direction: one pass per workgroup, all of them
// resident at once; 0 when the system does not fit (or B > 1)
int64_t fused_grid(const Handle &h, int W) {
    if (h.B != 1 || h.nseg > 0 || !h.fuse_update || h.upd_dir_resident <= 0) return 0;
    const int64_t per = (int64_t)kBlock * kFusedGroups;
    int64_t g = (h.n / W + per - 1) / per;
    if (g < 1) g = 1;
    return g <= h.upd_dir_resident ? g : 0;
}

// grid of the batched fused update + direction (one pass per workgroup, all
// resident); 0 when it does not fit or fusion is off
int64_t fused_bv_grid(const Handle &h, int W) {
    if (h.B < 2 || h.nseg > 0 || !h.fuse_update || h.upd_dir_bv_resident <= 0) return 0;
    const int64_t nc = h.n * h.B / W;
    const int64_t per = (int64_t)kBlock * kBvFusedGroups;
    int64_t g = (nc + per - 1) / per;
    if (g < 1) g = 1;
    return g <= h.upd_dir_bv_resident ? g : 0;
}

// the per-step solve folds the direction into the SpMV: fp64 storage (z is
// stored, and in fp64 z = dinv r rounds once where the direction formed it
// anyway; in fp32 storage it would add an fp32 rounding per step), a single
// system on ring-form tiles without long rows or a batch of 16-byte lanes,
// where the fused update + direction kernel does not apply (too large for
// one resident pass, or switched off)
bool want_fold(const Handle &h) {
    if (!h.fold_direction || h.vt != SLA_F64 || !fold_possible(h)) return false;
    const int W = h.vt == SLA_F64 ? VecW<double>::W : VecW<float>::W;
    return h.B > 1 ? fused_bv_grid(h, W) == 0 : fused_grid(h, W) == 0;
}

int64_t vec1_grid(int64_t n, int W) {
    const int64_t per = (int64_t)kBlock * kVecGroups * W;
    int64_t g = (n + per - 1) / per;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g < 1) g = 1;
    return g;
}

// p = dinv r + beta p for systems still running
template <typename T>
__global__ __launch_bounds__(kBlock) void k_direction(int64_t n, int B, const T *__restrict__ r,
                                                      T *__restrict__ p, const T *__restrict__ dinv,
                                                      const Ctl *__restrict__ ctl,
                                                      const SysState *__restrict__ st) {
    if (ctl->n_running == 0) return;
    const Lanes L(B);
    if (!L.on || st[L.b].status != kRunning) return;
    const double beta = st[L.b].beta;
    const int64_t rows_pass = (int64_t)L.J * kVecItems;
    for (int64_t r0 = (int64_t)blockIdx.x * rows_pass; r0 < n; r0 += (int64_t)gridDim.x * rows_pass) {
        const int64_t fb = r0 * B;
        const T *rb = r + fb;
        const T *db = dinv + fb;
        T *pb = p + fb;
        const int64_t left = n - r0;
        T rv[kVecItems], pv[kVecItems], dv[kVecItems];
#pragma unroll
        for (int u = 0; u < kVecItems; ++u) {
            const int ii = u * L.J + L.jr;
            const int o = ii * B + L.b;
            const bool in = ii < left;
            rv[u] = in ? rb[o] : (T)0;
            pv[u] = in ? pb[o] : (T)0;
            dv[u] = in ? db[o] : (T)0;
        }
#pragma unroll
        for (int u = 0; u < kVecItems; ++u) {
            const int ii = u * L.J + L.jr;
            if (ii < left) pb[ii * B + L.b] = (T)((double)dv[u] * (double)rv[u] + beta * (double)pv[u]);
        }
    }
}

// grad[b][k] = sign * a[row(k)][b] * x[col(k)][b] over the short-row tiles:
// one wavefront per tile (no workgroup barrier), wavefronts striding over the
// tiles. The row of each entry comes from the tile's 16-bit row offsets
// through a per-wavefront LDS table, and narrow tiles read 16-bit columns.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_grad_tile(const TileDesc *__restrict__ tiles,
                                                      int64_t ntiles,
                                                      const uint16_t *__restrict__ roff16,
                                                      const int32_t *__restrict__ col,
                                                      const uint16_t *__restrict__ col16,
                                                      int64_t nnz, int B, const T *__restrict__ lam,
                                                      const T *__restrict__ x,
                                                      T *__restrict__ grad, double sign) {
    __shared__ uint16_t rowid_all[kWaves][kTileCap];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    uint16_t *rowid = rowid_all[wv];
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t t = (int64_t)blockIdx.x * kWaves + wv; t < ntiles; t += stride) {
        const TileDesc d = tiles[t];
        const int nrows = d.re - d.rs;
        const int nk = (int)(d.k1 - d.k0);
        const uint16_t *rp = roff16 + d.rpos;
        for (int j = lane; j < nrows; j += 64) {
            const int a = rp[j], e = rp[j + 1];
            for (int k = a; k < e; ++k) rowid[k] = (uint16_t)j;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int kk = lane; kk < nk; kk += 64) {
            const int64_t i = d.rs + rowid[kk];
            const int64_t k = d.k0 + kk;
            const int64_t c = d.narrow ? (int64_t)d.cbase + col16[k] : (int64_t)col[k];
            for (int b = 0; b < B; ++b)
                grad[(int64_t)b * nnz + k] =
                    (T)(sign * ((double)lam[i * B + b] * (double)x[c * B + b]));
        }
        // the next tile's table is written after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// The same gradient, single system, over tiles in the ring form of the tile
// SpMV (every tile narrow; entries from k0 rounded down to a multiple of 4 up
// to k1 at most 256; at most 63 rows): lane l owns the 4-entry group 4 l, and
// each entry's lambda comes from a per-wavefront LDS table that the lanes of
// the tile's rows fill over their entry ranges. A tile's packed columns, row
// offsets and lambda of its rows are issued kGradRing tiles ahead and its x
// gathers two tiles ahead, so that each wait leaves the later tiles' loads
// in flight (memory operations complete in issue order); the stores of a
// tile go out before the loads it refills. Lanes whose group lies inside the
// tile store it whole, past the caches; the group a tile shares with its
// neighbour is stored through them, so that L2 merges its line. The walk
// over the tiles (a contiguous share per XCD, band-aligned when the band
// fits the grid) is the ring SpMV's. Same values as k_grad_tile, bit for
// bit. On the 133M-row Poisson matrix (5.3 GB of gradient) it took 2.21 ms
// against 3.13 for k_grad_tile (one run); streaming the whole-group stores
// took it from 2.80 to 2.48 ms (another run), while six or eight slots with
// gathers three or four tiles ahead, or eight workgroups per CU, were no
// faster.
constexpr int kGradRing = 4;
// four values as streaming (non-temporal) stores: the gradient is written
// once and not read back by the kernel, so its lines need not displace the
// gathered x and lambda in the caches
typedef double sla_d2 __attribute__((ext_vector_type(2)));
typedef float sla_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store4_stream(double *p, const double (&v)[4]) {
    const sla_d2 a = {v[0], v[1]}, b = {v[2], v[3]};
    __builtin_nontemporal_store(a, reinterpret_cast<sla_d2 *>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<sla_d2 *>(p) + 1);
}
__device__ __forceinline__ void store4_stream(float *p, const float (&v)[4]) {
    const sla_f4 a = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(a, reinterpret_cast<sla_f4 *>(p));
}
// unused LDS at launch so that the fp64 and fp32 forms both hold four
// workgroups per CU (static LDS 8 or 4 KB), the grid the band walk is cut for
constexpr size_t kGradLdsPad = 30 * 1024;

template <typename T>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_grad_ring(
    const TileDesc *__restrict__ tiles, int64_t ntiles, const uint16_t *__restrict__ roff16,
    const uint16_t *__restrict__ col16, const T *__restrict__ lam, const T *__restrict__ x,
    T *__restrict__ grad, double sign, int vec_store, int64_t band_l, int32_t band_p) {
    __shared__ __align__(16) T lt_all[kWaves][4 * 64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    T *lt = lt_all[wv];
    const int xcd = blockIdx.x % kXcds;
    int64_t stride = (int64_t)(gridDim.x / kXcds) * kWaves;
    const int64_t wid = (int64_t)(blockIdx.x / kXcds) * kWaves + wv;
    int64_t t_next = ntiles * xcd / kXcds + wid;
    int64_t t_end = ntiles * (xcd + 1) / kXcds;
    if (band_l > 0 && band_l * band_p == stride) {
        const int64_t T0 = t_next - wid, T1 = t_end;
        const int64_t panel = wid / band_l, colw = wid - panel * band_l;
        t_next = T0 + (T1 - T0) * panel / band_p + colw;
        t_end = T0 + (T1 - T0) * (panel + 1) / band_p;
        stride = band_l;
    }
    // slot u: tile, descriptor fields, the lane's packed 16-bit columns, row
    // offset and lambda; gather buffer h: x at the slot's columns
    int64_t s_t[kGradRing], s_base[kGradRing];
    int32_t s_nr[kGradRing], s_nk[kGradRing], s_shift[kGradRing], s_cb[kGradRing];
    uint2 s_c[kGradRing];
    int32_t s_ro[kGradRing];
    T s_l[kGradRing];
    double xv[2][4];
    TileDesc dn{0, 0, 0, 0, 0, 0, 0};
    if (t_next < t_end) dn = tiles[t_next];
    // Every load is issued by every lane, at a clamped offset where the lane
    // has nothing to load (past the end: an empty tile reading entry 0, row 0
    // and offset 0; the entry arrays are padded past nnz). What clamped lanes
    // load is never stored.
    auto fetch = [&](int u) {
        s_t[u] = t_next;
        TileDesc e{0, 0, 0, 0, 0, 0, 0};
        if (t_next < t_end) e = dn;
        const int nr = e.re - e.rs;
        s_nr[u] = nr;
        s_nk[u] = (int)(e.k1 - e.k0);
        s_shift[u] = (int)(e.k0 & 3);
        s_cb[u] = e.cbase;
        const int64_t base = e.k0 & ~(int64_t)3;
        s_base[u] = base;
        const int span = (int)(e.k1 - base);
        const int g = 4 * lane < span ? 4 * lane : 0;
        s_c[u] = *reinterpret_cast<const uint2 *>(col16 + base + g);
        s_ro[u] = (int32_t)roff16[e.rpos + (lane <= nr ? lane : nr)];
        s_l[u] = lam[e.rs + (lane < nr ? lane : 0)];
        if (t_next < t_end) t_next += stride;
    };
    auto load_desc = [&]() {
        if (t_next < t_end) dn = tiles[t_next];
    };
    auto gather = [&](int u, int hb) {
        const int shift = s_shift[u], nk = s_nk[u], cb = s_cb[u];
        const uint32_t raw[2] = {s_c[u].x, s_c[u].y};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = 4 * lane + k - shift;
            const int32_t c = cb + (int32_t)((raw[k >> 1] >> (16 * (k & 1))) & 0xffffu);
            xv[hb][k] = (double)x[(j >= 0 && j < nk) ? c : 0];
        }
    };
    auto step = [&](int u, int hb) {
        const int nrows = s_nr[u], shift = s_shift[u], nk = s_nk[u];
        // row r's entry slots are [roff[r], roff[r + 1]) + shift; lane r + 1
        // holds roff[r + 1] (lane nrows the end)
        const int a = s_ro[u] + shift;
        const int b = __shfl_down(s_ro[u], 1, 64) + shift;
        if (lane < nrows)
            for (int j = a; j < b; ++j) lt[j] = s_l[u];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        T l4[4];
        load4(lt + 4 * lane, l4);
        T gv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) gv[k] = (T)(sign * ((double)l4[k] * xv[hb][k]));
        const int j0 = 4 * lane - shift;
        T *gp = grad + s_base[u] + 4 * lane;
        if (vec_store && j0 >= 0 && j0 + 3 < nk) {
            store4_stream(gp, gv);
        } else {
            // the group shared with a neighbouring tile: cached stores, so
            // that its line is merged in L2 rather than written twice
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (j0 + k >= 0 && j0 + k < nk) gp[k] = gv[k];
        }
        fetch(u);
        gather((u + 2) % kGradRing, hb);
        load_desc();
        // the next tile's table is written after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if (t_next < t_end) {
#pragma unroll
        for (int u = 0; u < kGradRing; ++u) {
            fetch(u);
            load_desc();
        }
        gather(0, 0);
        gather(1, 1);
        // four steps per pass while all four slots hold a tile (one path
        // through the loop body keeps the waits for the in-order counter
        // tight), then the at most three tiles left
        while (s_t[3] < t_end) {
            step(0, 0);
            step(1, 1);
            step(2, 0);
            step(3, 1);
        }
        if (s_t[0] < t_end) {
            step(0, 0);
            if (s_t[1] < t_end) {
                step(1, 1);
                if (s_t[2] < t_end) step(2, 0);
            }
        }
    }
}

// resident workgroups of k_grad_ring<T> on a device (computed once per device)
template <typename T>
int64_t grad_ring_resident(int device) {
    constexpr int kDevs = 64;
    static std::atomic<int64_t> cache[kDevs];
    if (device < 0 || device >= kDevs)
        return resident_workgroups((const void *)&k_grad_ring<T>, device, kGradLdsPad);
    int64_t r = cache[device].load(std::memory_order_relaxed);
    if (r == 0) {
        r = resident_workgroups((const void *)&k_grad_ring<T>, device, kGradLdsPad);
        cache[device].store(r, std::memory_order_relaxed);
    }
    return r;
}

// W consecutive values of a row of an internal [n][B] vector: 16 bytes
// (16-byte aligned) or one value
__device__ __forceinline__ void loadw(const float *p, float (&o)[4]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void loadw(const double *p, double (&o)[2]) {
    const double2 a = *reinterpret_cast<const double2 *>(p);
    o[0] = a.x; o[1] = a.y;
}
template <typename T>
__device__ __forceinline__ void loadw(const T *p, T (&o)[1]) {
    o[0] = *p;
}

// The same gradient for a batch (lambda and x in the internal [n][B]
// layout), in blocks of W systems: W = 16 / sizeof(T) when B is a multiple
// of it, else 1. Lanes are (entry e of a run of EL consecutive entries,
// block q of W systems), so one load brings W systems of x at the entry's
// column (and of lambda at its row), a load instruction touches at most EL
// cache lines (against 64 when each lane gathers one system of its own
// entry), and the EL lanes of a block write EL consecutive entries of each
// of its W gradient planes. A wavefront takes one (tile, pass) pair, pass h
// covering blocks h QL .. h QL + QL - 1, so that a batch gives NQ / QL times
// as many wavefronts as tiles; entries go four runs at a time (loads first).
// Same values as k_grad_tile, bit for bit.
template <typename T, int QLOG, int W>
__global__ __launch_bounds__(kBlock) void k_grad_tile_bq(const TileDesc *__restrict__ tiles,
                                                         int64_t ntiles,
                                                         const uint16_t *__restrict__ roff16,
                                                         const int32_t *__restrict__ col,
                                                         const uint16_t *__restrict__ col16,
                                                         int64_t nnz, int B, const T *__restrict__ lam,
                                                         const T *__restrict__ x,
                                                         T *__restrict__ grad, double sign) {
    constexpr int QL = 1 << QLOG;
    constexpr int EL = 64 / QL;
    constexpr int U = 4;
    __shared__ uint16_t rowid_all[kWaves][kTileCap];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    uint16_t *rowid = rowid_all[wv];
    const int e = lane & (EL - 1);
    const int qq = lane / EL;
    const int NQ = B / W;
    const int NP = (NQ + QL - 1) / QL;
    const int64_t nv = ntiles * NP;
    const int64_t stride = (int64_t)gridDim.x * kWaves;
    for (int64_t v = (int64_t)blockIdx.x * kWaves + wv; v < nv; v += stride) {
        const int64_t t = v / NP;
        const int q = (int)(v - t * NP) * QL + qq;
        const TileDesc d = tiles[t];
        const int nrows = d.re - d.rs;
        const int nk = (int)(d.k1 - d.k0);
        const uint16_t *rp = roff16 + d.rpos;
        for (int j = lane; j < nrows; j += 64) {
            const int a = rp[j], b = rp[j + 1];
            for (int k = a; k < b; ++k) rowid[k] = (uint16_t)j;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (q < NQ) {
            const T *xq = x + q * W;
            const T *lq = lam + q * W;
            T *gq = grad + (int64_t)q * W * nnz + d.k0;
            for (int kb = 0; kb < nk; kb += U * EL) {
                T xv[U][W], lv[U][W];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // past the tile's end: entry 0's row and column (not stored)
                    const int kk = kb + u * EL + e < nk ? kb + u * EL + e : 0;
                    const int64_t k = d.k0 + kk;
                    const int64_t c = d.narrow ? (int64_t)d.cbase + col16[k] : (int64_t)col[k];
                    const int64_t i = d.rs + rowid[kk];
                    loadw(xq + c * B, xv[u]);
                    loadw(lq + i * B, lv[u]);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int kk = kb + u * EL + e;
                    if (kk < nk) {
#pragma unroll
                        for (int j = 0; j < W; ++j)
                            gq[(int64_t)j * nnz + kk] =
                                (T)(sign * ((double)lv[u][j] * (double)xv[u][j]));
                    }
                }
            }
        }
        // the next pair's table is written after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// the same for rows longer than kLongRow, one workgroup per row
template <typename T, typename RP>
__global__ __launch_bounds__(kBlock) void k_grad_long(const int32_t *__restrict__ long_rows,
                                                      const RP *__restrict__ row_ptr,
                                                      const int32_t *__restrict__ col, int64_t nnz,
                                                      int B, const T *__restrict__ lam,
                                                      const T *__restrict__ x,
                                                      T *__restrict__ grad, double sign) {
    const int64_t i = long_rows[blockIdx.x];
    const int64_t k0 = row_ptr[i], k1 = row_ptr[i + 1];
    for (int b = 0; b < B; ++b) {
        const double li = (double)lam[i * B + b];
        for (int64_t k = k0 + threadIdx.x; k < k1; k += kBlock)
            grad[(int64_t)b * nnz + k] = (T)(sign * (li * (double)x[(int64_t)col[k] * B + b]));
    }
}


template <typename T>
void iter_kernels_t(Handle &h, hipStream_t s, Launcher *lp) {
    const int64_t g = vec_grid(h.n, h.B);
    hipEvent_t a = nullptr;
    if (h.fold_active) {
        // direction folded into the SpMV; the update stores z, not x
        if (lp) lp->begin(SLA_KERNEL_SPMV_DOT, &a);
        launch_spmv_fold(h, s);
        if (lp) lp->end(SLA_KERNEL_SPMV_DOT, a);
        if (lp) lp->begin(SLA_KERNEL_UPDATE, &a);
        const Red red{h.part, h.gpart, h.sync + kCntUpdate * kCountersPerKind};
        if (h.B > 1) {
            const int64_t nc = h.n * h.B / VecW<T>::W;
            hipLaunchKernelGGL((k_update_bv<T, true>), dim3((unsigned)bv_grid(nc, h.bv_update_resident)),
                               dim3(kBlock), 0, s, nc, h.B, (T *)h.fold_z, (T *)h.r,
                               (const T *)nullptr, (const T *)h.q, (const T *)h.dinv,
                               (const double *)h.gpart_spmv, bvec_spmv_blocks(h), red, h.ctl,
                               h.st, h.d_running);
            SLA_HIP(hipGetLastError());
            if (lp) lp->end(SLA_KERNEL_UPDATE, a);
            return;
        }
        const int64_t g1 = vec1_grid(h.n, VecW<T>::W);
        const bool nt = h.n * (int64_t)sizeof(T) >= kNtVectorBytes;
        hipLaunchKernelGGL((nt ? k_update1<T, true, true> : k_update1<T, false, true>),
                           dim3((unsigned)g1), dim3(kBlock), 0, s, h.n, (T *)h.fold_z, (T *)h.r,
                           (const T *)nullptr, (const T *)h.q, (const T *)h.dinv,
                           (const double *)h.spart, spmv_blocks(h), red, h.ctl, h.st, h.d_running);
        SLA_HIP(hipGetLastError());
        if (lp) lp->end(SLA_KERNEL_UPDATE, a);
        return;
    }
    if (lp) lp->begin(SLA_KERNEL_SPMV_DOT, &a);
    launch_spmv_dot(h, s);
    if (lp) lp->end(SLA_KERNEL_SPMV_DOT, a);
    if (lp) lp->begin(SLA_KERNEL_UPDATE, &a);
    const Red red{h.part, h.gpart, h.sync + kCntUpdate * kCountersPerKind};
    const int64_t gf = fused_grid(h, VecW<T>::W);
    if (gf > 0) {
        hipLaunchKernelGGL(k_update_dir1<T>, dim3((unsigned)gf), dim3(kBlock), 0, s, h.n, (T *)h.x,
                           (T *)h.r, (T *)h.p, (const T *)h.q, (const T *)h.dinv,
                           (const double *)h.spart, spmv_blocks(h), red, h.ctl, h.st, h.d_running,
                           h.bcast);
        SLA_HIP(hipGetLastError());
        if (lp) lp->end(SLA_KERNEL_UPDATE, a);
        return;
    }
    if (h.B == 1) {
        const int64_t g1 = vec1_grid(h.n, VecW<T>::W);
        const bool nt = h.n * (int64_t)sizeof(T) >= kNtVectorBytes;
        hipLaunchKernelGGL((nt ? k_update1<T, true> : k_update1<T, false>), dim3((unsigned)g1),
                           dim3(kBlock), 0, s, h.n, (T *)h.x,
                           (T *)h.r, (const T *)h.p, (const T *)h.q, (const T *)h.dinv,
                           (const double *)h.spart, spmv_blocks(h), red, h.ctl, h.st, h.d_running);
    } else if (bv_ok<T>(h) && fused_bv_grid(h, VecW<T>::W) > 0) {
        const int64_t nc = h.n * h.B / VecW<T>::W;
        hipLaunchKernelGGL(k_update_dir_bv<T>, dim3((unsigned)fused_bv_grid(h, VecW<T>::W)),
                           dim3(kBlock), 0, s, nc, h.B, (T *)h.x, (T *)h.r, (T *)h.p,
                           (const T *)h.q, (const T *)h.dinv, (const double *)h.gpart_spmv,
                           bvec_spmv_blocks(h), red, h.ctl, h.st, h.d_running, h.bcast,
                           h.bcast_bv);
        SLA_HIP(hipGetLastError());
        if (lp) lp->end(SLA_KERNEL_UPDATE, a);
        return;
    } else if (bv_ok<T>(h)) {
        const int64_t nc = h.n * h.B / VecW<T>::W;
        hipLaunchKernelGGL(k_update_bv<T>, dim3((unsigned)bv_grid(nc, h.bv_update_resident)),
                           dim3(kBlock), 0, s, nc,
                           h.B, (T *)h.x, (T *)h.r, (const T *)h.p, (const T *)h.q,
                           (const T *)h.dinv, (const double *)h.gpart_spmv, bvec_spmv_blocks(h),
                           red, h.ctl, h.st, h.d_running);
    } else {
        hipLaunchKernelGGL(k_update<T>, dim3((unsigned)g), dim3(kBlock), 0, s, h.n, h.B, (T *)h.x,
                           (T *)h.r, (const T *)h.p, (const T *)h.q, (const T *)h.dinv, red, h.ctl,
                           h.st, h.d_running);
    }
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_UPDATE, a);
    if (lp) lp->begin(SLA_KERNEL_DIRECTION, &a);
    if (h.B == 1) {
        const int64_t g1 = vec1_grid(h.n, VecW<T>::W);
        const bool nt = h.n * (int64_t)sizeof(T) >= kNtVectorBytes;
        hipLaunchKernelGGL((nt ? k_direction1<T, true> : k_direction1<T, false>), dim3((unsigned)g1),
                           dim3(kBlock), 0, s, h.n,
                           (const T *)h.r, (T *)h.p, (const T *)h.dinv, (const Ctl *)h.ctl,
                           (const SysState *)h.st);
    } else if (bv_ok<T>(h)) {
        const int64_t nc = h.n * h.B / VecW<T>::W;
        hipLaunchKernelGGL(k_direction_bv<T>, dim3((unsigned)bv_grid(nc, h.bv_direction_resident)),
                           dim3(kBlock), 0, s, nc,
                           h.B, (const T *)h.r, (T *)h.p, (const T *)h.dinv, (const Ctl *)h.ctl,
                           (const SysState *)h.st);
    } else {
        hipLaunchKernelGGL(k_direction<T>, dim3((unsigned)g), dim3(kBlock), 0, s, h.n, h.B,
                           (const T *)h.r, (T *)h.p, (const T *)h.dinv, (const Ctl *)h.ctl,
                           (const SysState *)h.st);
    }
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_DIRECTION, a);
}

void iter_kernels(Handle &h, hipStream_t s, Launcher *lp) {
    if (h.nseg > 0) {
        seg_iter_kernels(h, s, lp);
        return;
    }
    if (h.vt == SLA_F64) iter_kernels_t<double>(h, s, lp);
    else iter_kernels_t<float>(h, s, lp);
}

void ensure_graph(Handle &h) {
    if (h.graph && h.graph_k == h.check_k) return;
    if (h.graph) {
        SLA_HIP(hipGraphExecDestroy(h.graph));
        h.graph = nullptr;
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
    h.graph = ex;
    h.graph_k = h.check_k;
}

template <typename T>
void init_t(Handle &h, const void *b_int, hipStream_t s, Launcher *lp) {
    const int64_t g = vec_grid(h.n, h.B);
    hipEvent_t a = nullptr;
    if (lp) lp->begin(SLA_KERNEL_INIT, &a);
    const Red red{h.part, h.gpart, h.sync + kCntInit * kCountersPerKind};
    hipLaunchKernelGGL(k_init<T>, dim3((unsigned)g), dim3(kBlock), 0, s, h.n, h.B, (const T *)b_int,
                       (T *)h.x, (T *)h.r, (T *)h.p, (const T *)h.dinv,
                       (T *)(h.fold_active ? h.fold_z : nullptr), red, h.ctl, h.st, h.d_running);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_INIT, a);
}

}  // namespace

void init_vector_limits(Handle &h) {
    if (h.B > 1)
        h.upd_dir_bv_resident = resident_workgroups(
            h.vt == SLA_F64 ? (const void *)&k_update_dir_bv<double>
                            : (const void *)&k_update_dir_bv<float>,
            h.device);
    if (h.B == 1) {
        h.upd_dir_resident = resident_workgroups(
            h.vt == SLA_F64 ? (const void *)&k_update_dir1<double> : (const void *)&k_update_dir1<float>,
            h.device);
        return;
    }
    if (h.vt == SLA_F64) {
        h.bv_update_resident = resident_workgroups((const void *)&k_update_bv<double>, h.device);
        h.bv_direction_resident = resident_workgroups((const void *)&k_direction_bv<double>, h.device);
    } else {
        h.bv_update_resident = resident_workgroups((const void *)&k_update_bv<float>, h.device);
        h.bv_direction_resident = resident_workgroups((const void *)&k_direction_bv<float>, h.device);
    }
}

// The general per-step kernels (fp64, one system) on caller-given buffers,
// for the allocation-free solve: every pointer is device memory, the
// reductions' partials, group sums and arrival counters come in `red` (the
// counters zero), `running` is device memory that receives the number of
// systems still running.
void launch_init_raw(int64_t n, const double *b, double *x, double *r, double *p,
                     const double *dinv, Red red, Ctl *ctl, SysState *st, int32_t *running,
                     hipStream_t s) {
    hipLaunchKernelGGL(k_init<double>, dim3((unsigned)vec_grid(n, 1)), dim3(kBlock), 0, s, n, 1, b,
                       x, r, p, dinv, (double *)nullptr, red, ctl, st, running);
    SLA_HIP(hipGetLastError());
}

void launch_update_raw(int64_t n, double *x, double *r, const double *p, const double *q,
                       const double *dinv, Red red, Ctl *ctl, SysState *st, int32_t *running,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_update<double>, dim3((unsigned)vec_grid(n, 1)), dim3(kBlock), 0, s, n, 1,
                       x, r, p, q, dinv, red, ctl, st, running);
    SLA_HIP(hipGetLastError());
}

void launch_direction_raw(int64_t n, const double *r, double *p, const double *dinv,
                          const Ctl *ctl, const SysState *st, hipStream_t s) {
    hipLaunchKernelGGL(k_direction<double>, dim3((unsigned)vec_grid(n, 1)), dim3(kBlock), 0, s, n, 1,
                       r, p, dinv, ctl, st);
    SLA_HIP(hipGetLastError());
}

// workgroups of those kernels (the rows of their partial tables)
int64_t raw_vec_grid(int64_t n) { return vec_grid(n, 1); }

void flush_profile(Handle &h) {
    for (auto &rec : h.pending) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, rec.a, rec.b) == hipSuccess) {
            h.prof_launches[rec.kind] += 1;
            h.prof_ms[rec.kind] += ms;
        }
        (void)hipEventDestroy(rec.a);
        (void)hipEventDestroy(rec.b);
    }
    h.pending.clear();
}

void spmv(Handle &h, const void *x, void *y, hipStream_t s) {
    Launcher L{h, s, h.profile};
    hipEvent_t a = nullptr;
    if (h.B == 1) {
        L.begin(SLA_KERNEL_SPMV, &a);
        launch_spmv_plain(h, x, y, s);
        L.end(SLA_KERNEL_SPMV, a);
    } else {
        transpose(x, h.p, h.B, h.n, h.vbytes, s);
        L.begin(SLA_KERNEL_SPMV, &a);
        launch_spmv_plain(h, h.p, h.q, s);
        L.end(SLA_KERNEL_SPMV, a);
        transpose(h.q, y, h.n, h.B, h.vbytes, s);
    }
    if (h.profile) {
        SLA_HIP(hipStreamSynchronize(s));
        flush_profile(h);
    }
}

// y = A x for a batch whose x is already in the internal [n][B] layout (not
// h.p, which takes the product) and y in the caller's [B][n]
void spmv_from_internal(Handle &h, const void *x_int, void *y, hipStream_t s) {
    Launcher L{h, s, h.profile};
    hipEvent_t a = nullptr;
    L.begin(SLA_KERNEL_SPMV, &a);
    launch_spmv_plain(h, x_int, h.p, s);
    L.end(SLA_KERNEL_SPMV, a);
    transpose(h.p, y, h.n, h.B, h.vbytes, s);
}

namespace {

// One attempt at a solve (see pcg). Returns false, having done nothing the
// caller can see, when a bounded grid-wide wait gave up; with allow_resident
// false the single-kernel solve is not tried.
bool pcg_attempt(Handle &h, const void *b_user, void *x_user, double tol, int32_t maxit,
                 sla_info *info, hipStream_t s, bool keep_internal_solution, bool allow_resident) {
    Launcher L{h, s, h.profile};
    Launcher *lp = h.profile ? &L : nullptr;
    // control block: tolerance and budget (the counters stay zero between launches)
    h.h_ctl->tol = tol;
    h.h_ctl->maxit = maxit;
    h.h_ctl->n_running = 0;
    h.h_ctl->epoch = ++h.epoch;
    h.h_ctl->error = 0;
    h.h_ctl->spin_limit = h.spin_limit;
    h.h_ctl->fold_iter = 0;
    SLA_HIP(hipMemcpyAsync(h.ctl, h.h_ctl, sizeof(Ctl), hipMemcpyHostToDevice, s));
    // the whole solve in one cooperative kernel (same recurrence; a batch
    // leaves x as [B][n] in q), unless the cooperative launch is refused
    // (see resident_solve): then the per-step kernels
    if (allow_resident && h.nseg == 0 && resident_ready(h, s)) {
        if (resident_solve(h, b_user, h.B == 1 ? h.x : h.q, tol, maxit, s)) {
            // (if a wait gave up, the re-run overwrites what is copied here)
            const size_t bytes = (size_t)h.n * h.B * h.vbytes;
            if (h.B == 1) {
                if (!keep_internal_solution)
                    SLA_HIP(hipMemcpyAsync(x_user, h.x, bytes, hipMemcpyDeviceToDevice, s));
            } else if (keep_internal_solution) {
                transpose(h.q, h.x, h.B, h.n, h.vbytes, s);
            } else {
                SLA_HIP(hipMemcpyAsync(x_user, h.q, bytes, hipMemcpyDeviceToDevice, s));
            }
            SLA_HIP(hipMemcpyAsync(h.h_state, h.st, sizeof(SysState) * h.B, hipMemcpyDeviceToHost,
                                   s));
            SLA_HIP(hipStreamSynchronize(s));
            if (h.profile) flush_profile(h);
            for (int b = 0; b < h.B; ++b) {
                const int32_t stb = h.h_state[b].status;
                if (stb != kRunning && (stb < 0 || stb > SLA_BREAKDOWN)) {
                    // a grid-wide wait gave up (workgroups not all running)
                    h.last_fallback |= kFallbackWaitTimedOut;
                    return false;
                }
            }
            for (int b = 0; b < h.B; ++b) {
                const SysState &st = h.h_state[b];
                info[b].iterations = st.iter;
                info[b].status = st.status == kRunning ? SLA_MAXIT : st.status;
                info[b].rel_residual = st.bb == 0.0 ? 0.0 : sqrt(st.rr / st.bb);
            }
            h.last_path = kPathSingleKernel;
            return true;
        }
        h.last_fallback |= kFallbackCoopRefused;
    }
    const void *b_int = b_user;
    if (h.B > 1) {
        transpose(b_user, h.q, h.B, h.n, h.vbytes, s);  // q is free until the first SpMV
        b_int = h.q;
    }
    h.fold_active = want_fold(h);
    if (h.fold_active && !h.fold_z) {
        h.fold_z = dalloc(h, (size_t)h.n * h.B * h.vbytes);
        h.fold_p2 = dalloc(h, (size_t)h.n * h.B * h.vbytes);
    }
    if (h.nseg > 0) seg_init(h, b_int, s, lp);
    else if (h.vt == SLA_F64) init_t<double>(h, b_int, s, lp);
    else init_t<float>(h, b_int, s, lp);

    const bool graph = h.use_graph && !h.profile;
    if (graph) ensure_graph(h);
    const int64_t k = h.check_k;
    const int64_t max_chunks = maxit <= 0 ? 0 : (maxit + k - 1) / k;
    for (int64_t ch = 0; ch < max_chunks; ++ch) {
        if (graph) {
            SLA_HIP(hipGraphLaunch(h.graph, s));
        } else {
            for (int64_t j = 0; j < k; ++j) iter_kernels(h, s, lp);
        }
        SLA_HIP(hipEventRecord(h.ev[ch & 1], s));
        // poll the block before this one while this one runs (the GPU never idles)
        if (ch >= 1) {
            SLA_HIP(hipEventSynchronize(h.ev[(ch - 1) & 1]));
            if (__atomic_load_n(h.h_running, __ATOMIC_ACQUIRE) == 0) break;
        }
    }
    if (h.fold_active && h.B > 1) {
        const int W = h.vt == SLA_F64 ? VecW<double>::W : VecW<float>::W;
        const int64_t nc = h.n * h.B / W;
        int64_t gb = (nc + kBlock - 1) / kBlock;
        if (gb > kMaxGrid) gb = kMaxGrid;
        if (h.vt == SLA_F64)
            hipLaunchKernelGGL(k_fold_finish_bv<double>, dim3((unsigned)gb), dim3(kBlock), 0, s, nc,
                               h.B, (double *)h.x, (const double *)h.p, (const double *)h.fold_p2,
                               (const Ctl *)h.ctl, (const SysState *)h.st);
        else
            hipLaunchKernelGGL(k_fold_finish_bv<float>, dim3((unsigned)gb), dim3(kBlock), 0, s, nc,
                               h.B, (float *)h.x, (const float *)h.p, (const float *)h.fold_p2,
                               (const Ctl *)h.ctl, (const SysState *)h.st);
        SLA_HIP(hipGetLastError());
    } else if (h.fold_active) {
        const int W = h.vt == SLA_F64 ? VecW<double>::W : VecW<float>::W;
        const unsigned gf = (unsigned)vec1_grid(h.n, W);
        if (h.vt == SLA_F64)
            hipLaunchKernelGGL(k_fold_finish<double>, dim3(gf), dim3(kBlock), 0, s, h.n,
                               (double *)h.x, (const double *)h.p, (const double *)h.fold_p2,
                               (const SysState *)h.st);
        else
            hipLaunchKernelGGL(k_fold_finish<float>, dim3(gf), dim3(kBlock), 0, s, h.n,
                               (float *)h.x, (const float *)h.p, (const float *)h.fold_p2,
                               (const SysState *)h.st);
        SLA_HIP(hipGetLastError());
    }
    if (!keep_internal_solution) {
        // (if a wait gave up, the re-run overwrites what is copied here)
        if (h.B == 1)
            SLA_HIP(hipMemcpyAsync(x_user, h.x, (size_t)h.n * h.vbytes, hipMemcpyDeviceToDevice, s));
        else
            transpose(h.x, x_user, h.n, h.B, h.vbytes, s);
    }
    const int32_t nsys = num_systems(h);
    SLA_HIP(hipMemcpyAsync(h.h_state, h.st, sizeof(SysState) * nsys, hipMemcpyDeviceToHost, s));
    SLA_HIP(hipMemcpyAsync(h.h_ctl, h.ctl, sizeof(Ctl), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    if (h.profile) flush_profile(h);
    if (h.h_ctl->error) {
        // the fused update's broadcast wait gave up: its workgroups are not
        // all running at once on this GPU now. The handle keeps to the two
        // kernels without grid-wide waits from here on (SLA_OPT_FUSED_UPDATE
        // turns the fused form back on).
        h.last_fallback |= kFallbackWaitTimedOut;
        h.fuse_update = false;
        if (h.graph) (void)hipGraphExecDestroy(h.graph);
        h.graph = nullptr;
        h.graph_k = 0;
        return false;
    }
    for (int b = 0; b < nsys; ++b) {
        const SysState &st = h.h_state[b];
        info[b].iterations = st.iter;
        info[b].status = st.status == kRunning ? SLA_MAXIT : st.status;
        info[b].rel_residual = st.bb == 0.0 ? 0.0 : sqrt(st.rr / st.bb);
    }
    h.last_path = kPathPerStep;
    return true;
}

}  // namespace

// Solve A x = b for every system. b_user / x_user are [B][n]. With
// keep_internal_solution the iterate stays in h.x (internal layout) and
// x_user may be null. The single-kernel solve and the fused update wait for
// other workgroups, with bounded waits; if a wait gives up (the GPU shared
// with other work, so that not all workgroups run at once), the solve is
// run again from the start without that kernel: first the per-step kernels,
// then, if the fused update's wait gives up too, the unfused ones, which
// never wait on other workgroups. h.last_path and h.last_fallback record
// what ran.
void pcg(Handle &h, const void *b_user, void *x_user, double tol, int32_t maxit, sla_info *info,
         hipStream_t s, bool keep_internal_solution) {
    h.last_path = kPathNone;
    h.last_fallback = 0;
    if (pcg_attempt(h, b_user, x_user, tol, maxit, info, s, keep_internal_solution, true)) return;
    if (pcg_attempt(h, b_user, x_user, tol, maxit, info, s, keep_internal_solution, false)) return;
    if (pcg_attempt(h, b_user, x_user, tol, maxit, info, s, keep_internal_solution, false)) return;
    fail(SLA_ERR_HIP, "a grid-wide wait gave up on a path that has none");
}

// grad [B][nnz] (CSR order) from lambda (internal layout, h.x) and the
// forward solution x_user [B][n].
void grad_vals(Handle &h, const void *lam_internal, const void *x_user, void *grad, hipStream_t s,
               double sign) {
    if (h.nnz == 0) return;
    Launcher L{h, s, h.profile};
    const void *x_int = x_user;
    if (h.B > 1) {
        transpose(x_user, h.p, h.B, h.n, h.vbytes, s);
        x_int = h.p;
    }
    hipEvent_t a = nullptr;
    L.begin(SLA_KERNEL_GRAD, &a);
    auto go = [&](auto ttag, auto rtag) {
        using T = decltype(ttag);
        using RP = decltype(rtag);
        if (h.ntiles > 0 && h.B == 1 && h.all_narrow && h.ring_tiles && h.spmv_ring) {
            int64_t g = (h.ntiles + kWaves - 1) / kWaves;
            g = (g + kXcds - 1) / kXcds * kXcds;
            const int64_t res = grad_ring_resident<T>(h.device);
            if (g > res) g = res;
            // band-aligned tiles: band_l wavefronts per XCD walk its whole
            // range band by band (one panel, as the ring SpMV does)
            if (h.band_l > 0 && h.band_l % kWaves == 0 && g % kXcds == 0 &&
                g / kXcds * kWaves > h.band_l)
                g = h.band_l / kWaves * kXcds;
            const int vec = ((uintptr_t)grad % 16) == 0;
            hipLaunchKernelGGL(k_grad_ring<T>, dim3((unsigned)g), dim3(kBlock), kGradLdsPad, s,
                               (const TileDesc *)h.tiles, h.ntiles, (const uint16_t *)h.roff16,
                               (const uint16_t *)h.col16, (const T *)lam_internal,
                               (const T *)x_int, (T *)grad, sign, vec, h.band_l, h.band_p);
        } else if (h.ntiles > 0 && h.B > 1) {
            constexpr int W16 = 16 / (int)sizeof(T);
            const bool wide = h.B % W16 == 0;
            const int nq = wide ? h.B / W16 : h.B;
            const int qlog = nq >= 4 ? 2 : nq >= 2 ? 1 : 0;
            const int np = (nq + (1 << qlog) - 1) >> qlog;
            int64_t g = (h.ntiles * np + kWaves - 1) / kWaves;
            if (g > 4 * kMaxGrid) g = 4 * kMaxGrid;
            auto kern = wide ? (qlog == 2   ? k_grad_tile_bq<T, 2, W16>
                                : qlog == 1 ? k_grad_tile_bq<T, 1, W16>
                                            : k_grad_tile_bq<T, 0, W16>)
                             : (qlog == 2 ? k_grad_tile_bq<T, 2, 1> : k_grad_tile_bq<T, 1, 1>);
            hipLaunchKernelGGL(kern, dim3((unsigned)g), dim3(kBlock), 0, s,
                               (const TileDesc *)h.tiles, h.ntiles, (const uint16_t *)h.roff16,
                               (const int32_t *)h.col, (const uint16_t *)h.col16, h.nnz, h.B,
                               (const T *)lam_internal, (const T *)x_int, (T *)grad, sign);
        } else if (h.ntiles > 0) {
            int64_t g = (h.ntiles + kWaves - 1) / kWaves;
            if (g > 4 * kMaxGrid) g = 4 * kMaxGrid;
            hipLaunchKernelGGL(k_grad_tile<T>, dim3((unsigned)g), dim3(kBlock), 0, s,
                               (const TileDesc *)h.tiles, h.ntiles, (const uint16_t *)h.roff16,
                               (const int32_t *)h.col, (const uint16_t *)h.col16, h.nnz, h.B,
                               (const T *)lam_internal, (const T *)x_int, (T *)grad, sign);
        }
        if (h.nlong > 0)
            hipLaunchKernelGGL((k_grad_long<T, RP>), dim3((unsigned)h.nlong), dim3(kBlock), 0, s,
                               (const int32_t *)h.long_rows, (const RP *)h.row_ptr,
                               (const int32_t *)h.col, h.nnz, h.B, (const T *)lam_internal,
                               (const T *)x_int, (T *)grad, sign);
    };
    if (h.vt == SLA_F64) {
        if (h.rp64) go(double(), int64_t());
        else go(double(), int32_t());
    } else {
        if (h.rp64) go(float(), int64_t());
        else go(float(), int32_t());
    }
    SLA_HIP(hipGetLastError());
    L.end(SLA_KERNEL_GRAD, a);
}

}  // namespace sla

// Segmented solves: a list of independent systems with distinct patterns
// (torch-sla's SparseTensorList, tensor-types passage: matrices of different
// patterns batched together) held as one block-diagonal matrix. The SpMV
// kernels run on it unchanged; the vector kernels here give every segment its
// own reductions, step sizes, stopping test and iteration count, exactly as
// if each system were solved alone with the PCG of the single-system path.
//
// Every workgroup of these kernels works inside one segment (blk_seg), on
// kSegBlockRows consecutive rows, so its partial sums belong to one system.
// The last workgroup of a segment to arrive sums the segment's partials in
// workgroup order (deterministic) and updates that segment's state. A
// segment that is not running returns at once in every workgroup of it.
// ctl->n_running counts running segments (integer atomics); the direction
// kernel's first workgroup mirrors it to the host's mapped flag.
#include "common.h"

#include <vector>

namespace sla {

void launch_spmv_dots(Handle &h, const void *x, void *y, const void *w, int ndot, double *spart,
                      const int32_t *status, hipStream_t s);

namespace {

constexpr int kSegRows = 4;                          // rows per lane
constexpr int64_t kSegBlockRows = (int64_t)kBlock * kSegRows;

struct Seg {
    const int64_t *rows;   // [nseg+1]
    const int32_t *blk;    // [grid] segment of each workgroup
    const int64_t *blk0;   // [nseg+1] first workgroup of each segment
    double *part;          // [2 * grid]
    uint32_t *sync;        // [nseg * kCounterStride]
    const int64_t *tile0;  // [nseg+1] first SpMV tile of each segment
    const int64_t *long0;  // [nseg+1] first long row of each segment
    uint8_t *live;         // [ntiles] 1 while the tile's segment runs
    const double *tdot;    // [ntiles] p.q of each tile (from the SpMV)
    const double *ldot;    // [nlong] p.q of each long row
};

// mark the tiles of segment s live or not (every thread of the calling block)
__device__ __forceinline__ void set_live(const Seg &g, int32_t s, uint8_t v) {
    for (int64_t t = g.tile0[s] + threadIdx.x; t < g.tile0[s + 1]; t += kBlock) g.live[t] = v;
}

struct Range {
    int32_t s;
    int64_t r0, r1, b0, nb;
};

__device__ __forceinline__ Range seg_range(const Seg &g) {
    Range q;
    q.s = g.blk[blockIdx.x];
    q.b0 = g.blk0[q.s];
    q.nb = g.blk0[q.s + 1] - q.b0;
    q.r0 = g.rows[q.s] + ((int64_t)blockIdx.x - q.b0) * kSegBlockRows;
    const int64_t end = g.rows[q.s + 1];
    q.r1 = q.r0 + kSegBlockRows < end ? q.r0 + kSegBlockRows : end;
    return q;
}

// A workgroup's rows as 16-byte groups of W rows ([g0, g1), W-aligned in
// absolute row numbers) plus the fewer than W rows before and after them,
// done one per lane
struct VecRows {
    int64_t g0, g1;   // groups
    int64_t h0, h1;   // head rows
    int64_t t0, t1;   // tail rows
};

template <int W>
__device__ __forceinline__ VecRows vec_rows(const Range &q) {
    int64_t a0 = (q.r0 + W - 1) / W * W;
    if (a0 > q.r1) a0 = q.r1;
    int64_t a1 = q.r1 / W * W;
    if (a1 < a0) a1 = a0;
    return VecRows{a0 / W, a1 / W, q.r0, a0, a1, q.r1};
}

// the single row a lane takes outside the groups (head rows on lanes 0..,
// tail rows on lanes 64..), or -1
__device__ __forceinline__ int64_t edge_row(const VecRows &v) {
    const int t = threadIdx.x;
    if (t < v.h1 - v.h0) return v.h0 + t;
    if (t >= 64 && t - 64 < v.t1 - v.t0) return v.t0 + (t - 64);
    return -1;
}

// 16-byte groups per lane that cover a workgroup's kSegBlockRows rows
template <typename T>
constexpr int seg_groups() {
    return (int)((kSegBlockRows / VecW<T>::W + kBlock - 1) / kBlock);
}

// Stores this workgroup's C partials and arrives at its segment's counter;
// true in the segment's last workgroup, which then holds the segment totals
// in tot[0..C) (partials summed in workgroup order by a fixed tree).
template <int C>
__device__ bool seg_reduce(const Seg &g, const Range &q, const double (&v)[C], double *lds4,
                           double *tot) {
    if (threadIdx.x == 0)
        for (int c = 0; c < C; ++c) store_partial(g.part + (int64_t)blockIdx.x * C + c, v[c]);
    if (!arrive(g.sync + (int64_t)q.s * kCounterStride, (uint32_t)q.nb)) return false;
    for (int c = 0; c < C; ++c) {
        double a = 0.0;
        for (int64_t j = threadIdx.x; j < q.nb; j += kBlock) a += load_partial(g.part + (q.b0 + j) * C + c);
        const double t = block_sum(a, lds4);
        if (threadIdx.x == 0) tot[c] = t;
    }
    __syncthreads();
    return true;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_seg_init(Seg g, const T *__restrict__ b,
                                                     T *__restrict__ x, T *__restrict__ r,
                                                     T *__restrict__ p, const T *__restrict__ dinv,
                                                     Ctl *__restrict__ ctl,
                                                     SysState *__restrict__ st) {
    __shared__ double lds4[kWaves];
    __shared__ double tot[2];
    const Range q = seg_range(g);
    double sbb = 0.0, srz = 0.0;
#pragma unroll
    for (int u = 0; u < kSegRows; ++u) {
        const int64_t i = q.r0 + threadIdx.x + (int64_t)u * kBlock;
        if (i < q.r1) {
            const T bv = b[i];
            const double z = (double)dinv[i] * (double)bv;
            x[i] = (T)0;
            r[i] = bv;
            p[i] = (T)z;
            sbb += (double)bv * (double)bv;
            srz += (double)bv * z;
        }
    }
    const double v[2] = {block_sum(sbb, lds4), block_sum(srz, lds4)};
    if (seg_reduce<2>(g, q, v, lds4, tot)) {
        SysState s;
        s.bb = tot[0];
        s.rho = tot[1];
        s.alpha = 0.0;
        s.alpha2 = 0.0;
        s.beta = 0.0;
        s.rr = s.bb;
        s.iter = 0;
        if (s.bb == 0.0) s.status = SLA_CONVERGED;
        else if (ctl->maxit <= 0) s.status = SLA_MAXIT;
        else s.status = kRunning;
        set_live(g, q.s, s.status == kRunning ? 1 : 0);
        if (threadIdx.x == 0) {
            st[q.s] = s;
            if (s.status == kRunning) atomicAdd(&ctl->n_running, 1);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_seg_update(Seg g, T *__restrict__ x, T *__restrict__ r,
                                                       const T *__restrict__ p,
                                                       const T *__restrict__ qv,
                                                       const T *__restrict__ dinv,
                                                       Ctl *__restrict__ ctl,
                                                       SysState *__restrict__ st) {
    __shared__ double lds4[kWaves];
    __shared__ double tot[2];
    if (ctl->n_running == 0) return;
    const Range q = seg_range(g);
    if (st[q.s].status != kRunning) return;
    // sigma = p.q of the segment from the SpMV's per-tile and per-long-row
    // partials, summed in one fixed order by every workgroup of the segment
    double sg = 0.0;
    {
        const int64_t t1 = g.tile0[q.s + 1];
        for (int64_t t = g.tile0[q.s] + threadIdx.x; t < t1; t += 8 * kBlock) {
            double v8[8];   // 8 loads in flight per lane
#pragma unroll
            for (int u = 0; u < 8; ++u) v8[u] = t + u * kBlock < t1 ? g.tdot[t + u * kBlock] : 0.0;
#pragma unroll
            for (int u = 0; u < 8; ++u) sg += v8[u];
        }
    }
    for (int64_t l = g.long0[q.s] + threadIdx.x; l < g.long0[q.s + 1]; l += kBlock) sg += g.ldot[l];
    const double sigma = block_sum(sg, lds4);
    const bool breakdown = !(sigma > 0.0) || !isfinite(sigma);
    const double alpha = breakdown ? 0.0 : st[q.s].rho / sigma;
    double srz = 0.0, srr = 0.0;
    auto row = [&](T &xe, T &re, T pe, T qe, T de) {
        xe = (T)((double)xe + alpha * (double)pe);
        re = (T)((double)re - alpha * (double)qe);
        const double z = (double)de * (double)re;
        srz += (double)re * z;
        srr += (double)re * (double)re;
    };
    constexpr int W = VecW<T>::W, G = seg_groups<T>();
    VecRows vr = vec_rows<W>(q);
    if (breakdown) vr = VecRows{0, 0, 0, 0, 0, 0};   // x and r stay as they are
    T xv[G][W], rv[G][W], pv[G][W], qq[G][W], dv[G][W];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t gi = vr.g0 + u * kBlock + threadIdx.x;
        if (gi < vr.g1) {
            vload(x + gi * W, xv[u]);
            vload(r + gi * W, rv[u]);
            vload(p + gi * W, pv[u]);
            vload(qv + gi * W, qq[u]);
            vload(dinv + gi * W, dv[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t gi = vr.g0 + u * kBlock + threadIdx.x;
        if (gi < vr.g1) {
#pragma unroll
            for (int k = 0; k < W; ++k) row(xv[u][k], rv[u][k], pv[u][k], qq[u][k], dv[u][k]);
            vstore(x + gi * W, xv[u]);
            vstore(r + gi * W, rv[u]);
        }
    }
    const int64_t ie = edge_row(vr);
    if (ie >= 0) {
        T xe = x[ie], re = r[ie];
        row(xe, re, p[ie], qv[ie], dinv[ie]);
        x[ie] = xe;
        r[ie] = re;
    }
    const double v[2] = {block_sum(srz, lds4), block_sum(srr, lds4)};
    if (seg_reduce<2>(g, q, v, lds4, tot)) {
        // every thread takes the same decision; thread 0 records it
        const double rz = tot[0], rr = tot[1];
        const SysState s0 = st[q.s];
        const int32_t iter = s0.iter + 1;
        int32_t status = kRunning;
        if (breakdown) status = SLA_BREAKDOWN;   // rr keeps the last residual
        else if (sqrt(rr) <= ctl->tol * sqrt(s0.bb)) status = SLA_CONVERGED;
        else if (iter >= ctl->maxit) status = SLA_MAXIT;
        if (status != kRunning) set_live(g, q.s, 0);
        if (threadIdx.x == 0) {
            SysState &s = st[q.s];
            s.iter = iter;
            s.alpha = alpha;
            if (!breakdown) s.rr = rr;
            s.status = status;
            if (status != kRunning) {
                atomicSub(&ctl->n_running, 1);
            } else {
                s.beta = rz / s.rho;
                s.rho = rz;
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_seg_direction(Seg g, const T *__restrict__ r,
                                                          T *__restrict__ p,
                                                          const T *__restrict__ dinv,
                                                          Ctl *__restrict__ ctl,
                                                          const SysState *__restrict__ st,
                                                          int32_t *__restrict__ h_running) {
    const int32_t running = ctl->n_running;
    // the count is final here (the update kernel has completed)
    if (blockIdx.x == 0 && threadIdx.x == 0) publish_running(ctl, h_running, running);
    if (running == 0) return;
    const Range q = seg_range(g);
    if (st[q.s].status != kRunning) return;
    const double beta = st[q.s].beta;
    constexpr int W = VecW<T>::W, G = seg_groups<T>();
    const VecRows vr = vec_rows<W>(q);
    T rv[G][W], pv[G][W], dv[G][W];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t gi = vr.g0 + u * kBlock + threadIdx.x;
        if (gi < vr.g1) {
            vload(r + gi * W, rv[u]);
            vload(p + gi * W, pv[u]);
            vload(dinv + gi * W, dv[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int64_t gi = vr.g0 + u * kBlock + threadIdx.x;
        if (gi < vr.g1) {
#pragma unroll
            for (int k = 0; k < W; ++k)
                pv[u][k] = (T)((double)dv[u][k] * (double)rv[u][k] + beta * (double)pv[u][k]);
            vstore(p + gi * W, pv[u]);
        }
    }
    const int64_t ie = edge_row(vr);
    if (ie >= 0) p[ie] = (T)((double)dinv[ie] * (double)r[ie] + beta * (double)p[ie]);
}

// every entry (i, j) must lie in row i's segment block
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_seg_check(const RP *__restrict__ row_ptr,
                                                      const int32_t *__restrict__ col, Seg g,
                                                      int32_t nseg, int *__restrict__ bad) {
    const Range q = seg_range(g);
    const int64_t c0 = g.rows[q.s], c1 = g.rows[q.s + 1];
    int nbad = 0;
    for (int64_t i = q.r0 + threadIdx.x; i < q.r1; i += kBlock)
        for (int64_t k = row_ptr[i]; k < (int64_t)row_ptr[i + 1]; ++k)
            nbad += (col[k] < c0 || col[k] >= c1);
    (void)nseg;
    if (nbad) atomicAdd(bad, nbad);
}

Seg seg_of(Handle &h) {
    return Seg{h.seg_rows,  h.blk_seg,   h.seg_blk0, h.seg_part, h.seg_sync,
               h.seg_tile0, h.seg_long0, h.tile_live, h.tile_dot, h.long_dot};
}

template <typename T>
void seg_iter_t(Handle &h, hipStream_t s, Launcher *lp) {
    const Seg g = seg_of(h);
    const dim3 grid((unsigned)h.seg_grid), blk(kBlock);
    hipEvent_t a = nullptr;
    if (lp) lp->begin(SLA_KERNEL_SPMV_DOT, &a);
    // q = A p over the live tiles, p.q per tile and long row
    launch_spmv_dots(h, h.p, h.q, h.p, 3, nullptr, nullptr, s);
    if (lp) lp->end(SLA_KERNEL_SPMV_DOT, a);
    if (lp) lp->begin(SLA_KERNEL_UPDATE, &a);
    hipLaunchKernelGGL(k_seg_update<T>, grid, blk, 0, s, g, (T *)h.x, (T *)h.r, (const T *)h.p,
                       (const T *)h.q, (const T *)h.dinv, h.ctl, h.st);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_UPDATE, a);
    if (lp) lp->begin(SLA_KERNEL_DIRECTION, &a);
    hipLaunchKernelGGL(k_seg_direction<T>, grid, blk, 0, s, g, (const T *)h.r, (T *)h.p,
                       (const T *)h.dinv, h.ctl, (const SysState *)h.st, h.d_running);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_DIRECTION, a);
}

}  // namespace

// Workgroup layout of the segment kernels; checks that no entry leaves its
// segment's diagonal block. seg_rows: host [nseg+1], validated by the caller.
void build_segments(Handle &h, const int64_t *seg_rows, int32_t nseg, hipStream_t s) {
    std::vector<int64_t> blk0((size_t)nseg + 1);
    blk0[0] = 0;
    for (int32_t q = 0; q < nseg; ++q) {
        const int64_t rows = seg_rows[q + 1] - seg_rows[q];
        blk0[(size_t)q + 1] = blk0[(size_t)q] + (rows + kSegBlockRows - 1) / kSegBlockRows;
    }
    const int64_t grid = blk0[(size_t)nseg];
    if (grid >= ((int64_t)1 << 31)) fail(SLA_ERR_INVALID_ARG, "too many segment workgroups");
    std::vector<int32_t> blk((size_t)grid);
    for (int32_t q = 0; q < nseg; ++q)
        for (int64_t b = blk0[(size_t)q]; b < blk0[(size_t)q + 1]; ++b) blk[(size_t)b] = q;
    h.nseg = nseg;
    h.seg_grid = grid;
    h.seg_rows = (int64_t *)dalloc(h, sizeof(int64_t) * ((size_t)nseg + 1));
    h.seg_blk0 = (int64_t *)dalloc(h, sizeof(int64_t) * ((size_t)nseg + 1));
    h.blk_seg = (int32_t *)dalloc(h, sizeof(int32_t) * (size_t)grid);
    h.seg_part = (double *)dalloc(h, sizeof(double) * 2 * (size_t)grid);
    h.seg_sync = (uint32_t *)dalloc(h, sizeof(uint32_t) * (size_t)nseg * kCounterStride);
    SLA_HIP(hipMemcpyAsync(h.seg_rows, seg_rows, sizeof(int64_t) * ((size_t)nseg + 1),
                           hipMemcpyHostToDevice, s));
    SLA_HIP(hipMemcpyAsync(h.seg_blk0, blk0.data(), sizeof(int64_t) * ((size_t)nseg + 1),
                           hipMemcpyHostToDevice, s));
    SLA_HIP(hipMemcpyAsync(h.blk_seg, blk.data(), sizeof(int32_t) * (size_t)grid,
                           hipMemcpyHostToDevice, s));
    SLA_HIP(hipMemsetAsync(h.seg_sync, 0, sizeof(uint32_t) * (size_t)nseg * kCounterStride, s));
    int *bad = nullptr;
    SLA_HIP(hipMalloc(&bad, sizeof(int)));
    int hb = 0;
    try {
        SLA_HIP(hipMemsetAsync(bad, 0, sizeof(int), s));
        if (h.rp64)
            hipLaunchKernelGGL(k_seg_check<int64_t>, dim3((unsigned)grid), dim3(kBlock), 0, s,
                               (const int64_t *)h.row_ptr, (const int32_t *)h.col, seg_of(h), nseg,
                               bad);
        else
            hipLaunchKernelGGL(k_seg_check<int32_t>, dim3((unsigned)grid), dim3(kBlock), 0, s,
                               (const int32_t *)h.row_ptr, (const int32_t *)h.col, seg_of(h), nseg,
                               bad);
        SLA_HIP(hipGetLastError());
        SLA_HIP(hipMemcpyAsync(&hb, bad, sizeof(int), hipMemcpyDeviceToHost, s));
        SLA_HIP(hipStreamSynchronize(s));
    } catch (...) {
        (void)hipFree(bad);
        throw;
    }
    SLA_HIP(hipFree(bad));
    if (hb) fail(SLA_ERR_INDEX_RANGE, "an entry lies outside its segment's diagonal block");
}

void seg_init(Handle &h, const void *b, hipStream_t s, Launcher *lp) {
    hipEvent_t a = nullptr;
    if (lp) lp->begin(SLA_KERNEL_INIT, &a);
    const dim3 grid((unsigned)h.seg_grid), blk(kBlock);
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_seg_init<double>, grid, blk, 0, s, seg_of(h), (const double *)b,
                           (double *)h.x, (double *)h.r, (double *)h.p, (const double *)h.dinv,
                           h.ctl, h.st);
    else
        hipLaunchKernelGGL(k_seg_init<float>, grid, blk, 0, s, seg_of(h), (const float *)b,
                           (float *)h.x, (float *)h.r, (float *)h.p, (const float *)h.dinv, h.ctl,
                           h.st);
    SLA_HIP(hipGetLastError());
    if (lp) lp->end(SLA_KERNEL_INIT, a);
}

void seg_iter_kernels(Handle &h, hipStream_t s, Launcher *lp) {
    if (h.vt == SLA_F64) seg_iter_t<double>(h, s, lp);
    else seg_iter_t<float>(h, s, lp);
}

}  // namespace sla

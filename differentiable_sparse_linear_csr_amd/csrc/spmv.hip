// Sparse matrix-vector products for gfx950 (the .matvec of SparseTensor and
// the q = A p step of CG; torch-sla API section and backend list).
//
// Single matrix (B = 1): row-binned CSR. Rows are grouped into tiles of about
// kTileUnits (rows + entries). A short-row tile streams its entries with
// coalesced loads, forms val * x[col] in fp64 and parks the products in LDS;
// the rows are then summed from LDS by groups of G lanes, G picked from the
// tile's row count (one lane per row for stencil-like rows, up to a whole
// wave for a few medium rows). A row longer than kLongRow is a tile of its own
// and gets a full workgroup.
//
// Batch sharing one pattern (B > 1): values [nnz][B] and vectors [n][B]; lane
// (row, b) walks its row, and the B lanes of a row read one index and B
// consecutive values, so col_idx / row_ptr are read once for all systems.
//
// The fused variants also form per-block partials of p.q for the CG step
// size; the last block to finish reduces them in block order (deterministic)
// and writes alpha = rho / p.q per system, or flags a breakdown.
#include "common.h"

namespace sla {

int64_t spmv_grid(const Handle &h);

namespace {

constexpr int kTileGroups = (kTileCap + 3 + 4 * 64 - 1) / (4 * 64);
// products sit at their place in the lane's 4-entry groups (entry k0 of a
// tile at slot k0 % 4); a group that holds any of the tile's entries is
// written whole
constexpr int kProdSlots = (kTileCap + 3 + 3) / 4 * 4;
constexpr int kSumBatch = 2;   // LDS reads issued together per row sum (4: 4% slower)
constexpr int kRowItems = (kTileUnits + 1 + 63) / 64;  // row offsets per lane

// Rows longer than kLongRow: one workgroup per row, 8 entries in flight per
// lane. Runs before the tile kernel. With DOT >= 1 it also leaves w_i q_i of
// each long row in long_dot[l] (and q_i q_i in long_dot[nlong + l] with
// DOT = 2) for the tile kernel's reduction; it does nothing unless *status is
// still running.
template <typename T, typename RP, int DOT>
__global__ __launch_bounds__(kBlock) void k_spmv_long(
    const int32_t *__restrict__ long_rows, int64_t nlong, const RP *__restrict__ row_ptr,
    const int32_t *__restrict__ col, const T *__restrict__ val, const T *__restrict__ x,
    T *__restrict__ y, const T *__restrict__ w, double *__restrict__ long_dot,
    const int32_t *__restrict__ status) {
    __shared__ double lds4[kWaves];
    if (DOT > 0 && DOT != 3 && *status != kRunning) return;
    const int tid = threadIdx.x;
    const int64_t i = long_rows[blockIdx.x];
    const int64_t k0 = row_ptr[i], len = (int64_t)row_ptr[i + 1] - k0;
    const int32_t *cp = col + k0;
    const T *vp = val + k0;
    constexpr int kU = 8;
    double s = 0.0;
    for (int64_t base = 0; base < len; base += (int64_t)kU * kBlock) {
        int32_t c[kU];
        T v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = base + tid + u * kBlock;
            c[u] = j < len ? cp[j] : 0;
            v[u] = j < len ? vp[j] : (T)0;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) s += (double)v[u] * (double)x[c[u]];
    }
    s = block_sum(s, lds4);
    if (tid == 0) {
        const T q = (T)s;
        y[i] = q;
        if (DOT > 0) long_dot[blockIdx.x] = (double)w[i] * (double)q;
        if (DOT == 2) long_dot[nlong + blockIdx.x] = (double)q * (double)q;
    }
}

// Short-row tiles, one wavefront per tile. Every wavefront runs its own
// software pipeline with its own LDS slice and no workgroup barrier: the next
// tile's entries and row offsets are loaded while the current tile's fp64
// products are parked in LDS and summed by G lanes per row (G from the tile's
// row count). LDS accesses of one wavefront complete in order, so only a
// wave-level scheduling barrier separates the stores from the sums.
// Wavefronts walk the tiles in an XCD-contiguous order: workgroup b runs on
// XCD b % 8, and the wavefronts of one XCD take one contiguous eighth of the
// tiles, so the gathered vector segments they share stay in that XCD's L2.
// The grid is persistent (a multiple of 8, at most kMaxGrid workgroups),
// which also bounds the reduction partials. With DOT >= 1 (the fused forms)
// it adds w.q of its rows, and of the long rows in a fixed order, to a
// per-workgroup partial spart[DOT * block], and with DOT = 2 also q.q to
// spart[2 * block + 1]; the fused forms do nothing unless *status is running.
//
// DOT = 3 is the form of a list of systems (segmented handle, tiles never
// straddle two members): tiles whose member has finished (live[t] = 0) are
// skipped, and each tile's w.q goes to tile_dot[t] for its member's update.
template <typename T, typename RP, int DOT, bool NARROW>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void k_spmv_tile(
    const TileDesc *__restrict__ tiles, int64_t ntiles, const uint16_t *__restrict__ roff16,
    const int32_t *__restrict__ col, const uint16_t *__restrict__ col16, const T *__restrict__ val,
    const T *__restrict__ x, T *__restrict__ y, const T *__restrict__ w,
    const double *__restrict__ long_dot, int64_t nlong, double *__restrict__ spart,
    const int32_t *__restrict__ status, const uint8_t *__restrict__ live,
    double *__restrict__ tile_dot) {
    constexpr bool FUSED = DOT > 0;
    constexpr bool PERTILE = DOT == 3;
    __shared__ __align__(16) double prod_all[kWaves][kProdSlots];
    __shared__ int32_t roff_all[kWaves][kTileUnits + 1];
    __shared__ double pown_all[FUSED ? kWaves : 1][FUSED ? kTileUnits : 1];
    __shared__ double lds4[kWaves];
    if (FUSED && !PERTILE && *status != kRunning) return;

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    double *prod = prod_all[wv];
    int32_t *roff = roff_all[wv];
    double *pown = pown_all[FUSED ? wv : 0];  // w of the tile's own rows (fused forms)
    const int xcd = blockIdx.x % kXcds;
    const int64_t waves_per_xcd = (int64_t)(gridDim.x / kXcds) * kWaves;
    const int64_t wid = (int64_t)(blockIdx.x / kXcds) * kWaves + wv;  // rank within its XCD
    int64_t t = ntiles * xcd / kXcds + wid;
    const int64_t t_end = ntiles * (xcd + 1) / kXcds;
    double dot = 0.0, dot2 = 0.0;

    TileDesc d{0, 0, 0, 0, 0, 0, 0};
    int32_t c[kTileGroups][4];
    T v[kTileGroups][4];
    int32_t ro[kRowItems];
    // Entries come in groups of 4 from base = k0 rounded down to a multiple
    // of 4 (index and value arrays are allocated 256-byte aligned): 16-byte
    // value loads, and 8-byte loads of 16-bit columns when every tile is
    // narrow (the tile's smallest column added back) or 16-byte loads of
    // 32-bit columns otherwise. Groups wholly outside [k0, k1) are not loaded, partial ones
    // are masked when consumed. Row offsets are the tile's 16-bit ones.
    auto fetch = [&](const TileDesc &e) {
        const int64_t base = e.k0 & ~(int64_t)3;
        const int span = (int)(e.k1 - base);
        const int nr = e.re - e.rs;
        const T *vp = val + base;
        if (NARROW) {
            const uint16_t *cp = col16 + base;
            const int32_t cb = e.cbase;
#pragma unroll
            for (int u = 0; u < kTileGroups; ++u) {
                const int g = 4 * (lane + u * 64);
                if (g < span) {
                    const uint2 raw = *reinterpret_cast<const uint2 *>(cp + g);
                    c[u][0] = cb + (int32_t)(raw.x & 0xffffu);
                    c[u][1] = cb + (int32_t)(raw.x >> 16);
                    c[u][2] = cb + (int32_t)(raw.y & 0xffffu);
                    c[u][3] = cb + (int32_t)(raw.y >> 16);
                    load4(vp + g, v[u]);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        c[u][k] = 0;
                        v[u][k] = (T)0;
                    }
                }
            }
        } else {
            const int32_t *cp = col + base;
#pragma unroll
            for (int u = 0; u < kTileGroups; ++u) {
                const int g = 4 * (lane + u * 64);
                if (g < span) {
                    load4(cp + g, c[u]);
                    load4(vp + g, v[u]);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        c[u][k] = 0;
                        v[u][k] = (T)0;
                    }
                }
            }
        }
        const uint16_t *rp = roff16 + e.rpos;
#pragma unroll
        for (int u = 0; u < kRowItems; ++u) {
            const int j = lane + u * 64;
            ro[u] = j <= nr ? (int32_t)rp[j] : 0;
        }
    };
    // first live tile at or after u in this wavefront's sequence
    auto next_live = [&](int64_t u) {
        if (PERTILE)
            while (u < t_end && !live[u]) u += waves_per_xcd;
        return u;
    };
    t = next_live(t);
    if (t < t_end) {
        d = tiles[t];
        fetch(d);
    }
    while (t < t_end) {
        const int64_t tn = next_live(t + waves_per_xcd);
        TileDesc dn{0, 0, 0, 0, 0, 0, 0};
        if (tn < t_end) dn = tiles[tn];
        const int nrows = d.re - d.rs;
        const int shift = (int)(d.k0 & 3);           // entries of the first group before k0
        const int nk = (int)(d.k1 - d.k0);
#pragma unroll
        for (int u = 0; u < kTileGroups; ++u) {
            double xv[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = 4 * (lane + u * 64) + k - shift;  // entry index within the tile
                xv[k] = (double)x[(j >= 0 && j < nk) ? c[u][k] : 0];  // masked lanes read x[0]
            }
            // 32 consecutive bytes per lane (no bank conflicts); slots of
            // entries outside [k0, k1) are never read
            const int g = 4 * (lane + u * 64);
            if (g < nk + shift) {
                double2 *pd = reinterpret_cast<double2 *>(prod + g);
                pd[0] = make_double2((double)v[u][0] * xv[0], (double)v[u][1] * xv[1]);
                pd[1] = make_double2((double)v[u][2] * xv[2], (double)v[u][3] * xv[3]);
            }
        }
#pragma unroll
        for (int u = 0; u < kRowItems; ++u) {
            const int j = lane + u * 64;
            if (j <= nrows) roff[j] = ro[u];
        }
        if (FUSED) {
            // w of the tile's own rows, loaded next to the gathers (same latency)
            const T *pp = w + d.rs;
#pragma unroll
            for (int u = 0; u < kTileUnits / 64; ++u) {
                const int i = lane + u * 64;
                if (i < nrows) pown[i] = (double)pp[i];
            }
        }
        if (tn < t_end) fetch(dn);  // in flight during the sums below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int G = 1;
        while (G < 64 && G * 2 * nrows <= 64) G *= 2;
        const int lg = lane & (G - 1);
        const int grp = lane / G;
        const int ngrp = 64 / G;
        for (int i = grp; i < nrows; i += ngrp) {
            const int a = roff[i] + shift, b = roff[i + 1] + shift;
            // the lane's first kSB entries are read together, then added in
            // order
            constexpr int kSB = kSumBatch;
            double pv[kSB];
#pragma unroll
            for (int q = 0; q < kSB; ++q) {
                const int j = a + lg + q * G;
                pv[q] = prod[j < kProdSlots - 1 ? j : kProdSlots - 1];   // clamped; unused past b
            }
            double s = 0.0;
#pragma unroll
            for (int q = 0; q < kSB; ++q)
                if (a + lg + q * G < b) s += pv[q];
            for (int j = a + lg + kSB * G; j < b; j += G) s += prod[j];
            for (int off = G >> 1; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
            if (lg == 0) {
                const T q = (T)s;
                y[d.rs + i] = q;
                if (FUSED) dot += pown[i] * (double)q;
                if (DOT == 2) dot2 += (double)q * (double)q;
            }
        }
        if (PERTILE) {
            // the tile's w.q (lanes summed by a fixed tree) for its member
            const double td = wave_sum(dot);
            if (lane == 0) tile_dot[t] = td;
            dot = 0.0;
        }
        // this wavefront's next stores to its LDS slice come after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        t = tn;
        d = dn;
    }
    if (FUSED && !PERTILE) {
        // this workgroup's partials; the next kernel sums them (every
        // workgroup there, in block order) and forms its step, so this
        // kernel ends without a grid-wide arrival
        for (int64_t l = blockIdx.x + (int64_t)threadIdx.x * gridDim.x; l < nlong;
             l += (int64_t)kBlock * gridDim.x) {
            dot += long_dot[l];
            if (DOT == 2) dot2 += long_dot[nlong + l];
        }
        dot = block_sum(dot, lds4);
        if (DOT == 2) dot2 = block_sum(dot2, lds4);
        if (threadIdx.x == 0) {
            spart[(int64_t)DOT * blockIdx.x] = dot;
            if (DOT == 2) spart[2 * (int64_t)blockIdx.x + 1] = dot2;
        }
    }
}

// Batch sharing one pattern (B > 1), general B: lane (row slot jr, system b)
// walks its row; the B lanes of a row read one index and B consecutive
// values, so col_idx / row_ptr are read once for all systems.
template <typename T, typename RP, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_spmv_batched(
    int64_t n, int B, int rows_per_lane, const RP *__restrict__ row_ptr,
    const int32_t *__restrict__ col, const T *__restrict__ val, const T *__restrict__ x,
    T *__restrict__ y, Red red, Ctl *__restrict__ ctl, SysState *__restrict__ st,
    int32_t *__restrict__ h_running) {
    __shared__ double tmp[kBlock];
    __shared__ double tot[kMaxBatch];
    __shared__ double blk[kMaxBatch];
    if (FUSED && ctl->n_running == 0) return;
    const Lanes L(B);
    const bool active = L.on && (!FUSED || st[L.b].status == kRunning);
    double dot = 0.0;
    const int64_t row0 = (int64_t)blockIdx.x * L.J * rows_per_lane;
    if (active) {
        for (int j = 0; j < rows_per_lane; ++j) {
            const int64_t i = row0 + (int64_t)j * L.J + L.jr;
            if (i >= n) break;
            const int64_t ka = row_ptr[i], kb = row_ptr[i + 1];
            double s = 0.0;
            for (int64_t k = ka; k < kb; ++k)
                s += (double)val[k * B + L.b] * (double)x[(int64_t)col[k] * B + L.b];
            const T q = (T)s;
            y[i * B + L.b] = q;
            if (FUSED) dot += (double)x[i * B + L.b] * (double)q;
        }
    }
    if (FUSED) {
        block_sum_per_system(dot, L, tmp, blk);
        if (threadIdx.x < B)
            store_partial(red.part + (int64_t)blockIdx.x * B + threadIdx.x, blk[threadIdx.x]);
        if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, B, tmp, tot))
            finish_alpha(tot, B, ctl, st, h_running);
    }
}

static int batched_rows_per_lane(const Handle &h) {
    const int64_t J = kBlock / h.B;
    int rpl = 1;
    while ((h.n + J * rpl - 1) / (J * rpl) > kMaxGrid) rpl *= 2;
    return rpl;
}

// Batch with Q = B / W a power of two (W = 16 / sizeof(T)): a lane carries W
// adjacent systems of a row, so each value load, gather, p load and q store
// is one 16-byte access, and the Q lanes of a row cover an entry's B values
// as one contiguous run (index and values of an entry are read once for the
// whole batch). A pass takes kBvRows rows per lane; the loads of a row's
// first kBvEntries entries are issued together (row pointers, then indices
// and values, then the gathers), longer rows finish in a loop. Workgroups
// take contiguous row ranges, XCD-contiguous (workgroup b runs on XCD
// b % 8; consecutive ranges go to the same XCD so stencil neighbours share
// its L2).
constexpr int kBvRows = 2;
constexpr int kBvEntries = 5;

template <typename T, typename RP, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_spmv_bvec(
    int64_t n, int B, int64_t rows_block, const RP *__restrict__ row_ptr,
    const int32_t *__restrict__ col, const T *__restrict__ val, const T *__restrict__ x,
    T *__restrict__ y, Red red, Ctl *__restrict__ ctl, SysState *__restrict__ st,
    int32_t *__restrict__ h_running) {
    constexpr int W = VecW<T>::W;
    __shared__ double tmp[4 * kMaxBatch];
    __shared__ double tot[kMaxBatch];
    __shared__ double blk[kMaxBatch];
    if (FUSED && ctl->n_running == 0) return;
    const int Q = B / W;
    const int t = threadIdx.x;
    const int s0 = (t & (Q - 1)) * W;
    const int J = kBlock / Q;
    const int jr = t / Q;
    bool any = !FUSED;
    if (FUSED) {
#pragma unroll
        for (int k = 0; k < W; ++k) any |= st[s0 + k].status == kRunning;
    }
    const int64_t G = gridDim.x;  // a multiple of kXcds
    const int64_t lb = (int64_t)(blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;
    const int64_t r_begin = lb * rows_block;
    const int64_t r_end = r_begin + rows_block < n ? r_begin + rows_block : n;
    double dot[W];
#pragma unroll
    for (int k = 0; k < W; ++k) dot[k] = 0.0;
    if (any) {
        for (int64_t r0 = r_begin; r0 < r_end; r0 += (int64_t)J * kBvRows) {
            int64_t ri[kBvRows], ka[kBvRows], kb[kBvRows];
#pragma unroll
            for (int u = 0; u < kBvRows; ++u) {
                ri[u] = r0 + (int64_t)u * J + jr;
                const bool in = ri[u] < r_end;
                ka[u] = in ? (int64_t)row_ptr[ri[u]] : 0;
                kb[u] = in ? (int64_t)row_ptr[ri[u] + 1] : 0;
            }
            int32_t c[kBvRows][kBvEntries];
            T v[kBvRows][kBvEntries][W], xv[kBvRows][kBvEntries][W], pv[kBvRows][W];
#pragma unroll
            for (int u = 0; u < kBvRows; ++u)
#pragma unroll
                for (int e = 0; e < kBvEntries; ++e) {
                    const int64_t k = ka[u] + e;
                    if (k < kb[u]) {
                        c[u][e] = col[k];
                        vload(val + k * B + s0, v[u][e]);
                    } else {
                        c[u][e] = 0;
#pragma unroll
                        for (int w = 0; w < W; ++w) v[u][e][w] = (T)0;
                    }
                }
#pragma unroll
            for (int u = 0; u < kBvRows; ++u) {
#pragma unroll
                for (int e = 0; e < kBvEntries; ++e) {
                    if (ka[u] + e < kb[u]) {
                        vload(x + (int64_t)c[u][e] * B + s0, xv[u][e]);
                    } else {
#pragma unroll
                        for (int w = 0; w < W; ++w) xv[u][e][w] = (T)0;
                    }
                }
                if (FUSED) {
                    if (ri[u] < r_end) {
                        vload(x + ri[u] * B + s0, pv[u]);
                    } else {
#pragma unroll
                        for (int w = 0; w < W; ++w) pv[u][w] = (T)0;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kBvRows; ++u) {
                if (ri[u] >= r_end) continue;
                double sum[W];
#pragma unroll
                for (int w = 0; w < W; ++w) sum[w] = 0.0;
#pragma unroll
                for (int e = 0; e < kBvEntries; ++e)
#pragma unroll
                    for (int w = 0; w < W; ++w) sum[w] += (double)v[u][e][w] * (double)xv[u][e][w];
                for (int64_t k = ka[u] + kBvEntries; k < kb[u]; ++k) {
                    T a[W], b[W];
                    vload(val + k * B + s0, a);
                    vload(x + (int64_t)col[k] * B + s0, b);
#pragma unroll
                    for (int w = 0; w < W; ++w) sum[w] += (double)a[w] * (double)b[w];
                }
                T qv[W];
#pragma unroll
                for (int w = 0; w < W; ++w) qv[w] = (T)sum[w];
                vstore(y + ri[u] * B + s0, qv);
                if (FUSED) {
#pragma unroll
                    for (int w = 0; w < W; ++w) dot[w] += (double)pv[u][w] * (double)qv[w];
                }
            }
        }
    }
    if (FUSED) {
        block_sum_systems<W>(dot, Q, tmp, blk);
        for (int s = t; s < B; s += kBlock)
            store_partial(red.part + (int64_t)blockIdx.x * B + s, blk[s]);
        if (last_block_sums(red.part, red.gpart, red.sync, gridDim.x, B, tmp, tot))
            finish_alpha(tot, B, ctl, st, h_running);
    }
}

template <typename T>
bool bvec_ok(const Handle &h) {
    constexpr int W = VecW<T>::W;
    if (h.B < 2 || h.B % W) return false;
    const int Q = h.B / W;
    return (Q & (Q - 1)) == 0 && Q <= kBlock;
}

// rows per workgroup of the vectorized batched kernel: whole passes, spread
// over at most the workgroups that are resident at once
template <typename T, bool FUSED>
int64_t bvec_rows_block(const Handle &h) {
    const int64_t rows_pass = (int64_t)(kBlock / (h.B / VecW<T>::W)) * kBvRows;
    const int64_t total = (h.n + rows_pass - 1) / rows_pass;
    const int64_t g = h.bvec_resident[FUSED ? 1 : 0];
    const int64_t passes = (total + g - 1) / g;
    return rows_pass * (passes > 0 ? passes : 1);
}

// a multiple of the XCD count, at most the resident count (itself one)
template <typename T, bool FUSED>
int64_t bvec_grid(const Handle &h) {
    const int64_t rb = bvec_rows_block<T, FUSED>(h);
    const int64_t g = (h.n + rb - 1) / rb;
    return (g + kXcds - 1) / kXcds * kXcds;
}

template <typename T>
int64_t batched_grid_t(const Handle &h) {
    if (bvec_ok<T>(h)) return bvec_grid<T, true>(h);
    const int64_t rows_block = (int64_t)(kBlock / h.B) * batched_rows_per_lane(h);
    return (h.n + rows_block - 1) / rows_block;
}

// Single system: the long-row kernel (if any) and the tile kernel, with DOT
// fused inner products against w (see k_spmv_tile).
template <typename T, typename RP, int DOT>
void launch_tiles(Handle &h, const void *x, void *y, const void *w, double *spart,
                  const int32_t *status, hipStream_t s) {
    if (h.nlong > 0)
        hipLaunchKernelGGL((k_spmv_long<T, RP, DOT>), dim3((unsigned)h.nlong), dim3(kBlock), 0, s,
                           (const int32_t *)h.long_rows, h.nlong, (const RP *)h.row_ptr,
                           (const int32_t *)h.col, (const T *)h.vals, (const T *)x, (T *)y,
                           (const T *)w, h.long_dot, status);
    const int64_t grid = spmv_grid(h);
    auto kern = h.all_narrow ? k_spmv_tile<T, RP, DOT, true> : k_spmv_tile<T, RP, DOT, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), 0, s, (const TileDesc *)h.tiles,
                       h.ntiles, (const uint16_t *)h.roff16, (const int32_t *)h.col,
                       (const uint16_t *)h.col16, (const T *)h.vals, (const T *)x, (T *)y,
                       (const T *)w, (const double *)h.long_dot, h.nlong, spart, status,
                       (const uint8_t *)h.tile_live, h.tile_dot);
}

template <typename T, typename RP, bool FUSED>
void launch_spmv_t(Handle &h, const void *x, void *y, hipStream_t s) {
    const Red red{h.part, h.gpart, h.sync + kCntSpmv * kCountersPerKind};
    if (h.B == 1) {
        launch_tiles<T, RP, FUSED ? 1 : 0>(h, x, y, x, h.spart, &h.st[0].status, s);
    } else if (bvec_ok<T>(h)) {
        hipLaunchKernelGGL((k_spmv_bvec<T, RP, FUSED>), dim3((unsigned)bvec_grid<T, FUSED>(h)),
                           dim3(kBlock), 0, s, h.n, h.B, bvec_rows_block<T, FUSED>(h),
                           (const RP *)h.row_ptr, (const int32_t *)h.col, (const T *)h.vals,
                           (const T *)x, (T *)y, red, h.ctl, h.st, h.d_running);
    } else {
        hipLaunchKernelGGL((k_spmv_batched<T, RP, FUSED>), dim3((unsigned)batched_grid_t<T>(h)),
                           dim3(kBlock), 0, s, h.n, h.B, batched_rows_per_lane(h),
                           (const RP *)h.row_ptr, (const int32_t *)h.col, (const T *)h.vals,
                           (const T *)x, (T *)y, red, h.ctl, h.st, h.d_running);
    }
    SLA_HIP(hipGetLastError());
}

}  // namespace

int64_t spmv_grid(const Handle &h) {
    if (h.B == 1) {
        const int64_t blocks = (h.ntiles + kWaves - 1) / kWaves;   // one tile per wavefront
        int64_t g = (blocks + kXcds - 1) / kXcds * kXcds;         // multiple of the XCD count
        if (g < kXcds) g = kXcds;
        return g < h.spmv_resident ? g : h.spmv_resident;
    }
    return h.vt == SLA_F64 ? batched_grid_t<double>(h) : batched_grid_t<float>(h);
}

// Resident capacity of the persistent tile kernel: every workgroup of the
// grid must be on a CU at once, or the later ones start only when earlier
// ones finish and the kernel runs in two rounds.
int64_t resident_workgroups(const void *kernel, int device) {
    int cus = 0, per_cu = 0;
    SLA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device));
    SLA_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0));
    int64_t g = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    g = g / kXcds * kXcds;
    if (g < kXcds) g = kXcds;
    if (g > kMaxGrid) g = kMaxGrid;
    return g;
}

void init_launch_limits(Handle &h) {
    const void *fn = nullptr;
    if (h.vt == SLA_F64) {
        if (h.all_narrow)
            fn = h.rp64 ? (const void *)&k_spmv_tile<double, int64_t, 1, true>
                        : (const void *)&k_spmv_tile<double, int32_t, 1, true>;
        else
            fn = h.rp64 ? (const void *)&k_spmv_tile<double, int64_t, 1, false>
                        : (const void *)&k_spmv_tile<double, int32_t, 1, false>;
    } else {
        if (h.all_narrow)
            fn = h.rp64 ? (const void *)&k_spmv_tile<float, int64_t, 1, true>
                        : (const void *)&k_spmv_tile<float, int32_t, 1, true>;
        else
            fn = h.rp64 ? (const void *)&k_spmv_tile<float, int64_t, 1, false>
                        : (const void *)&k_spmv_tile<float, int32_t, 1, false>;
    }
    h.spmv_resident = resident_workgroups(fn, h.device);
    if (h.B > 1) {
        auto pick = [&](auto ttag, auto rtag) {
            using T = decltype(ttag);
            using RP = decltype(rtag);
            h.bvec_resident[0] = resident_workgroups((const void *)&k_spmv_bvec<T, RP, false>, h.device);
            h.bvec_resident[1] = resident_workgroups((const void *)&k_spmv_bvec<T, RP, true>, h.device);
        };
        if (h.vt == SLA_F64) {
            if (h.rp64) pick(double(), int64_t());
            else pick(double(), int32_t());
        } else {
            if (h.rp64) pick(float(), int64_t());
            else pick(float(), int32_t());
        }
    }
}

// q = A p on the solve workspace, fused with the p.q partials and alpha.
void launch_spmv_dot(Handle &h, hipStream_t s) {
    if (h.vt == SLA_F64) {
        if (h.rp64) launch_spmv_t<double, int64_t, true>(h, h.p, h.q, s);
        else launch_spmv_t<double, int32_t, true>(h, h.p, h.q, s);
    } else {
        if (h.rp64) launch_spmv_t<float, int64_t, true>(h, h.p, h.q, s);
        else launch_spmv_t<float, int32_t, true>(h, h.p, h.q, s);
    }
}

// plain y = A x, both in internal layout ([n][B])
void launch_spmv_plain(Handle &h, const void *x, void *y, hipStream_t s) {
    if (h.vt == SLA_F64) {
        if (h.rp64) launch_spmv_t<double, int64_t, false>(h, x, y, s);
        else launch_spmv_t<double, int32_t, false>(h, x, y, s);
    } else {
        if (h.rp64) launch_spmv_t<float, int64_t, false>(h, x, y, s);
        else launch_spmv_t<float, int32_t, false>(h, x, y, s);
    }
}

// Single system: y = A x with ndot (0, 1 or 2) inner products fused: w.y into
// spart[ndot * block] and, for ndot = 2, y.y into spart[2 * block + 1], one
// partial per workgroup of spmv_grid(h); skipped unless *status is running
// (ndot > 0). spart holds ndot * spmv_grid(h) doubles. ndot = 3: segmented
// handle, w.y per tile into h.tile_dot (and per long row into h.long_dot),
// tiles with h.tile_live[t] = 0 skipped; status and spart unused.
void launch_spmv_dots(Handle &h, const void *x, void *y, const void *w, int ndot, double *spart,
                      const int32_t *status, hipStream_t s) {
    auto go = [&](auto ttag, auto rtag) {
        using T = decltype(ttag);
        using RP = decltype(rtag);
        if (ndot == 0) launch_tiles<T, RP, 0>(h, x, y, w, spart, status, s);
        else if (ndot == 1) launch_tiles<T, RP, 1>(h, x, y, w, spart, status, s);
        else if (ndot == 2) launch_tiles<T, RP, 2>(h, x, y, w, spart, status, s);
        else launch_tiles<T, RP, 3>(h, x, y, w, spart, status, s);
    };
    if (h.vt == SLA_F64) {
        if (h.rp64) go(double(), int64_t());
        else go(double(), int32_t());
    } else {
        if (h.rp64) go(float(), int64_t());
        else go(float(), int32_t());
    }
    SLA_HIP(hipGetLastError());
}

}  // namespace sla

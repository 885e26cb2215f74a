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
    double *__restrict__ tile_dot, int64_t band_l, int32_t band_p) {
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
    int64_t waves_per_xcd = (int64_t)(gridDim.x / kXcds) * kWaves;
    const int64_t wid = (int64_t)(blockIdx.x / kXcds) * kWaves + wv;  // rank within its XCD
    int64_t t = ntiles * xcd / kXcds + wid;
    int64_t t_end = ntiles * (xcd + 1) / kXcds;
    if (!PERTILE && band_l > 0 && band_l * band_p == waves_per_xcd) {
        // band-aligned tiles: the XCD's range splits into band_p panels of
        // band_l columns; wavefront `col` of a panel walks tiles col, col + L,
        // col + 2L, ... of it, so the p lines that tile j gathers near +N are
        // gathered again, as its own rows, one step later by the same
        // wavefront (tile j + L), and near -N one step after that
        const int64_t T0 = t - wid, T1 = t_end;
        const int64_t panel = wid / band_l, col = wid - panel * band_l;
        t = T0 + (T1 - T0) * panel / band_p + col;
        t_end = T0 + (T1 - T0) * (panel + 1) / band_p;
        waves_per_xcd = band_l;   // the stride of the walk
    }
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

// The folded direction p = z + beta p_old of one row, rounded to T: the same
// fused multiply-add wherever it is formed (a tile's own rows and every
// gathered column), so each row's p_new is one value.
template <typename T>
__device__ __forceinline__ T fold_p(double z, double pold, double beta) {
    return (T)__builtin_fma(beta, pold, z);
}

// The same product for tiles that each fit one 4-entry group per lane and one
// row offset per lane (entries from k0 rounded down to a multiple of 4 up to
// k1 at most 256, at most 63 rows) with 16-bit columns: a ring of kRing tiles
// per wavefront. Memory operations complete in issue order, so a wavefront
// that waits for a tile's gathers also waits for everything issued before
// them; here a tile's entries (packed columns, values, row offsets and w of
// its rows) are issued kRing tiles, and its gathers two tiles, before the
// tile is summed, and each wait leaves the later tiles' loads in flight
// (in k_spmv_tile a tile's gathers are waited for with nothing else of the
// wavefront's in flight). Descriptors come one tile ahead of the entries.
// Same tiles, walk, sums and results as k_spmv_tile.
constexpr int kRing = 4;
// Unused LDS requested at launch so that every form (fp64 or fp32, 0 to 3
// fused dots; static LDS 9 to 11 KB) holds four workgroups per CU (160 KB
// each), whatever its register count: the grid is the resident count of one
// form, and the band-aligned walk needs the wavefronts per XCD it was built
// for. Four rather than five (the most registers allow): 512 wavefronts per
// XCD make 45-row tiles of the 11548-row band (640: 36 rows), and on the
// 133M-row Poisson matrix the SpMV took 2.05 ms against 2.14 (kernel trace;
// 23-row tiles 2.52 ms, 30-row 2.20 ms, the usual tiles 2.40 ms).
constexpr size_t kRingLdsPad = 24 * 1024;

template <typename T, typename RP, int DOT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_spmv_tile_ring(
    const TileDesc *__restrict__ tiles, int64_t ntiles, const uint16_t *__restrict__ roff16,
    const uint16_t *__restrict__ col16, const T *__restrict__ val, const T *__restrict__ x,
    T *__restrict__ y, const T *__restrict__ w, const double *__restrict__ long_dot, int64_t nlong,
    double *__restrict__ spart, const int32_t *__restrict__ status, const uint8_t *__restrict__ live,
    double *__restrict__ tile_dot, int64_t band_l, int32_t band_p, FoldArgs fa) {
    constexpr bool FUSED = DOT > 0;
    constexpr bool PERTILE = DOT == 3;
    constexpr bool FOLD = DOT == 4;   // direction folded in (see FoldArgs); w.q with w = p_new
    __shared__ __align__(16) double prod_all[kWaves][4 * 64];
    __shared__ int32_t roff_all[kWaves][64];
    __shared__ double pown_all[FUSED ? kWaves : 1][FUSED ? 64 : 1];
    __shared__ double lds4[kWaves];
    if (FUSED && !PERTILE && *status != kRunning) return;

    const int lane = threadIdx.x & 63;
    // wave-uniform, so that tile indices and descriptors live in scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    double *prod = prod_all[wv];
    int32_t *roff = roff_all[wv];
    double *pown = pown_all[FUSED ? wv : 0];
    const int xcd = blockIdx.x % kXcds;
    int64_t stride = (int64_t)(gridDim.x / kXcds) * kWaves;
    const int64_t wid = (int64_t)(blockIdx.x / kXcds) * kWaves + wv;
    int64_t t_next = ntiles * xcd / kXcds + wid;
    int64_t t_end = ntiles * (xcd + 1) / kXcds;
    if (!PERTILE && band_l > 0 && band_l * band_p == stride) {
        const int64_t T0 = t_next - wid, T1 = t_end;
        const int64_t panel = wid / band_l, colw = wid - panel * band_l;
        t_next = T0 + (T1 - T0) * panel / band_p + colw;
        t_end = T0 + (T1 - T0) * (panel + 1) / band_p;
        stride = band_l;
    }
    // the live flags read as 32-bit words from wave-uniform addresses
    // (scalar loads, which the in-order vector counter does not wait for)
    const uint32_t *live32 = reinterpret_cast<const uint32_t *>(live);
    auto next_live = [&](int64_t u) {
        if (PERTILE)
            while (u < t_end && ((live32[u >> 2] >> (8 * (u & 3))) & 0xffu) == 0) u += stride;
        return u;
    };
    double dot = 0.0, dot2 = 0.0;
    // folded form: the gathers read z and p_old; x is updated in place on
    // every other launch (xstep: an odd count of completed updates), with
    // the two steps pending since the last such launch, in their order:
    // alpha2 p_old2 (the step before, its direction still in the buffer
    // p_new is about to take) and alpha p_old. Each step rounds x as it
    // would on its own, so x takes the same values as when updated on every
    // launch, and the x stream (read and write, 16 bytes a row) is replaced
    // by 12 bytes a row on average.
    double beta = 0.0, ax = 0.0, ax2 = 0.0;
    bool xstep = false;
    const T *zz = nullptr, *pold = nullptr;
    T *pnew = nullptr, *xx = nullptr;
    if (FOLD) {
        const SysState s0 = *fa.st;
        beta = s0.beta;
        ax = s0.alpha;
        ax2 = s0.alpha2;
        xstep = (s0.iter & 1) != 0;
        const int par = s0.iter & 1;
        zz = (const T *)fa.z;
        pold = (const T *)fa.p[par];
        pnew = (T *)fa.p[par ^ 1];
        xx = (T *)fa.x;
    }

    // slot u: tile, descriptor fields, the lane's packed 16-bit columns,
    // values, row offset and w; gather buffer h: x at the slot's columns
    int64_t s_t[kRing];
    int32_t s_rs[kRing], s_nr[kRing], s_nk[kRing], s_shift[kRing], s_cb[kRing];
    uint2 s_c[kRing];
    T s_v[kRing][4];
    int32_t s_ro[kRing];
    T s_w[kRing];
    double xv[2][4];
    // folded form: p_old at the columns, z and p_old of the lane's own row
    // (gathered with the columns) and x of it (fetched with the entries: it
    // is read nowhere else, so it comes from HBM)
    double pg[FOLD ? 2 : 1][4];
    T oz[FOLD ? 2 : 1], op[FOLD ? 2 : 1], op2[FOLD ? 2 : 1], s_x[FOLD ? kRing : 1];
    t_next = next_live(t_next);
    TileDesc dn{0, 0, 0, 0, 0, 0, 0};
    if (t_next < t_end) dn = tiles[t_next];
    // Slot u takes tile t_next (descriptor dn; past the end, an empty tile
    // whose loads read entry 0, row 0 and offset 0). Every load is issued by
    // every lane, at a clamped offset where the lane has nothing to load:
    // loads that are always issued let the compiler wait for a tile's loads
    // while the later ones stay in flight. What clamped lanes load is never
    // used: their products go to slots the sums do not read, their gathers
    // read x[0], their offsets and w are not stored.
    auto fetch = [&](int u) {
        s_t[u] = t_next;
        TileDesc e{0, 0, 0, 0, 0, 0, 0};
        if (t_next < t_end) e = dn;
        s_rs[u] = e.rs;
        s_nr[u] = e.re - e.rs;
        s_nk[u] = (int)(e.k1 - e.k0);
        s_shift[u] = (int)(e.k0 & 3);
        s_cb[u] = e.cbase;
        const int64_t base = e.k0 & ~(int64_t)3;
        const int span = (int)(e.k1 - base);
        const int g = 4 * lane < span ? 4 * lane : 0;
        s_c[u] = *reinterpret_cast<const uint2 *>(col16 + base + g);
        load4(val + base + g, s_v[u]);
        const int nr = s_nr[u];
        s_ro[u] = (int32_t)roff16[e.rpos + (lane <= nr ? lane : nr)];
        if (FUSED && !FOLD) s_w[u] = w[e.rs + (lane < nr ? lane : 0)];
        // (x only where this launch updates it; else every lane reads x[0],
        // one cached line, so that the load is still always issued)
        if (FOLD) s_x[FOLD ? u : 0] = xx[xstep ? e.rs + (lane < nr ? lane : 0) : 0];
        if (t_next < t_end) t_next = next_live(t_next + stride);
    };
    // the descriptor of the tile the next fetch takes (scalar loads; issued
    // after a tile's sums, it is back by the next fetch)
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
            const int32_t cc = (j >= 0 && j < nk) ? c : 0;
            if (FOLD) {
                xv[hb][k] = (double)zz[cc];
                pg[FOLD ? hb : 0][k] = (double)pold[cc];
            } else {
                xv[hb][k] = (double)x[cc];
            }
        }
        if (FOLD) {
            const int64_t i = s_rs[u] + (lane < s_nr[u] ? lane : 0);
            oz[FOLD ? hb : 0] = zz[i];
            op[FOLD ? hb : 0] = pold[i];
            op2[FOLD ? hb : 0] = pnew[xstep ? i : 0];   // read before this lane writes it
        }
    };
    // the tile of slot u (gathers in xv[hb]): products, row offsets and w to
    // LDS; slot u refilled with the next tile; the gathers of the tile two
    // on issued; the row sums; the next descriptor requested
    auto step = [&](int u, int hb) {
        const int nrows = s_nr[u], shift = s_shift[u], nk = s_nk[u], rs = s_rs[u];
        const int64_t ti = s_t[u];
        {
            const int g = 4 * lane;
            if (FOLD) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xv[hb][q] = (double)fold_p<T>(xv[hb][q], pg[FOLD ? hb : 0][q], beta);
            }
            if (g < nk + shift) {
                double2 *pd = reinterpret_cast<double2 *>(prod + g);
                pd[0] = make_double2((double)s_v[u][0] * xv[hb][0], (double)s_v[u][1] * xv[hb][1]);
                pd[1] = make_double2((double)s_v[u][2] * xv[hb][2], (double)s_v[u][3] * xv[hb][3]);
            }
            if (lane <= nrows) roff[lane] = s_ro[u];
            if (FOLD) {
                if (lane < nrows) {
                    const int hf = FOLD ? hb : 0;
                    const T pn = fold_p<T>((double)oz[hf], (double)op[hf], beta);
                    if (xstep) {
                        T xn = s_x[FOLD ? u : 0];
                        if (ax2 != 0.0) xn = (T)((double)xn + ax2 * (double)op2[hf]);
                        if (ax != 0.0) xn = (T)((double)xn + ax * (double)op[hf]);
                        xx[rs + lane] = xn;
                    }
                    pnew[rs + lane] = pn;
                    pown[lane] = (double)pn;
                }
            } else if (FUSED && lane < nrows) {
                pown[lane] = (double)s_w[u];
            }
        }
        fetch(u);
        gather((u + 2) % kRing, hb);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // groups of G lanes, G the largest power of two with 2 G nrows <= 64
        // (64 for nrows <= 1): 64 / G >= nrows groups, one row each
        int G = 1;
        while (G < 64 && G * 2 * nrows <= 64) G *= 2;
        const int lg = lane & (G - 1);
        const int i = lane / G;
        if (i < nrows) {
            const int a = roff[i] + shift, b = roff[i + 1] + shift;
            constexpr int kSB = kSumBatch;
            double pv[kSB];
#pragma unroll
            for (int q = 0; q < kSB; ++q) {
                const int j = a + lg + q * G;
                pv[q] = prod[j < 4 * 64 - 1 ? j : 4 * 64 - 1];   // clamped; unused past b
            }
            double sm = 0.0;
#pragma unroll
            for (int q = 0; q < kSB; ++q)
                if (a + lg + q * G < b) sm += pv[q];
            for (int j = a + lg + kSB * G; j < b; j += G) sm += prod[j];
            for (int off = G >> 1; off > 0; off >>= 1) sm += __shfl_xor(sm, off, 64);
            if (lg == 0) {
                const T q = (T)sm;
                y[rs + i] = q;
                if (FUSED) dot += pown[i] * (double)q;
                if (DOT == 2) dot2 += (double)q * (double)q;
            }
        }
        if (PERTILE) {
            const double td = wave_sum(dot);
            if (lane == 0 && ti < t_end) tile_dot[ti] = td;
            dot = 0.0;
        }
        load_desc();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // (a wavefront without tiles loads nothing: x and w may be empty)
    if (t_next < t_end) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            fetch(u);
            load_desc();
        }
        gather(0, 0);
        gather(1, 1);
        // The slots hold consecutive tiles of the walk. Four steps per pass
        // while all four slots hold a tile, with no exit between them (a
        // single path through the loop body keeps the compiler's waits for
        // the in-order counter tight); then the at most three tiles left.
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
    if (FUSED && !PERTILE) {
        for (int64_t l = blockIdx.x + (int64_t)threadIdx.x * gridDim.x; l < nlong;
             l += (int64_t)kBlock * gridDim.x) {
            dot += long_dot[l];
            if (DOT == 2) dot2 += long_dot[nlong + l];
        }
        dot = block_sum(dot, lds4);
        if (DOT == 2) dot2 = block_sum(dot2, lds4);
        if (threadIdx.x == 0) {
            spart[(int64_t)(FOLD ? 1 : DOT) * blockIdx.x] = dot;
            if (DOT == 2) spart[2 * (int64_t)blockIdx.x + 1] = dot2;
        }
    }
}

// Single system held by diagonals (Handle.dia_*, M of them): one row per
// lane, kDiaRows rows per lane in flight; every load of a wavefront is 512
// contiguous bytes (a diagonal's values, or the gathered vector at a fixed
// offset from the rows). Each XCD takes a contiguous eighth of the rows
// (workgroup b runs on XCD b % 8) and its workgroups take their row groups
// interleaved, so the XCD streams one stretch of the diagonals and the
// vector lines near +-offset are shared in its L2. A row's sum runs over
// the diagonals in column order (one fused multiply-add each; an absent
// entry is a 0 at a clamped column). DOT 0: y = A x; 1: and the w.y partial
// of each workgroup in spart; 4: the folded direction as in the ring form
// (p_new formed at every gathered column and at the own row, x updated on
// every other launch, p_new.q partials); 2: w.y and y.y partials (BiCGStab),
// spart[2 b] and spart[2 b + 1].
constexpr int kDiaRows = 4;

template <typename T, int M, int DOT>
__global__ __launch_bounds__(kBlock) void k_spmv_dia(
    int64_t n, const int32_t *__restrict__ dia_off, const T *__restrict__ dval,
    const T *__restrict__ x, T *__restrict__ y, const T *__restrict__ w,
    double *__restrict__ spart, const int32_t *__restrict__ status, FoldArgs fa) {
    constexpr bool FOLD = DOT == 4;
    __shared__ double lds4[kWaves];
    if (DOT > 0 && *status != kRunning) return;
    int off[M];
#pragma unroll
    for (int d = 0; d < M; ++d) off[d] = dia_off[d];
    double beta = 0.0, ax = 0.0, ax2 = 0.0;
    bool xstep = false;
    const T *zz = nullptr, *pold = nullptr;
    T *pnew = nullptr, *xx = nullptr;
    if (FOLD) {
        const SysState s0 = *fa.st;
        beta = s0.beta;
        ax = s0.alpha;
        ax2 = s0.alpha2;
        xstep = (s0.iter & 1) != 0;
        const int par = s0.iter & 1;
        zz = (const T *)fa.z;
        pold = (const T *)fa.p[par];
        pnew = (T *)fa.p[par ^ 1];
        xx = (T *)fa.x;
    }
    const int64_t G = gridDim.x;   // a multiple of kXcds
    const int64_t X = G / kXcds, xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int64_t xs = n * xcd / kXcds, xe = n * (xcd + 1) / kXcds;
    const int64_t step = X * kBlock * kDiaRows;
    double dot = 0.0, dot2 = 0.0;
    for (int64_t r0 = xs + jx * kBlock * kDiaRows; r0 < xe; r0 += step) {
        double v[kDiaRows][M], g[kDiaRows][M], gp[FOLD ? kDiaRows : 1][FOLD ? M : 1];
        T oz[kDiaRows], op[kDiaRows], op2[kDiaRows], ox[kDiaRows], ow[kDiaRows];
#pragma unroll
        for (int u = 0; u < kDiaRows; ++u) {
            const int64_t i = r0 + u * kBlock + threadIdx.x;
            const bool in = i < xe;
            const int64_t ii = in ? i : 0;
#pragma unroll
            for (int d = 0; d < M; ++d) {
                int64_t c = i + off[d];
                c = c < 0 ? 0 : (c >= n ? n - 1 : c);
                c = in ? c : 0;
                v[u][d] = in ? (double)dval[dia_slot(d, i, M)] : 0.0;
                if (FOLD) {
                    g[u][d] = (double)zz[c];
                    gp[FOLD ? u : 0][FOLD ? d : 0] = (double)pold[c];
                } else {
                    g[u][d] = (double)x[c];
                }
            }
            if (FOLD) {
                oz[u] = zz[ii];
                op[u] = pold[ii];
                op2[u] = pnew[xstep ? ii : 0];   // read before this lane writes it
                ox[u] = xx[xstep ? ii : 0];
            }
            if (DOT == 1 || DOT == 2) ow[u] = w[ii];
        }
#pragma unroll
        for (int u = 0; u < kDiaRows; ++u) {
            const int64_t i = r0 + u * kBlock + threadIdx.x;
            double acc = 0.0;
#pragma unroll
            for (int d = 0; d < M; ++d) {
                const double gv = FOLD ? (double)fold_p<T>(g[u][d], gp[FOLD ? u : 0][FOLD ? d : 0], beta)
                                       : g[u][d];
                acc = __builtin_fma(v[u][d], gv, acc);
            }
            if (i < xe) {
                const T q = (T)acc;
                y[i] = q;
                if (DOT == 1 || DOT == 2) dot += (double)ow[u] * (double)q;
                if (DOT == 2) dot2 += (double)q * (double)q;
                if (FOLD) {
                    const T pn = fold_p<T>((double)oz[u], (double)op[u], beta);
                    if (xstep) {
                        T xn = ox[u];
                        if (ax2 != 0.0) xn = (T)((double)xn + ax2 * (double)op2[u]);
                        if (ax != 0.0) xn = (T)((double)xn + ax * (double)op[u]);
                        xx[i] = xn;
                    }
                    pnew[i] = pn;
                    dot += (double)pn * (double)q;
                }
            }
        }
    }
    if (DOT > 0) {
        dot = block_sum(dot, lds4);
        if (DOT == 2) dot2 = block_sum(dot2, lds4);
        if (threadIdx.x == 0) {
            spart[(DOT == 2 ? 2 : 1) * (int64_t)blockIdx.x] = dot;
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
// and values, then the gathers), longer rows finish in a loop. Each XCD
// takes a contiguous share of the rows (workgroup b runs on XCD b % 8), so
// stencil neighbours share its L2, and its X workgroups take that share's
// passes interleaved (workgroup j: passes j, j + X, ...), so the XCD reads
// one stretch of the values at a time rather than X of them (on the 512^2 x
// 32 fp32 batch 47.1 -> 46.4 us, the iteration 0.1217 -> 0.1203 ms).
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
    // the XCD's share: X workgroups' rows_block rows (whole passes, so the
    // shares cover the rows), its passes dealt out in turn
    const int64_t G = gridDim.x;  // a multiple of kXcds
    const int64_t X = G / kXcds, xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int64_t pass = (int64_t)J * kBvRows;
    const int64_t xs = xcd * X * rows_block;
    const int64_t r_end = xs + X * rows_block < n ? xs + X * rows_block : n;
    double dot[W];
#pragma unroll
    for (int k = 0; k < W; ++k) dot[k] = 0.0;
    if (any) {
        for (int64_t r0 = xs + jx * pass; r0 < r_end; r0 += X * pass) {
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
        // group sums only: the update finishes the sum (group_total), forms
        // alpha and takes the breakdown test, so this kernel ends without
        // the grid-wide tail
        block_sum_systems<W>(dot, Q, tmp, blk);
        for (int s = t; s < B; s += kBlock)
            store_partial(red.part + (int64_t)blockIdx.x * B + s, blk[s]);
        last_group_sums(red.part, red.gpart, red.sync, gridDim.x, B, tmp, tot);
    }
}

// The folded-direction form of k_spmv_bvec for a per-step batched solve
// (see FoldArgs): one row per lane and pass; the gathers read z and p_old,
// p_new = z + beta_b p_old is formed per system (one fused multiply-add) at
// every gathered column and at the lane's own row, x += alpha_b p_old is
// applied to the own row, and q = A p_new with its p_new.q partials. The
// direction buffers are picked by ctl->fold_iter (updates completed in this
// solve, the same for all systems). A system that has stopped keeps x and
// copies p_old into p_new, so that the newest buffer holds its last
// direction for the final x update.
template <typename T, typename RP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_spmv_bvec_fold(
    int64_t n, int B, int64_t rows_block, const RP *__restrict__ row_ptr,
    const int32_t *__restrict__ col, const T *__restrict__ val, T *__restrict__ y, Red red,
    Ctl *__restrict__ ctl, SysState *__restrict__ st, int32_t *__restrict__ h_running,
    FoldArgs fa) {
    constexpr int W = VecW<T>::W;
    constexpr int E = kBvEntries;
    __shared__ double tmp[4 * kMaxBatch];
    __shared__ double tot[kMaxBatch];
    __shared__ double blk[kMaxBatch];
    // beta and alpha of every system in LDS (read where used: registers are
    // what limits how many wavefronts a CU holds here)
    __shared__ double s_beta[kMaxBatch], s_ax[kMaxBatch];
    if (ctl->n_running == 0) return;
    const int Q = B / W;
    const int t = threadIdx.x;
    const int s0 = (t & (Q - 1)) * W;
    const int J = kBlock / Q;
    const int jr = t / Q;
    for (int b = t; b < B; b += kBlock) {
        s_beta[b] = st[b].beta;
        s_ax[b] = st[b].alpha;
    }
    uint32_t run = 0;   // bit w: system s0 + w still runs
#pragma unroll
    for (int w = 0; w < W; ++w) run |= (st[s0 + w].status == kRunning ? 1u : 0u) << w;
    const bool any = run != 0;
    __syncthreads();
    const int par = ctl->fold_iter & 1;
    const T *zz = (const T *)fa.z;
    const T *pold = (const T *)fa.p[par];
    T *pnew = (T *)fa.p[par ^ 1];
    T *xx = (T *)fa.x;
    auto runs = [&](int w) { return ((run >> w) & 1u) != 0; };
    auto pn = [&](int w, T z, T p) {
        return runs(w) ? fold_p<T>((double)z, (double)p, s_beta[s0 + w]) : p;
    };
    const int64_t G = gridDim.x;  // a multiple of kXcds
    const int64_t lb = (int64_t)(blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;
    const int64_t r_begin = lb * rows_block;
    const int64_t r_end = r_begin + rows_block < n ? r_begin + rows_block : n;
    double dot[W];
#pragma unroll
    for (int k = 0; k < W; ++k) dot[k] = 0.0;
    if (any) {
        for (int64_t ri = r_begin + jr; ri < r_end; ri += J) {
            const int64_t ka = (int64_t)row_ptr[ri], kb = (int64_t)row_ptr[ri + 1];
            int32_t c[E];
            T v[E][W], gz[E][W], gp[E][W], oz[W], op[W], ox[W];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t k = ka + e;
                c[e] = k < kb ? col[k] : 0;
                vload(val + (k < kb ? k : 0) * B + s0, v[e]);
            }
            vload(zz + ri * B + s0, oz);
            vload(pold + ri * B + s0, op);
            vload(xx + ri * B + s0, ox);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                vload(zz + (int64_t)c[e] * B + s0, gz[e]);
                vload(pold + (int64_t)c[e] * B + s0, gp[e]);
            }
            double sum[W];
#pragma unroll
            for (int w = 0; w < W; ++w) sum[w] = 0.0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool in = ka + e < kb;
#pragma unroll
                for (int w = 0; w < W; ++w)
                    if (in) sum[w] += (double)v[e][w] * (double)pn(w, gz[e][w], gp[e][w]);
            }
            for (int64_t k = ka + E; k < kb; ++k) {
                T a[W], bz[W], bp[W];
                const int64_t ck = col[k];
                vload(val + k * B + s0, a);
                vload(zz + ck * B + s0, bz);
                vload(pold + ck * B + s0, bp);
#pragma unroll
                for (int w = 0; w < W; ++w) sum[w] += (double)a[w] * (double)pn(w, bz[w], bp[w]);
            }
            T qv[W], pw[W], xw[W];
#pragma unroll
            for (int w = 0; w < W; ++w) {
                qv[w] = (T)sum[w];
                pw[w] = pn(w, oz[w], op[w]);
                xw[w] = runs(w) ? (T)((double)ox[w] + s_ax[s0 + w] * (double)op[w]) : ox[w];
                dot[w] += (double)pw[w] * (double)qv[w];
            }
            vstore(y + ri * B + s0, qv);
            vstore(pnew + ri * B + s0, pw);
            vstore(xx + ri * B + s0, xw);
        }
    } else {
        // every system of this lane has stopped: carry its directions over
        for (int64_t ri = r_begin + jr; ri < r_end; ri += J) {
            T op[W];
            vload(pold + ri * B + s0, op);
            vstore(pnew + ri * B + s0, op);
        }
    }
    block_sum_systems<W>(dot, Q, tmp, blk);
    for (int s = t; s < B; s += kBlock)
        store_partial(red.part + (int64_t)blockIdx.x * B + s, blk[s]);
    last_group_sums(red.part, red.gpart, red.sync, gridDim.x, B, tmp, tot);   // as k_spmv_bvec
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

bool use_ring(const Handle &h) { return h.all_narrow && h.ring_tiles && h.spmv_ring; }

// the per-step SpMV of a single system held by diagonals
bool use_dia_step(const Handle &h) { return h.dia_m > 0 && h.spmv_dia && h.B == 1 && h.nseg == 0; }

int64_t dia_grid(const Handle &h) {
    const int64_t per = (int64_t)kBlock * kDiaRows;
    int64_t g = (h.n + per - 1) / per;
    g = (g + kXcds - 1) / kXcds * kXcds;
    return g < kDiaGridMax ? g : kDiaGridMax;
}

template <typename T, int DOT>
void launch_dia(Handle &h, const void *x, void *y, const void *w, double *spart,
                const int32_t *status, const FoldArgs &fa, hipStream_t s) {
    const dim3 g((unsigned)dia_grid(h)), b(kBlock);
    if (h.dia_m == 5)
        hipLaunchKernelGGL((k_spmv_dia<T, 5, DOT>), g, b, 0, s, h.n, (const int32_t *)h.dia_off,
                           (const T *)h.dia_val, (const T *)x, (T *)y, (const T *)w, spart, status, fa);
    else
        hipLaunchKernelGGL((k_spmv_dia<T, 7, DOT>), g, b, 0, s, h.n, (const int32_t *)h.dia_off,
                           (const T *)h.dia_val, (const T *)x, (T *)y, (const T *)w, spart, status, fa);
}

const void *ring_kernel(const Handle &h) {
    if (h.vt == SLA_F64)
        return h.rp64 ? (const void *)&k_spmv_tile_ring<double, int64_t, 1>
                      : (const void *)&k_spmv_tile_ring<double, int32_t, 1>;
    return h.rp64 ? (const void *)&k_spmv_tile_ring<float, int64_t, 1>
                  : (const void *)&k_spmv_tile_ring<float, int32_t, 1>;
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
    if (use_ring(h)) {
        hipLaunchKernelGGL((k_spmv_tile_ring<T, RP, DOT>), dim3((unsigned)grid), dim3(kBlock),
                           kRingLdsPad, s,
                           (const TileDesc *)h.tiles, h.ntiles, (const uint16_t *)h.roff16,
                           (const uint16_t *)h.col16, (const T *)h.vals, (const T *)x, (T *)y,
                           (const T *)w, (const double *)h.long_dot, h.nlong, spart, status,
                           (const uint8_t *)h.tile_live, h.tile_dot, h.band_l, h.band_p,
                           FoldArgs{});
        return;
    }
    auto kern = h.all_narrow ? k_spmv_tile<T, RP, DOT, true> : k_spmv_tile<T, RP, DOT, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBlock), 0, s, (const TileDesc *)h.tiles,
                       h.ntiles, (const uint16_t *)h.roff16, (const int32_t *)h.col,
                       (const uint16_t *)h.col16, (const T *)h.vals, (const T *)x, (T *)y,
                       (const T *)w, (const double *)h.long_dot, h.nlong, spart, status,
                       (const uint8_t *)h.tile_live, h.tile_dot, h.band_l, h.band_p);
}

template <typename T, typename RP, bool FUSED>
void launch_spmv_t(Handle &h, const void *x, void *y, hipStream_t s) {
    const Red red{h.part, h.gpart, h.sync + kCntSpmv * kCountersPerKind};
    if (h.B == 1 && use_dia_step(h)) {
        launch_dia<T, FUSED ? 1 : 0>(h, x, y, x, h.spart, &h.st[0].status, FoldArgs{}, s);
    } else if (h.B == 1) {
        launch_tiles<T, RP, FUSED ? 1 : 0>(h, x, y, x, h.spart, &h.st[0].status, s);
    } else if (bvec_ok<T>(h)) {
        const Red red_g{h.part, h.gpart_spmv, h.sync + kCntSpmv * kCountersPerKind};
        hipLaunchKernelGGL((k_spmv_bvec<T, RP, FUSED>), dim3((unsigned)bvec_grid<T, FUSED>(h)),
                           dim3(kBlock), 0, s, h.n, h.B, bvec_rows_block<T, FUSED>(h),
                           (const RP *)h.row_ptr, (const int32_t *)h.col, (const T *)h.vals,
                           (const T *)x, (T *)y, red_g, h.ctl, h.st, h.d_running);
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
        const int64_t res = use_ring(h) ? h.ring_resident : h.spmv_resident;
        g = g < res ? g : res;
        // Band-aligned tiles under the ring SpMV: one panel per XCD. The grid
        // keeps band_l wavefronts per XCD, so the plain walk (wavefront w:
        // tiles T0 + w, T0 + w + band_l, ...) is the band walk over the XCD's
        // whole range, one band after the other: the p lines a tile gathers
        // near +N are used again one and two steps later while only one band
        // of rows per XCD streams in between (with band_p panels side by
        // side, band_p bands' entries and gathers pass through the L2 in that
        // time). On the 133M-row Poisson matrix, 2 panels -> 1: folded SpMV
        // 2.82 -> 2.74 ms.
        if (use_ring(h) && h.band_p > 1 && g % kXcds == 0 && (g / kXcds) % h.band_p == 0 &&
            g / kXcds / h.band_p * kWaves == h.band_l)
            g /= h.band_p;
        return g;
    }
    return h.vt == SLA_F64 ? batched_grid_t<double>(h) : batched_grid_t<float>(h);
}

// Resident capacity of the persistent tile kernel: every workgroup of the
// grid must be on a CU at once, or the later ones start only when earlier
// ones finish and the kernel runs in two rounds.
int64_t resident_workgroups(const void *kernel, int device, size_t dyn_lds) {
    int cus = 0, per_cu = 0;
    SLA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device));
    SLA_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, dyn_lds));
    int64_t g = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    g = g / kXcds * kXcds;
    if (g < kXcds) g = kXcds;
    if (g > kMaxGrid) g = kMaxGrid;
    return g;
}

// Wavefronts per XCD of the tile SpMV when its grid is the resident count (the
// narrow and wide forms have the same occupancy; ring: the ring form's)
int64_t tile_spmv_waves_per_xcd(const Handle &h, bool ring) {
    if (ring) return resident_workgroups(ring_kernel(h), h.device, kRingLdsPad) / kXcds * kWaves;
    const void *fn = h.vt == SLA_F64
                         ? (h.rp64 ? (const void *)&k_spmv_tile<double, int64_t, 1, true>
                                   : (const void *)&k_spmv_tile<double, int32_t, 1, true>)
                         : (h.rp64 ? (const void *)&k_spmv_tile<float, int64_t, 1, true>
                                   : (const void *)&k_spmv_tile<float, int32_t, 1, true>);
    return resident_workgroups(fn, h.device) / kXcds * kWaves;
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
    h.ring_resident = resident_workgroups(ring_kernel(h), h.device, kRingLdsPad);
    if (h.B > 1) {
        auto pick = [&](auto ttag, auto rtag) {
            using T = decltype(ttag);
            using RP = decltype(rtag);
            h.bvec_resident[0] = resident_workgroups((const void *)&k_spmv_bvec<T, RP, false>, h.device);
            h.bvec_resident[1] = resident_workgroups((const void *)&k_spmv_bvec<T, RP, true>, h.device);
            h.bvec_fold_resident = resident_workgroups((const void *)&k_spmv_bvec_fold<T, RP>, h.device);
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

// q = A p fused with the p.q partials and alpha, for one fp64 system held
// only as caller CSR arrays (int32 row_ptr and columns), on caller-given
// buffers (the allocation-free solve): one lane per row, rows_per_lane rows
// per lane so that the grid stays within kMaxGrid (the rows of red.part).
void launch_spmv_csr_dot_raw(int64_t n, const int32_t *row_ptr, const int32_t *col,
                             const double *val, const double *p, double *q, Red red, Ctl *ctl,
                             SysState *st, int32_t *running, hipStream_t s) {
    int rpl = 1;
    while ((n + (int64_t)kBlock * rpl - 1) / ((int64_t)kBlock * rpl) > kMaxGrid) rpl *= 2;
    const int64_t grid = (n + (int64_t)kBlock * rpl - 1) / ((int64_t)kBlock * rpl);
    hipLaunchKernelGGL((k_spmv_batched<double, int32_t, true>), dim3((unsigned)grid), dim3(kBlock),
                       0, s, n, 1, rpl, row_ptr, col, val, p, q, red, ctl, st, running);
    SLA_HIP(hipGetLastError());
}

// The folded-direction SpMV of a per-step single-system solve (see
// FoldArgs): p_new = z + beta p_old, x += alpha p_old on the own rows,
// q = A p_new and the p_new.q partials. Needs use_ring(h) and no long rows.
// grid (and rows per workgroup) of the folded batched SpMV: one row per
// lane and pass, the grid filling the resident workgroups
int64_t bvec_fold_grid(const Handle &h, int64_t *rows_block_out) {
    const int W = h.vt == SLA_F64 ? VecW<double>::W : VecW<float>::W;
    const int64_t J = kBlock / (h.B / W);
    const int64_t slots = (h.n + J - 1) / J;
    const int64_t R = h.bvec_fold_resident > 0 ? h.bvec_fold_resident : kXcds;
    const int64_t rows_block = J * ((slots + R - 1) / R);
    int64_t grid = (h.n + rows_block - 1) / rows_block;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    if (rows_block_out) *rows_block_out = rows_block;
    return grid;
}

// blocks of the batched SpMV the update consumes the group sums of
int64_t bvec_spmv_blocks(const Handle &h) {
    if (h.fold_active) return bvec_fold_grid(h, nullptr);
    return h.vt == SLA_F64 ? bvec_grid<double, true>(h) : bvec_grid<float, true>(h);
}

bool fold_possible(const Handle &h) {
    if (h.nseg > 0) return false;
    if (h.B > 1) return h.vt == SLA_F64 ? bvec_ok<double>(h) : bvec_ok<float>(h);
    return use_dia_step(h) || (h.nlong == 0 && use_ring(h));
}

int64_t spmv_blocks(const Handle &h) { return use_dia_step(h) ? dia_grid(h) : spmv_grid(h); }

void launch_spmv_fold(Handle &h, hipStream_t s) {
    const FoldArgs fa{h.fold_z, {h.p, h.fold_p2}, h.x, h.st};
    if (h.B > 1) {
        int64_t rows_block = 0;
        const int64_t grid = bvec_fold_grid(h, &rows_block);
        const Red red{h.part, h.gpart_spmv, h.sync + kCntSpmv * kCountersPerKind};
        auto go = [&](auto ttag, auto rtag) {
            using T = decltype(ttag);
            using RP = decltype(rtag);
            hipLaunchKernelGGL((k_spmv_bvec_fold<T, RP>), dim3((unsigned)grid), dim3(kBlock), 0, s,
                               h.n, h.B, rows_block, (const RP *)h.row_ptr, (const int32_t *)h.col,
                               (const T *)h.vals, (T *)h.q, red, h.ctl, h.st, h.d_running, fa);
        };
        if (h.vt == SLA_F64) {
            if (h.rp64) go(double(), int64_t());
            else go(double(), int32_t());
        } else {
            if (h.rp64) go(float(), int64_t());
            else go(float(), int32_t());
        }
        SLA_HIP(hipGetLastError());
        return;
    }
    const int64_t grid = spmv_grid(h);
    auto go = [&](auto ttag, auto rtag) {
        using T = decltype(ttag);
        using RP = decltype(rtag);
        hipLaunchKernelGGL((k_spmv_tile_ring<T, RP, 4>), dim3((unsigned)grid), dim3(kBlock),
                           kRingLdsPad, s, (const TileDesc *)h.tiles, h.ntiles,
                           (const uint16_t *)h.roff16, (const uint16_t *)h.col16,
                           (const T *)h.vals, (const T *)nullptr, (T *)h.q, (const T *)nullptr,
                           (const double *)h.long_dot, h.nlong, h.spart, &h.st[0].status,
                           (const uint8_t *)nullptr, (double *)nullptr, h.band_l, h.band_p, fa);
    };
    // fp32 values never fold (a stored z would add an fp32 rounding)
    if (h.vt != SLA_F64) fail(SLA_ERR_HIP, "internal: folded direction with fp32 values");
    if (use_dia_step(h)) {
        launch_dia<double, 4>(h, nullptr, h.q, nullptr, h.spart, &h.st[0].status, fa, s);
        SLA_HIP(hipGetLastError());
        return;
    }
    if (h.rp64) go(double(), int64_t());
    else go(double(), int32_t());
    SLA_HIP(hipGetLastError());
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
        if (use_dia_step(h) && ndot <= 2) {
            if (ndot == 0) launch_dia<T, 0>(h, x, y, w, spart, status, FoldArgs{}, s);
            else if (ndot == 1) launch_dia<T, 1>(h, x, y, w, spart, status, FoldArgs{}, s);
            else launch_dia<T, 2>(h, x, y, w, spart, status, FoldArgs{}, s);
            return;
        }
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

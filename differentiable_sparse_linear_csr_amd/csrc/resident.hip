// Single-system Jacobi-PCG as one cooperative kernel whose vectors stay on
// chip. The recurrence is the textbook PCG of the multi-kernel path (torch-sla,
// pytorch-native CG backend with Jacobi preconditioning; distributed-CG
// paragraph: every tensor stays on the device and the step sizes come from
// global reductions); only where the data lives changes.
//
// One workgroup of kRT = 512 threads per CU at most, all co-resident
// (cooperative launch). Wavefront w owns a contiguous range of at most
// 64 * kRJ rows and holds x, r and p of those rows in registers and dinv in
// its LDS slice for the whole solve (lane l holds rows R0 + l + 64 j). Per
// iteration:
//   A   q = A p over the workgroup's tiles (each wavefront a run of them,
//       weighted by the SIMD slot it holds, walked backwards on every other
//       iteration), gathering p from a global copy,
//       with kRD tiles in flight (the entries of the next tiles and the
//       gathers of the tile two on are loading while a tile is summed); q
//       goes to the LDS slot of its rows' owner; p.q from registers and LDS
//   R1  grid all-reduce of p.q -> alpha, or breakdown
//   B   x += alpha p, r -= alpha q, z = dinv r; r.z and r.r
//   R2  grid all-reduce -> stopping test, iteration budget, beta
//   C   p = z + beta p; own rows written to the global copy
//   R3  barrier: the copy is complete before the next gathers, waiting only
//       for the workgroups that own columns of this workgroup's rows
// so HBM sees the matrix, the p gathers and the p store per iteration.
//
// A batch of B systems sharing the pattern runs as B independent groups of
// workgroups in the same launch: group b solves system b with its own values
// (a batch-major copy made at the start of the solve), its own stamps, its
// own stopping test and iteration count.
//
// All-reduces: every workgroup stores its partials, stamped with a sequence
// number, with device-coherent stores; one wavefront of every workgroup polls
// all stamped partials and sums them itself in one fixed order, so every
// workgroup holds the same bits and takes the same stopping decisions. Polls
// are bounded: a workgroup that waits longer than a set number of polls
// reports a failure instead of hanging (the host then re-runs the solve on
// the per-step kernels).
#include "common.h"

#include <algorithm>
#include <vector>

namespace sla {

namespace {

constexpr int kRT = 512;              // threads per workgroup
constexpr int kRW = kRT / 64;         // wavefronts per workgroup
constexpr int kRJ = 16;               // rows per lane held in registers, at most
// tiles of at most kRUnits rows + entries: with the up-to-3 entries before k0
// of the first 16-byte group, a tile's entries fit one group per lane
constexpr int kRUnits = 4 * 64 - 3;
static_assert(kRUnits < 256, "a tile's row offsets are bytes, at most 4 per lane");
constexpr int kSumBatch = 4;          // LDS reads issued together per row sum (2: 42.9, 6: 43.2, 8: 44.4 us per iteration at 2.1M rows against 42.0)
constexpr double kFastShare = 1.0625;   // tile share of a SIMD's first wavefront (vs 0.9375)
constexpr int kRD = 4;                // tiles in flight per wavefront (even)
constexpr int kResFailed = 100;       // status written when a wait timed out

// sum over the workgroup with a fixed tree (identical in every workgroup)
__device__ __forceinline__ double rblock_sum(double v, double *lds) {
    v = wave_sum(v);
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wv] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kRW; ++w) s += lds[w];
    __syncthreads();
    return s;
}

// two sums over the workgroup at once (one LDS round trip, one tree each)
__device__ __forceinline__ void rblock_sum2(double &a, double &b, double *lds2) {
    a = wave_sum(a);
    b = wave_sum(b);
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        lds2[wv] = a;
        lds2[kRW + wv] = b;
    }
    __syncthreads();
    double sa = 0.0, sb = 0.0;
#pragma unroll
    for (int w = 0; w < kRW; ++w) {
        sa += lds2[w];
        sb += lds2[kRW + w];
    }
    __syncthreads();
    a = sa;
    b = sb;
}

// a value that is the same in every lane, moved to scalar registers
__device__ __forceinline__ double uniform(double v) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
}

struct GridSync {
    uint64_t *slot;      // [2][G][2 * kMaxC] stamped halves of each workgroup's partials
    uint64_t *flag;      // [G] the last barrier each workgroup has arrived at
    const int32_t *dep;  // [G + 1] starts (absolute), then the lists: whose rows a
                         // workgroup's rows read, for each one in row order
    int G;               // workgroups of one system
    int lb;              // this workgroup's index among them
    uint32_t spin_limit; // polls of a wait before it gives up
    int interleave;      // SpMV phase: the workgroup's tiles interleaved over its wavefronts
};
constexpr int kMaxC = 2;
// workgroups one polling lane covers: a system has at most 64 * kPollSlots
// workgroups, so every poll round issues all its loads before waiting on any
constexpr int kPollSlots = 4;

// Grid all-reduce of C values (block totals, valid in every thread).
// A partial travels as two 64-bit words, (seq << 32 | upper half) and
// (seq << 32 | lower half), each written and read single-copy atomically,
// so a poll that sees both stamps equal to seq has the partial: arrival and
// value arrive in one round trip, with no separate flag and no ordering
// between the two stores. Slots alternate with the parity of seq: a
// workgroup rewrites a slot only after every workgroup has passed the next
// all-reduce, i.e. has read this one. With `publish`, every global store this
// workgroup made before the call is complete before its partials are written,
// so other workgroups see that data once they return. Returns false on a
// timed-out wait.
template <int C>
__device__ __forceinline__ bool grid_allreduce(const GridSync &gs, uint32_t seq, const double (&v)[C],
                                               double (&tot)[C], double *lds, bool publish) {
    const int t = threadIdx.x;
    uint64_t *slot = gs.slot + (size_t)(seq & 1u) * gs.G * (2 * kMaxC);
    if (publish) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    const uint64_t stamp = (uint64_t)seq << 32;
    if (t < 2 * C) {
        const uint64_t bits = (uint64_t)__double_as_longlong(v[t >> 1]);
        const uint64_t half = (t & 1) ? (bits & 0xffffffffull) : (bits >> 32);
        __hip_atomic_store(slot + gs.lb * (2 * kMaxC) + t, stamp | half, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // wavefront 0 polls every partial (lane l: workgroups l, l + 64, ...)
    // until all carry this stamp, and sums them: lane l in workgroup order,
    // then the wavefront tree, the same in every workgroup
    if (t < 64) {
        uint32_t spins = 0;
        double a[C];
        bool done = false;
        while (true) {
            bool arrived = true;
#pragma unroll
            for (int c = 0; c < C; ++c) a[c] = 0.0;
            // a slot past G reads as arrived +0.0, which leaves the sum's bits
            // unchanged (it starts at +0.0, so it is never -0.0)
            uint64_t w[kPollSlots][2 * C];
#pragma unroll
            for (int i = 0; i < kPollSlots; ++i) {
                const int q = t + 64 * i;
#pragma unroll
                for (int k = 0; k < 2 * C; ++k)
                    w[i][k] = q < gs.G ? __hip_atomic_load(slot + q * (2 * kMaxC) + k, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT)
                                       : stamp;
            }
#pragma unroll
            for (int i = 0; i < kPollSlots; ++i) {
#pragma unroll
                for (int k = 0; k < 2 * C; ++k) arrived &= (w[i][k] >> 32) == seq;
#pragma unroll
                for (int c = 0; c < C; ++c)
                    a[c] += __longlong_as_double((int64_t)(((w[i][2 * c] & 0xffffffffull) << 32) |
                                                           (w[i][2 * c + 1] & 0xffffffffull)));
            }
            if (__all(arrived)) {
                done = true;
                break;
            }
            if (++spins > gs.spin_limit) break;
            __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) a[c] = wave_sum(a[c]);
        if (t == 0) {
#pragma unroll
            for (int c = 0; c < C; ++c) lds[c] = a[c];
            lds[kMaxC] = done ? 1.0 : 0.0;
        }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) tot[c] = uniform(lds[c]);
    const bool arrived_all = lds[kMaxC] != 0.0;
    __syncthreads();
    if (!arrived_all) return false;
    return true;
}

// Point-to-point barrier: every global store this workgroup made before the
// call is complete, then it stamps its flag with bseq and waits only for the
// workgroups its rows read from (list L of gs.dep, launch indices) to stamp
// theirs. A workgroup stamps its flag again only after the next all-reduce,
// which it cannot pass before every other workgroup has left this wait, so
// one flag per workgroup suffices. Returns false on a timed-out wait.
__device__ __forceinline__ bool grid_wait_deps(const GridSync &gs, uint32_t bseq, int L, double *lds) {
    const int t = threadIdx.x;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0)
        __hip_atomic_store(gs.flag + gs.lb, (uint64_t)bseq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t < 64) {
        const int d0 = gs.dep[L], d1 = gs.dep[L + 1];
        uint32_t spins = 0;
        bool done = false;
        while (true) {
            bool arrived = true;
            uint64_t f[kPollSlots];
#pragma unroll
            for (int i = 0; i < kPollSlots; ++i) {
                const int q = d0 + t + 64 * i;
                f[i] = q < d1 ? __hip_atomic_load(gs.flag + gs.dep[q], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : (uint64_t)bseq;
            }
#pragma unroll
            for (int i = 0; i < kPollSlots; ++i) arrived &= f[i] == (uint64_t)bseq;
            if (__all(arrived)) {
                done = true;
                break;
            }
            if (++spins > gs.spin_limit) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (t == 0) lds[kMaxC] = done ? 1.0 : 0.0;
    }
    __syncthreads();
    const bool ok = lds[kMaxC] != 0.0;
    __syncthreads();
    return ok;
}

template <typename T>
__device__ __forceinline__ void store_shared(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// System sys = blockIdx.x / G of B: values val + sys * vstride (batch-major),
// dinv[row * B + sys] (the internal interleaved layout), b, x_out and the
// global p copy pg at sys * n, stamps at sys * 2 * G * 2 * kMaxC, st[sys].
template <typename T, bool NARROW, int DIA>
__global__ __launch_bounds__(kRT, 1) void k_cg_resident(
    const ResTile *__restrict__ tiles, const int32_t *__restrict__ wave_row0,
    const int32_t *__restrict__ wave_tile0, const uint8_t *__restrict__ roff8,
    const int32_t *__restrict__ col, const uint16_t *__restrict__ col16,
    const T *__restrict__ val_all, int64_t vstride,
    const T *__restrict__ dinv_all, const T *__restrict__ b_all, T *__restrict__ x_all,
    T *pg_all, GridSync gs, int B, int64_t n, double tol, int32_t maxit,
    SysState *__restrict__ st_all, const int32_t *__restrict__ dia_off, int dia_m,
    const T *__restrict__ dia_val) {
    __shared__ __align__(16) double prod_all[kRW][4 * 64];
    __shared__ __align__(16) int32_t roff_all[kRW][256];
    __shared__ T qbuf_all[kRW][64 * kRJ];
    __shared__ T dinv_lds_all[kRW][64 * kRJ];
    __shared__ double lds[2 * kRW];

    const int sys = blockIdx.x / gs.G;
    const int lbk = blockIdx.x - sys * gs.G;   // index inside the system's group
    const T *__restrict__ val = val_all + (int64_t)sys * vstride;
    const T *__restrict__ b = b_all + (int64_t)sys * n;
    T *__restrict__ x_out = x_all + (int64_t)sys * n;
    T *pg = pg_all + (int64_t)sys * n;
    SysState *__restrict__ st = st_all + sys;
    gs.slot += (size_t)sys * 2 * gs.G * (2 * kMaxC);
    gs.flag += (size_t)sys * gs.G;
    gs.lb = lbk;

    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar registers): the row range, the tile range and
    // every tile descriptor then come through scalar loads
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD-contiguous order: workgroup b runs on XCD b % 8 (G is a multiple of
    // 8, so the same holds inside every group); each XCD takes one contiguous
    // eighth of the rows, so halo lines are shared inside its L2
    const int lb = (lbk % kXcds) * (gs.G / kXcds) + lbk / kXcds;
    const int w = lb * kRW + wv;
    const int R0 = wave_row0[w], R1 = wave_row0[w + 1];
    // the wavefront's tiles: t0, t0 + ts, ... (nt of them). A contiguous run
    // of the workgroup's tiles (the plan gives a SIMD's first wavefront the
    // larger share), or, interleaved, every kRW-th one from the wavefront's
    // index, so that the workgroup's wavefronts read neighbouring tiles at
    // once: a CU then streams one stretch of the matrix, not kRW of them,
    // which helps where the matrix comes from HBM (on the 2M-point kNN
    // matrix 31.0 -> 29.4 ms per solve; no change where it stays in the
    // Infinity Cache). The same tiles and sums either way.
    int t0 = wave_tile0[w], nt = wave_tile0[w + 1] - t0, ts = 1;
    if (gs.interleave) {
        const int g0 = wave_tile0[lb * kRW], gn = wave_tile0[lb * kRW + kRW] - g0;
        t0 = g0 + wv;
        nt = gn > wv ? (gn - wv + kRW - 1) / kRW : 0;
        ts = kRW;
    }
    double *prod = prod_all[wv];
    int32_t *roff = roff_all[wv];
    // q of the workgroup's rows (wavefront v's rows in qbuf_all[v]); a tile
    // may be summed by another wavefront of the workgroup than its rows'
    // owner, and its descriptor gives its first row's slot
    T *qwg = &qbuf_all[0][0];
    T *qbuf = qbuf_all[wv];
    T *ql = qbuf + lane;             // this lane's rows: ql[64 j]
    T *pgl = pg + R0 + lane;          // and their global p: pgl[64 j]
    T *dl = dinv_lds_all[wv] + lane;  // and their dinv: dl[64 j]
    const int nl = R1 - R0 - lane;    // row j of this lane exists iff 64 j < nl

    // Register arrays are updated unconditionally (a lane's rows past the
    // wavefront's range hold zeros and contribute nothing); only global
    // accesses are masked. Conditional writes to the arrays would make the
    // compiler copy them whole.
    for (int j = lane; j < 64 * kRJ; j += 64) qbuf[j] = (T)0;
    T xr[kRJ], rr[kRJ], pr[kRJ];
    double s_bb = 0.0, s_rz = 0.0;
#pragma unroll
    for (int j = 0; j < kRJ; ++j) {
        const bool in = 64 * j < nl;
        const T bv = in ? b[R0 + lane + 64 * j] : (T)0;
        const T dv = in ? dinv_all[(int64_t)(R0 + lane + 64 * j) * B + sys] : (T)0;
        dl[64 * j] = dv;
        rr[j] = bv;
        xr[j] = (T)0;
        const double z = (double)dv * (double)bv;
        pr[j] = (T)z;
        if (in) store_shared(pgl + 64 * j, pr[j]);
        s_bb += (double)bv * (double)bv;
        s_rz += (double)bv * z;
    }
    uint32_t seq = 1, bseq = 1;
    bool ok;
    double bb, rho;
    {
        rblock_sum2(s_bb, s_rz, lds);
        const double v[2] = {s_bb, s_rz};
        double tot[2];
        ok = grid_allreduce<2>(gs, seq++, v, tot, lds, true);
        bb = tot[0];
        rho = tot[1];
    }
    int status = bb == 0.0 ? SLA_CONVERGED : (maxit <= 0 ? SLA_MAXIT : kRunning);
    int iter = 0;
    double rrv = bb, alpha = 0.0, beta = 0.0;
    const double thresh = tol * sqrt(bb);

    // ring of kRD tiles: slot u holds the entries (columns, values, row
    // offsets relative to k0) of the wavefront's tiles i with i % kRD == u,
    // as loaded (no arithmetic on them before they are used, so no load is
    // waited for early); xv[h] holds the gathered p of tile i with
    // i % 2 == h. Tile i's entries are requested kRD steps and its gathers
    // two steps before it is summed. Columns are 16-bit offsets from the
    // tile's smallest one (NARROW) or 32-bit; row offsets are bytes, lane l
    // holding those of rows 4 l .. 4 l + 3.
    int32_t cs[kRD][NARROW ? 2 : 4];
    T vs[kRD][4];
    uint32_t ros[kRD];
    int32_t d_nr[kRD], d_nk[kRD], d_k0[kRD], d_cb[kRD], d_qb[kRD];
    double xv[2][4];
    auto fetch = [&](int u, const ResTile &e) {
        const int nr = (int)(e.packed & 0xffu);
        d_nr[u] = nr;
        d_nk[u] = (int)((e.packed >> 8) & 0xffu);
        d_k0[u] = e.k0;
        d_cb[u] = e.cbase;
        d_qb[u] = (int)(e.packed >> 16);
        const int64_t base = (int64_t)(e.k0 & ~3);
        const int span = (int)(e.k0 + d_nk[u] - base);
        const int g = 4 * lane;
        if (g < span) {
            if constexpr (NARROW) {
                const uint2 raw = *reinterpret_cast<const uint2 *>(col16 + base + g);
                cs[u][0] = (int32_t)raw.x;
                cs[u][1] = (int32_t)raw.y;
            } else {
                load4(col + base + g, cs[u]);
            }
            load4(val + base + g, vs[u]);
        } else {
#pragma unroll
            for (int k = 0; k < (NARROW ? 2 : 4); ++k) cs[u][k] = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) vs[u][k] = (T)0;
        }
        ros[u] = g <= nr ? *reinterpret_cast<const uint32_t *>(roff8 + e.rpos + g) : 0u;
    };
    // masked lanes read pg[0]
    auto gather = [&](int u, int h) {
        const int shift = d_k0[u] & 3;
        const int nk = d_nk[u];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = 4 * lane + k - shift;
            int32_t c;
            if constexpr (NARROW)
                c = d_cb[u] + (int32_t)(((uint32_t)cs[u][k >> 1] >> (16 * (k & 1))) & 0xffffu);
            else
                c = cs[u][k];
            xv[h][k] = (double)pg[(j >= 0 && j < nk) ? c : 0];
        }
    };

    // the matrix does not change: the entries of the first kRD tiles are
    // loaded before the loop and again at the end of every SpMV phase, for
    // the next iteration, while the all-reduces and updates run
    auto fetch_head = [&]() {
#pragma unroll
        for (int u = 0; u < kRD; ++u)
            if (u < nt) fetch(u, tiles[t0 + u * ts]);
    };
    // DIA (the number of diagonals, or 0): their offsets (wave-uniform) and
    // the walk direction
    constexpr int ND = DIA > 0 ? DIA : 1;
    int doff[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) doff[d] = DIA > 0 ? dia_off[d] : 0;
    const int n32 = (int)n;   // m n < 2^31 for a matrix held by diagonals
    bool back = false;
    if (!DIA) fetch_head();
    while (ok && status == kRunning) {
        // p written by other workgroups (other XCDs) since these caches last
        // held it: drop stale lines before gathering. The CU's L1 and the
        // XCD's L2 are shared by the workgroup's wavefronts, so one of them
        // invalidates (an invalidation per wavefront costs ~13 us per
        // iteration on a full chip) and the barrier orders the others after it.
        if (wv == 0) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        if constexpr (DIA > 0) {
        // ---- A by diagonals: lane l sums its rows R0 + l + 64 j over the
        // diagonals in column order, q_i = sum_d val[d][i] p[i + off_d],
        // into its own LDS slots; two row groups' loads (values and
        // gathers, all coalesced) in flight at a time, the groups walked
        // backwards on every other iteration. A row without an entry on a
        // diagonal holds 0 there (its column clamped into the matrix).
#pragma unroll 1
        for (int jj = 0; jj < kRJ; jj += 2) {
            const int jb = back ? kRJ - 2 - jj : jj;
            if (64 * jb >= R1 - R0) {   // wave-uniform: no rows of this wavefront there
                if (back) continue;
                break;
            }
            double dv2[2][ND], dg2[2][ND];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int j = jb + h2;
                const bool in = 64 * j < nl;
                const int i = R0 + lane + 64 * j;
#pragma unroll
                for (int d = 0; d < ND; ++d) {
                    int c = i + doff[d];
                    c = c < 0 ? 0 : (c >= n32 ? n32 - 1 : c);
                    dv2[h2][d] = in ? (double)dia_val[dia_slot(d, i, ND)] : 0.0;
                    dg2[h2][d] = (double)pg[in ? c : 0];
                }
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int j = jb + h2;
                double acc = 0.0;
#pragma unroll
                for (int d = 0; d < ND; ++d) acc = __builtin_fma(dv2[h2][d], dg2[h2][d], acc);
                if (64 * j < nl) ql[64 * j] = (T)acc;
            }
        }
        back = !back;
        } else {
        // ---- A: q = A p on this wavefront's tiles, into its LDS slice (the
        // entries of its first kRD tiles are already in the ring)
        if (nt > 0) gather(0, 0);
        if (nt > 1) gather(1, 1);
        // descriptor of the tile fetched next, read one step before its fetch
        ResTile en = kRD < nt ? tiles[t0 + kRD * ts] : ResTile{0, 0, 0, 0};
        for (int i0 = 0; i0 < nt; i0 += kRD) {
#pragma unroll
            for (int u = 0; u < kRD; ++u) {
                const int i = i0 + u;
                if (i >= nt) break;
                const ResTile ef = en;
                if (i + kRD + 1 < nt) en = tiles[t0 + (i + kRD + 1) * ts];
                const int nrows = d_nr[u];
                const int qb = d_qb[u];
                const int shift = d_k0[u] & 3;
                // products at their place in the lane's 16-byte group (entry
                // k0 of the tile is prod[shift]); lanes write 32 consecutive
                // bytes each, the row offsets 16 (no bank conflicts). Slots
                // outside [k0, k1) hold products nobody reads.
                {
                    double2 *pd = reinterpret_cast<double2 *>(prod + 4 * lane);
                    pd[0] = make_double2((double)vs[u][0] * xv[u & 1][0], (double)vs[u][1] * xv[u & 1][1]);
                    pd[1] = make_double2((double)vs[u][2] * xv[u & 1][2], (double)vs[u][3] * xv[u & 1][3]);
                    const uint32_t rw = ros[u];
                    int4 q4;
                    q4.x = (int32_t)(rw & 0xffu) + shift;
                    q4.y = (int32_t)((rw >> 8) & 0xffu) + shift;
                    q4.z = (int32_t)((rw >> 16) & 0xffu) + shift;
                    q4.w = (int32_t)(rw >> 24) + shift;
                    *reinterpret_cast<int4 *>(roff + 4 * lane) = q4;
                }
                // slot u and xv[u & 1] are free again: tile i + kRD's
                // entries and tile i + 2's gathers load during the sums
                if (i + kRD < nt) fetch(u, ef);
                if (i + 2 < nt) gather((u + 2) % kRD, u & 1);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                int G = 1;
                while (G < 64 && G * 2 * nrows <= 64) G *= 2;
                const int lg = lane & (G - 1);
                const int grp = lane / G;
                const int ngrp = 64 / G;
                for (int r = grp; r < nrows; r += ngrp) {
                    const int a = roff[r], e = roff[r + 1];
                    // the lane's first kSumBatch entries are read together,
                    // then added in order
                    double pv[kSumBatch];
#pragma unroll
                    for (int q = 0; q < kSumBatch; ++q) {
                        const int j = a + lg + q * G;
                        pv[q] = prod[j < 4 * 64 - 1 ? j : 4 * 64 - 1];   // clamped; unused past e
                    }
                    double sm = 0.0;
#pragma unroll
                    for (int q = 0; q < kSumBatch; ++q)
                        if (a + lg + q * G < e) sm += pv[q];
                    for (int j = a + lg + kSumBatch * G; j < e; j += G) sm += prod[j];
                    for (int off = G >> 1; off > 0; off >>= 1) sm += __shfl_xor(sm, off, 64);
                    if (lg == 0) qwg[qb + r] = (T)sm;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        // The tiles are walked forwards and backwards on alternate
        // iterations, so that each SpMV phase starts on the lines the last
        // one read most recently, which the Infinity Cache may still hold
        // where the whole matrix does not fit it (on the 2M-point kNN
        // matrix, 378 MB as held here: 110 -> 95 us per iteration; at 2.1M
        // rows of 3D diffusion, which fits, 0.3-1 us less of ~40). Each
        // tile's sums do not depend on the order: the results are the same
        // bits.
        if (nt > 0) {
            t0 += (nt - 1) * ts;
            ts = -ts;
        }
        fetch_head();
        }
        // q rows summed by other wavefronts
        __syncthreads();
        // ---- sigma = p.q
        double s_pq = 0.0;
#pragma unroll
        for (int j = 0; j < kRJ; ++j) {
            s_pq += (double)pr[j] * (double)ql[64 * j];
        }
        double sigma;
        {
            const double vv[1] = {rblock_sum(s_pq, lds)};
            double tot[1];
            ok = grid_allreduce<1>(gs, seq++, vv, tot, lds, false);
            sigma = tot[0];
        }
        if (!ok) break;
        if (!(sigma > 0.0) || !isfinite(sigma)) {
            status = SLA_BREAKDOWN;
            iter += 1;
            break;
        }
        alpha = rho / sigma;
        // ---- B: x += alpha p, r -= alpha q, z = dinv r; r.z and r.r
        double s_rz2 = 0.0, s_rr = 0.0;
#pragma unroll
        for (int j = 0; j < kRJ; ++j) {
            const T qv = ql[64 * j];
            xr[j] = (T)((double)xr[j] + alpha * (double)pr[j]);
            rr[j] = (T)((double)rr[j] - alpha * (double)qv);
            const double z = (double)dl[64 * j] * (double)rr[j];
            s_rz2 += (double)rr[j] * z;
            s_rr += (double)rr[j] * (double)rr[j];
        }
        double rz;
        {
            rblock_sum2(s_rz2, s_rr, lds);
            const double vv[2] = {s_rz2, s_rr};
            double tot[2];
            ok = grid_allreduce<2>(gs, seq++, vv, tot, lds, false);
            rz = tot[0];
            rrv = tot[1];
        }
        if (!ok) break;
        iter += 1;
        if (sqrt(rrv) <= thresh) {
            status = SLA_CONVERGED;
            break;
        }
        if (iter >= maxit) {
            status = SLA_MAXIT;
            break;
        }
        beta = rz / rho;
        rho = rz;
        // ---- C: p = z + beta p, own rows to the global copy. The base is
        // redefined here so that the compiler forms the row addresses in this
        // phase instead of keeping all of them live across the loop.
        T *pw = pgl;
        __asm__ volatile("" : "+v"(pw));
#pragma unroll
        for (int j = 0; j < kRJ; ++j) {
            pr[j] = (T)((double)dl[64 * j] * (double)rr[j] + beta * (double)pr[j]);
            if (64 * j < nl) store_shared(pw + 64 * j, pr[j]);
        }
        // only the workgroups whose rows the next product reads need to
        // have written theirs
        ok = grid_wait_deps(gs, bseq++, lb, lds);
    }
#pragma unroll
    for (int j = 0; j < kRJ; ++j)
        if (64 * j < nl) x_out[R0 + lane + 64 * j] = xr[j];
    if (lbk == 0 && threadIdx.x == 0) {
        SysState s;
        s.bb = bb;
        s.rho = rho;
        s.alpha = alpha;
        s.alpha2 = 0.0;
        s.beta = beta;
        s.rr = rrv;
        s.iter = iter;
        s.status = ok ? status : kResFailed;
        *st = s;
    }
}

// out[b * stride + k] = vals[k * B + b]
template <typename T>
__global__ __launch_bounds__(kBlock) void k_vals_bm(const T *__restrict__ vals, int64_t nnz, int B,
                                                    T *__restrict__ out, int64_t stride) {
    const int64_t total = nnz * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t k = f / B;
        const int b = (int)(f - k * B);
        out[(int64_t)b * stride + k] = vals[f];
    }
}

bool use_dia(const Handle &h) {
    return h.dia_m > 0 && h.res_dia_on && h.res_dia_fits && h.B == 1;
}

// the form by diagonals for m diagonals (the 2D and 3D stencils' counts)
template <typename T>
const void *dia_kernel(int m) {
    return m == 5 ? (const void *)&k_cg_resident<T, false, 5>
                  : (const void *)&k_cg_resident<T, false, 7>;
}

const void *kernel_for(const Handle &h) {
    if (h.vt == SLA_F64) {
        if (use_dia(h)) return dia_kernel<double>(h.dia_m);
        return h.res_narrow ? (const void *)&k_cg_resident<double, true, 0>
                            : (const void *)&k_cg_resident<double, false, 0>;
    }
    if (use_dia(h)) return dia_kernel<float>(h.dia_m);
    return h.res_narrow ? (const void *)&k_cg_resident<float, true, 0>
                        : (const void *)&k_cg_resident<float, false, 0>;
}

template <typename RP>
void build_plan(Handle &h, int64_t G, int64_t rpw, hipStream_t s) {
    const int64_t n = h.n;
    const int64_t waves = G * kRW;
    std::vector<RP> rp((size_t)n + 1);
    std::vector<int32_t> col((size_t)h.nnz);
    SLA_HIP(hipMemcpyAsync(rp.data(), h.row_ptr, sizeof(RP) * (size_t)(n + 1),
                           hipMemcpyDeviceToHost, s));
    if (h.nnz > 0)
        SLA_HIP(hipMemcpyAsync(col.data(), h.col, sizeof(int32_t) * (size_t)h.nnz,
                               hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    std::vector<int32_t> wave((size_t)(2 * (waves + 1)));
    std::vector<TileDesc> tiles;
    tiles.reserve((size_t)(n / 16 + waves + 1));
    // row offsets of every tile as bytes, each tile's run starting at a
    // multiple of 4 (rpos)
    std::vector<uint8_t> roff8;
    roff8.reserve((size_t)(n + 4 * (n / 16 + waves + 1)));
    bool narrow = true;
    for (int64_t w = 0; w <= waves; ++w) {
        const int64_t r0 = w * rpw < n ? w * rpw : n;
        wave[(size_t)w] = (int32_t)r0;
        wave[(size_t)(waves + 1 + w)] = (int32_t)tiles.size();
        if (w == waves) break;
        const int64_t r1 = (w + 1) * rpw < n ? (w + 1) * rpw : n;
        // tiles of at most kRUnits rows + entries inside [r0, r1) (a lone row
        // has at most kLongRow entries, well within one group per lane)
        int64_t a = r0;
        while (a < r1) {
            int64_t e = a + 1;
            while (e < r1 && (e + 1 - a) + (int64_t)(rp[(size_t)e + 1] - rp[(size_t)a]) <= kRUnits)
                ++e;
            const int64_t k0 = (int64_t)rp[(size_t)a], k1 = (int64_t)rp[(size_t)e];
            int32_t mn = 0, mx = 0;
            for (int64_t k = k0; k < k1; ++k) {
                const int32_t c = col[(size_t)k];
                if (k == k0 || c < mn) mn = c;
                if (k == k0 || c > mx) mx = c;
            }
            if ((int64_t)mx - (int64_t)mn >= 65536) narrow = false;
            const int64_t rpos = (int64_t)roff8.size();
            for (int64_t r = a; r <= e; ++r) roff8.push_back((uint8_t)(rp[(size_t)r] - (RP)k0));
            while (roff8.size() % 4) roff8.push_back(0);
            // narrow: the slot of row a in the workgroup's q buffer (wavefront
            // w % kRW holds its rows from kRJ * 64 * (w % kRW))
            const int32_t qslot = (int32_t)((w % kRW) * 64 * kRJ + (a - r0));
            tiles.push_back(TileDesc{(int32_t)a, (int32_t)e, k0, k1, rpos, mn, qslot});
            a = e;
        }
    }
    // Which wavefront sums which tiles: a workgroup's tiles are re-split among
    // its wavefronts by rows + entries, the first wavefront of each SIMD
    // (kRW / 2 of them, older, more issue slots) taking kFastShare of an even
    // share and the second the rest, so that the two finish together. Row
    // ownership (x, r, p in registers) does not change; a tile's q goes to
    // its owner's slot.
    for (int64_t g = 0; g < waves / kRW; ++g) {
        const int64_t ta = wave[(size_t)(waves + 1 + g * kRW)];
        const int64_t tb = wave[(size_t)(waves + 1 + (g + 1) * kRW)];
        std::vector<double> cum((size_t)(tb - ta + 1), 0.0);
        for (int64_t t = ta; t < tb; ++t) {
            const TileDesc &d = tiles[(size_t)t];
            cum[(size_t)(t - ta + 1)] = cum[(size_t)(t - ta)] + (double)(d.re - d.rs) + (double)(d.k1 - d.k0);
        }
        const double total = cum.back();
        double acc = 0.0;
        int64_t t = ta;
        for (int v = 1; v < kRW; ++v) {
            acc += (v - 1 < kRW / 2 ? kFastShare : 2.0 - kFastShare) / kRW;
            while (t < tb && cum[(size_t)(t - ta + 1)] <= acc * total + 0.5 * (cum[(size_t)(t - ta + 1)] - cum[(size_t)(t - ta)]))
                ++t;
            wave[(size_t)(waves + 1 + g * kRW + v)] = (int32_t)t;
        }
    }
    // For the barrier before each product: for every workgroup (rows
    // [L per, (L + 1) per)), the other workgroups owning a column of its rows,
    // as launch indices (logical L runs as (L % (G / 8)) * 8 + L / (G / 8))
    {
        const int64_t per = rpw * kRW, X = G / kXcds;
        const size_t base = wave.size();
        wave.resize(base + (size_t)G + 1);
        std::vector<int64_t> seen((size_t)G, -1);
        for (int64_t L = 0; L < G; ++L) {
            wave[base + (size_t)L] = (int32_t)(wave.size() - base);
            const int64_t ra = L * per < n ? L * per : n, rb = (L + 1) * per < n ? (L + 1) * per : n;
            std::vector<int32_t> list;
            for (int64_t k = (int64_t)rp[(size_t)ra]; k < (int64_t)rp[(size_t)rb]; ++k) {
                const int64_t o = col[(size_t)k] / per;
                if (o != L && seen[(size_t)o] != L) {
                    seen[(size_t)o] = L;
                    list.push_back((int32_t)((o % X) * kXcds + o / X));
                }
            }
            std::sort(list.begin(), list.end());
            wave.insert(wave.end(), list.begin(), list.end());
        }
        wave[base + (size_t)G] = (int32_t)(wave.size() - base);
    }
    // a lane reads 4 bytes at rpos + 4 l for 4 l <= the tile's row count
    roff8.resize(roff8.size() + 256, 0);
    h.res_narrow = narrow;
    if (narrow) {
        // columns as offsets from their tile's smallest one; the 16-byte
        // groups a tile reads start up to 3 entries before its first
        std::vector<uint16_t> c16((size_t)h.nnz + 8, 0);
        for (const TileDesc &t : tiles)
            for (int64_t k = t.k0; k < t.k1; ++k)
                c16[(size_t)k] = (uint16_t)(col[(size_t)k] - t.cbase);
        h.res_col16 = (uint16_t *)dalloc(h, sizeof(uint16_t) * c16.size());
        SLA_HIP(hipMemcpyAsync(h.res_col16, c16.data(), sizeof(uint16_t) * c16.size(),
                               hipMemcpyHostToDevice, s));
        SLA_HIP(hipStreamSynchronize(s));
    }
    h.res_roff8 = (uint8_t *)dalloc(h, roff8.size());
    SLA_HIP(hipMemcpyAsync(h.res_roff8, roff8.data(), roff8.size(), hipMemcpyHostToDevice, s));
    std::vector<ResTile> rt(tiles.size());
    for (size_t t = 0; t < tiles.size(); ++t) {
        const TileDesc &d = tiles[t];
        rt[t] = ResTile{(int32_t)d.k0, d.cbase, (int32_t)d.rpos,
                        (uint32_t)(d.re - d.rs) | ((uint32_t)(d.k1 - d.k0) << 8) |
                            ((uint32_t)d.narrow << 16)};
    }
    h.res_tiles = (ResTile *)dalloc(h, sizeof(ResTile) * (rt.size() + 1));
    h.res_wave = (int32_t *)dalloc(h, sizeof(int32_t) * wave.size());
    h.res_slot = (uint64_t *)dalloc(h, sizeof(uint64_t) * (size_t)(2 * G * 2 * kMaxC + G) * h.B);
    if (h.B > 1)
        h.res_vals = dalloc(h, (size_t)((h.nnz + 31) / 32 * 32) * h.B * h.vbytes + 256);
    if (!rt.empty())
        SLA_HIP(hipMemcpyAsync(h.res_tiles, rt.data(), sizeof(ResTile) * rt.size(),
                               hipMemcpyHostToDevice, s));
    SLA_HIP(hipMemcpyAsync(h.res_wave, wave.data(), sizeof(int32_t) * wave.size(),
                           hipMemcpyHostToDevice, s));
    SLA_HIP(hipStreamSynchronize(s));
}

// false when the cooperative launch is refused: not all workgroups can run
// at once now (CUs taken by other work), or another process holds the
// device's cooperative-launch resource
template <typename T>
bool launch(Handle &h, const void *b, void *x, double tol, int32_t maxit, hipStream_t s) {
    const int64_t waves = h.res_grid * kRW;
    const ResTile *tiles = h.res_tiles;
    const int32_t *wrow = h.res_wave;
    const int32_t *wtile = h.res_wave + waves + 1;
    const uint8_t *roff8 = h.res_roff8;
    const int32_t *col = h.col;
    const uint16_t *col16 = h.res_col16;
    const T *val = (const T *)h.vals;
    int64_t vstride = 0;
    if (h.B > 1) {
        // batch-major values, each system's row 256-byte aligned
        vstride = (h.nnz + 31) / 32 * 32;
        if (h.nnz > 0) {
            int64_t g = (h.nnz * h.B + kBlock - 1) / kBlock;
            if (g > 4 * kMaxGrid) g = 4 * kMaxGrid;
            hipLaunchKernelGGL(k_vals_bm<T>, dim3((unsigned)g), dim3(kBlock), 0, s,
                               (const T *)h.vals, h.nnz, h.B, (T *)h.res_vals, vstride);
            SLA_HIP(hipGetLastError());
        }
        val = (const T *)h.res_vals;
    }
    const T *dinv = (const T *)h.dinv;
    const T *bp = (const T *)b;
    T *xo = (T *)x;
    T *pg = (T *)h.p;
    const bool dia = use_dia(h);
    const int32_t *doff = dia ? h.dia_off : nullptr;
    int dm = dia ? h.dia_m : 0;
    const T *dval = dia ? (const T *)h.dia_val : nullptr;
    // interleaved walk: forced, or where the matrix (values and columns of
    // every system) exceeds the 256 MB Infinity Cache
    const double mat_bytes = (double)h.nnz * (h.vbytes * h.B + (h.res_narrow ? 2 : 4));
    const int interleave = h.res_walk == 2 ? (mat_bytes > 256.0 * (1 << 20) ? 1 : 0) : h.res_walk;
    GridSync gs{h.res_slot, h.res_slot + (size_t)(2 * h.res_grid * 2 * kMaxC) * h.B,
                h.res_wave + 2 * (waves + 1), (int)h.res_grid, 0, h.spin_limit, interleave};
    const int B = h.B;
    const int64_t n = h.n;
    SysState *st = h.st;
    void *args[] = {(void *)&tiles, (void *)&wrow, (void *)&wtile, (void *)&roff8, (void *)&col,
                    (void *)&col16, (void *)&val, (void *)&vstride, (void *)&dinv, (void *)&bp, (void *)&xo,
                    (void *)&pg, (void *)&gs, (void *)&B, (void *)&n, (void *)&tol,
                    (void *)&maxit, (void *)&st, (void *)&doff, (void *)&dm, (void *)&dval};
    if (h.res_coop) {
        const hipError_t e = hipLaunchCooperativeKernel(
            kernel_for(h), dim3((unsigned)(h.res_grid * h.B)), dim3(kRT), args, 0, s);
        if (e == hipErrorCooperativeLaunchTooLarge || e == hipErrorIllegalState) {
            (void)hipGetLastError();
            return false;
        }
        SLA_HIP(e);
    } else {
        SLA_HIP(hipLaunchKernel(kernel_for(h), dim3((unsigned)(h.res_grid * h.B)), dim3(kRT),
                                args, 0, s));
    }
    return true;
}

}  // namespace

// Whether the single-system solve can run as one cooperative kernel with
// on-chip vectors; builds the per-wavefront plan on first use.
bool resident_ready(Handle &h, hipStream_t s) {
    // automatic choice (mode 1) and forced (mode 2) alike: wherever it
    // applies, this path was the faster one at every size measured on MI355X
    // (per iteration 12.7 against 16.2 us at 4096 rows, 33.9 against 43.7 at
    // 10^6, 50.6 against 71.3 at 2.1M, 120 against 153 on a 2M-point kNN
    // graph): the matrix is the only large stream, and it stays in the
    // Infinity Cache between iterations
    if (h.res_mode == 0) return false;
    if (h.res_state != 0) return h.res_state > 0;
    h.res_state = -1;
    // tiles address entries with 32-bit offsets (rows of at most 128
    // entries and 8192 rows per CU keep nnz far below that on this chip)
    if (h.nlong != 0 || h.nseg > 0 || h.nnz >= ((int64_t)1 << 31)) return false;
    int coop = 0, cus = 0, per_cu = 0;
    SLA_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, h.device));
    SLA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h.device));
    SLA_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel_for(h), kRT, 0));
    if (!coop || per_cu < 1) return false;
    // one workgroup per CU at most, a multiple of the XCD count, shared by
    // the B systems' groups
    int64_t gmax = (int64_t)cus / kXcds * kXcds / h.B / kXcds * kXcds;
    if (gmax < kXcds) return false;
    // at least one row per lane for every wavefront
    int64_t G = (h.n + (int64_t)kRW * 64 - 1) / ((int64_t)kRW * 64);
    G = (G + kXcds - 1) / kXcds * kXcds;
    if (G > gmax) G = gmax;
    if (G > 64 * kPollSlots) G = 64 * kPollSlots;
    const int64_t waves = G * kRW;
    const int64_t rpw = (h.n + waves - 1) / waves;
    if (rpw > 64 * kRJ) return false;
    h.res_grid = G;
    h.res_rows_per_wave = rpw;
    if (h.rp64) build_plan<int64_t>(h, G, rpw, s);
    else build_plan<int32_t>(h, G, rpw, s);
    if (h.dia_m > 0) {
        // the form by diagonals must fit one workgroup per CU as well
        int dia_cu = 0;
        SLA_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &dia_cu,
            h.vt == SLA_F64 ? dia_kernel<double>(h.dia_m) : dia_kernel<float>(h.dia_m),
            kRT, 0));
        h.res_dia_fits = dia_cu >= 1;
    }
    h.res_state = 1;
    return true;
}

// Whole solve from x0 = 0 of every system: b and x are [B][n] (the caller's
// layout), the state st[0..B). The stamps restart at zero for every solve
// (sequence numbers start at 1).
bool resident_solve(Handle &h, const void *b, void *x, double tol, int32_t maxit, hipStream_t s) {
    SLA_HIP(hipMemsetAsync(h.res_slot, 0,
                           sizeof(uint64_t) * (size_t)(2 * h.res_grid * 2 * kMaxC + h.res_grid) * h.B, s));
    hipEvent_t a = nullptr, e = nullptr;
    if (h.profile) {
        SLA_HIP(hipEventCreate(&a));
        SLA_HIP(hipEventCreate(&e));
        SLA_HIP(hipEventRecord(a, s));
    }
    const bool launched = h.vt == SLA_F64 ? launch<double>(h, b, x, tol, maxit, s)
                                          : launch<float>(h, b, x, tol, maxit, s);
    if (h.profile) {
        if (launched) {
            SLA_HIP(hipEventRecord(e, s));
            h.pending.push_back({SLA_KERNEL_CG_RESIDENT, a, e});
        } else {
            (void)hipEventDestroy(a);
            (void)hipEventDestroy(e);
        }
    }
    return launched;
}

}  // namespace sla

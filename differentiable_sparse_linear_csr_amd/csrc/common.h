// Internal declarations of the MI355X sparse solve library (gfx950 / CDNA4).
//
// Device layout
//  - CSR: row_ptr (int32 or int64, [n+1]), col (int32, [nnz]), values
//    entry-major [nnz][B] so that the B value sets of one entry share a cache
//    line (B = 1: plain [nnz]).
//  - Solve vectors x, r, p, q and the Jacobi reciprocal dinv are row-major
//    [n][B] (interleaved): the B systems of one row are contiguous, so the
//    column gather of a batched SpMV reads one line for all systems.
//  - Device scalars per system (SysState) and a control block (Ctl) hold
//    everything the iteration needs; the host only polls a mapped copy of the
//    number of running systems.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "sla.h"

namespace sla {

constexpr int kBlock = 256;                        // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kTileUnits = 256;                    // rows + entries per SpMV tile (one wavefront)
constexpr int kLongRow = 128;                      // longer rows get a workgroup each
constexpr int kTileCap = kTileUnits + kLongRow;    // max entries of a short tile
constexpr int kMaxGrid = 2048;                     // grid cap of the persistent / grid-stride kernels
constexpr int kXcds = 8;                           // workgroups go round-robin over 8 XCDs
constexpr int kMaxBatch = 256;
constexpr int kDiaMax = 8;   // diagonals of a matrix the single-kernel solve holds by diagonals
constexpr int kDiaGridMax = 8192;   // grid cap of the per-step SpMV by diagonals (spart entries)
// diagonal values by blocks of kDiaBlock rows: block c holds its rows' m
// diagonals one after the other, so a lane's loads stay 512 contiguous
// bytes per wavefront and the whole matrix is one stream
constexpr int kDiaBlock = 1024;
__host__ __device__ inline int64_t dia_slot(int d, int64_t i, int m) {
    return (i / kDiaBlock) * ((int64_t)m * kDiaBlock) + (int64_t)d * kDiaBlock + (i % kDiaBlock);
}
inline int64_t dia_slots(int64_t n, int m) { return (n + kDiaBlock - 1) / kDiaBlock * m * kDiaBlock; }
// col and values carry this many spare entries past nnz: the SpMV reads
// entries in 16-byte groups from a 4-aligned base and may touch (never use)
// up to 3 entries beyond a tile's end.
constexpr int kEntryPad = 4;

// per-system status codes on the device: running, or an sla_outcome
constexpr int32_t kRunning = -1;

struct SysState {
    double bb;      // ||b||^2
    double rho;     // r.z of the current residual
    double alpha;   // step of the current iteration
    double beta;    // direction update factor
    double rr;      // ||r||^2 of the last updated residual
    double alpha2;  // folded single-system solve: the step before alpha (0 when none)
    int32_t iter;   // completed iterations
    int32_t status; // kRunning or sla_outcome
};

// A run of short rows [rs, re) whose entries are [k0, k1), at most kTileCap.
// A run of short rows [rs, re) with entries [k0, k1). The single-system SpMV
// reads its indices in 16-bit form: row offsets relative to k0 at
// roff16[rpos ...], and, when every tile's columns span less than 2^16
// (narrow), columns as col16[k] = col[k] - cbase.
struct TileDesc {
    int32_t rs, re;
    int64_t k0, k1;
    int64_t rpos;
    int32_t cbase;
    int32_t narrow;
};

// A tile of the single-kernel solve in 16 bytes, so that the descriptors of
// a CU's wavefronts stay in the scalar cache from one iteration to the next:
// first entry (the solve needs nnz < 2^31), smallest column, position of its
// byte row offsets, and rows | entries << 8 | q slot of its first row << 16.
struct ResTile {
    int32_t k0;
    int32_t cbase;
    int32_t rpos;
    uint32_t packed;
};

struct Ctl {
    double tol;
    int32_t maxit;
    int32_t n_running;
    uint32_t epoch;   // solve counter: with the iteration count it names a broadcast
    int32_t error;    // set by a kernel whose bounded wait timed out (sticky for the solve)
    uint32_t spin_limit;  // polls a bounded grid-wide wait makes before it gives up
    int32_t fold_iter;    // folded batched solve: updates completed (picks the direction buffer)
};

// polls of a bounded grid-wide wait before it gives up (about a second)
constexpr uint32_t kDefaultSpinLimit = 1u << 22;

// how the last solve on a handle ran (sla_csr_get_last_path)
constexpr int32_t kPathNone = 0, kPathSingleKernel = 1, kPathPerStep = 2;
constexpr uint32_t kFallbackCoopRefused = 1u, kFallbackWaitTimedOut = 2u;

// Step scalars broadcast by the last workgroup of the fused update +
// direction kernel to the others: gen = epoch << 32 | iteration number.
struct Bcast {
    uint64_t gen;
    double beta;
    int32_t running;
    int32_t pad;
};

// The direction update folded into the SpMV of a single system (per-step
// solve): p_new = z + beta p_old is formed where the SpMV reads it, at every
// gathered column and at the tile's own rows, and x += alpha p_old (the step
// of the update before) is applied to the own rows. p_old = p[iter & 1],
// p_new = p[(iter + 1) & 1], so that a captured block of iterations reads
// the buffers from the iteration count, not from its arguments.
struct FoldArgs {
    const void *z;        // z = dinv r of the last update
    void *p[2];           // the two direction buffers
    void *x;              // the iterate
    const SysState *st;   // beta, alpha (0: no pending step) and iter
};

// Arrival counters of the grid reductions: per kernel kind, kGroups group
// counters and one top counter, each on its own 256-byte line so that
// arrivals at different counters do not serialize.
constexpr int kGroups = 32;
constexpr int kCounterStride = 64;                       // uint32 per line
constexpr int kCountersPerKind = (kGroups + 1) * kCounterStride;
enum CounterSlot { kCntSpmv = 0, kCntUpdate = 1, kCntInit = 2, kCntKinds = 3 };

struct Error {
    sla_status st;
    std::string msg;
};

[[noreturn]] void fail(sla_status st, const std::string &msg);

#define SLA_HIP(expr)                                                                     \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess) {                                                           \
            if (e_ == hipErrorOutOfMemory)                                                \
                ::sla::fail(SLA_ERR_OOM, std::string(#expr) + ": out of device memory");  \
            ::sla::fail(SLA_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));  \
        }                                                                                 \
    } while (0)

// ------------------------------------------------------------------ handle

struct ProfileRec {
    int kind;
    hipEvent_t a, b;
};

struct Handle {
    int64_t n = 0, nnz = 0, nnz_in = 0;
    int32_t B = 1;
    sla_dtype vt = SLA_F64;
    int vbytes = 8;
    bool rp64 = false;       // row_ptr element type
    uint32_t flags = 0;

    void *row_ptr = nullptr;
    int32_t *col = nullptr;
    void *vals = nullptr;    // [nnz][B]
    // a single system held by diagonals as well (its entries on 5 or 7
    // distinct offsets j - i, at most a quarter more slots than entries):
    // dia_val[d][row] = the entry (row, row + dia_off[d]), 0 where absent;
    // kept in step with vals (load_values, child_values)
    int32_t dia_m = 0;              // diagonals (0: not held by diagonals)
    int32_t *dia_off = nullptr;     // [m] offsets, ascending (column order)
    int32_t *dia_map = nullptr;     // [nnz] CSR entry -> d * n + row
    void *dia_val = nullptr;        // [m][n]
    bool spmv_dia = true;           // SLA_OPT_SPMV_DIA: the per-step SpMV by diagonals
    int64_t *slot = nullptr; // input entry -> CSR position (null: identity)
    int64_t *perm = nullptr; // sorted position -> input entry (null: identity)
    int64_t *run = nullptr;  // [nnz+1] first sorted position of each CSR entry
    TileDesc *tiles = nullptr;   // short-row tiles, in row order
    int64_t ntiles = 0;
    uint16_t *col16 = nullptr;   // [nnz + pad] tile-relative columns of narrow tiles
    uint16_t *roff16 = nullptr;  // per tile: row offsets relative to the tile's k0
    bool all_narrow = false;     // every tile narrow: the SpMV reads col16 only
    bool ring_tiles = false;     // every tile narrow, <= 256 entry slots and <= 63 rows
    bool spmv_ring = true;       // SpMV on ring_tiles handles: the ring form
    bool fold_direction = true;  // per-step single-system solve: direction folded into the SpMV
    bool fold_active = false;    // the solve being run folds it (set per attempt)
    void *fold_z = nullptr;      // z = dinv r (folded solves)
    void *fold_p2 = nullptr;     // second direction buffer (folded solves)
    // band-aligned tiles (see choose_band): band N rows, L tiles per N rows,
    // P panels of L wavefronts per XCD; 0 when the tiles are the usual runs
    int64_t band_n = 0, band_l = 0;
    int32_t band_p = 0;
    int32_t *long_rows = nullptr; // rows longer than kLongRow, in row order
    int64_t nlong = 0;
    double *long_dot = nullptr;   // [nlong] p_i q_i of the long rows (fused SpMV)
    void *dinv = nullptr;    // [n][B]
    bool diag_ok = false;     // every diagonal present, positive, finite (PCG)
    bool diag_nonzero = false; // every diagonal present, non-zero, finite (BiCGStab)

    // solve workspace
    void *x = nullptr, *r = nullptr, *p = nullptr, *q = nullptr; // [n][B]
    double *part = nullptr;
    int64_t part_len = 0;
    double *gpart = nullptr;       // [kGroups][C] group sums of the grid reductions
    double *gpart_spmv = nullptr;  // [kGroups][B] group sums a batched SpMV leaves for the update
    double *spart = nullptr;      // [spmv grid] p.q partials of the single-system SpMV
    uint32_t *sync = nullptr;     // [kCntKinds][kCountersPerKind] arrival counters
    SysState *st = nullptr;
    Ctl *ctl = nullptr;
    Bcast *bcast = nullptr;
    uint32_t epoch = 0;            // solves started on this handle
    uint32_t spin_limit = kDefaultSpinLimit;  // bounded grid-wide waits (SLA_OPT_SPIN_LIMIT)
    int32_t last_path = kPathNone; // how the last solve ran, and why not the preferred way
    uint32_t last_fallback = 0;
    int64_t upd_dir_resident = 0;  // resident workgroups of the fused update + direction
    int64_t upd_dir_bv_resident = 0;  // the same for batches
    int64_t bvec_fold_resident = 0;   // resident workgroups of the folded batched SpMV
    double *bcast_bv = nullptr;    // [2][kMaxBatch] beta and running flag per system
    bool fuse_update = true;       // single system: update and direction in one kernel
    int32_t *h_running = nullptr; // pinned, mapped
    int32_t *d_running = nullptr; // device alias of h_running
    SysState *h_state = nullptr;  // pinned
    Ctl *h_ctl = nullptr;         // pinned staging for the control block

    // resident workgroups of the persistent SpMV on this device (CUs x occupancy,
    // a multiple of the XCD count): larger grids would run in two rounds
    int64_t spmv_resident = kMaxGrid;
    int64_t ring_resident = kMaxGrid;
    // the same for the batched 16-byte-lane kernels: SpMV (plain, fused),
    // update, direction
    int64_t bvec_resident[2] = {kMaxGrid, kMaxGrid};
    int64_t bv_update_resident = kMaxGrid, bv_direction_resident = kMaxGrid;

    // single-system solve as one cooperative kernel with on-chip vectors
    // (built at the first solve that can use it; -1: not applicable)
    int res_state = 0;
    int res_mode = 1;              // 0 never, 1 automatic, 2 whenever applicable
    int64_t res_grid = 0;          // workgroups (one per CU at most)
    int64_t res_rows_per_wave = 0;
    ResTile *res_tiles = nullptr;  // tiles that never cross a wavefront's row range
    int32_t *res_wave = nullptr;   // [2][waves+1]: first row, first tile of each wavefront;
                                   // then each workgroup's barrier dependencies
    uint64_t *res_slot = nullptr;  // [B][2][res_grid][4] stamped all-reduce partials, then
                                   // [B][res_grid] barrier stamps
    void *res_vals = nullptr;      // [B][padded nnz] batch-major values (B > 1)
    uint8_t *res_roff8 = nullptr;  // row offsets of the tiles as bytes (TileDesc.rpos)
    uint16_t *res_col16 = nullptr; // columns minus their tile's smallest (res_narrow)
    bool res_narrow = false;       // every tile's columns span less than 2^16
    bool res_coop = true;          // cooperative launch (else an ordinary one)
    int res_walk = 2;              // SpMV phase: 0 contiguous runs, 1 interleaved, 2 by size
    bool res_dia_on = true;        // SLA_OPT_RESIDENT_DIA
    bool res_dia_fits = true;      // the single-kernel form by diagonals fits a CU

    // symmetric reordering for locality (reverse Cuthill-McKee): the solver
    // runs on `inner`, a handle of P A P^T; this handle keeps the caller's CSR
    // and maps vectors, values and gradients between the two orders
    Handle *inner = nullptr;
    int32_t *new2old = nullptr;   // [n]: row of A that is row i of P A P^T
    int64_t *map_in = nullptr;    // [nnz]: inner CSR position -> this CSR position
    int64_t *map_out = nullptr;   // [nnz]: this CSR position -> inner CSR position
    void *rtmp[2] = {nullptr, nullptr};  // [B][n] vectors in the inner order
    void *rtmp_grad = nullptr;    // [B][nnz] value gradient in the inner order
    int64_t wide_tiles = 0;       // tiles whose columns span 2^16 or more
    // segmented handle: a block-diagonal matrix of nseg independent systems
    // (distinct patterns) solved together, each with its own scalars and test
    int32_t nseg = 0;
    int64_t *seg_rows = nullptr;  // [nseg+1] first row of each segment
    int32_t *blk_seg = nullptr;   // [seg_grid] segment of each workgroup of the vector kernels
    int64_t *seg_blk0 = nullptr;  // [nseg+1] first workgroup of each segment
    int64_t seg_grid = 0;
    uint32_t *seg_sync = nullptr; // [nseg] arrival counters (one line each)
    double *seg_part = nullptr;   // [2 * seg_grid] workgroup partials
    // SpMV tiles of a segmented handle never straddle two members: the tiles
    // and long rows of member q are [seg_tile0[q], seg_tile0[q+1]) and
    // [seg_long0[q], seg_long0[q+1]); the solve's SpMV skips tiles whose
    // member has finished (tile_live 0) and leaves each tile's p.q in tile_dot
    int64_t *seg_tile0 = nullptr, *seg_long0 = nullptr;
    uint8_t *tile_live = nullptr;
    double *tile_dot = nullptr;
    // A^T for the backward of y = A x (built at the first backward)
    Handle *tr = nullptr;
    int64_t *tr_map = nullptr;    // [nnz]: A^T CSR position -> this CSR position
    bool tr_stale = false;        // values changed since A^T's were gathered

    // BiCGStab workspace (allocated at the first BiCGStab solve): r^, p^, s^,
    // t; partials and counters of its reductions; its scalars; its graph
    void *bi_vec[4] = {nullptr, nullptr, nullptr, nullptr};
    double *bi_part = nullptr, *bi_gpart = nullptr, *bi_spart2 = nullptr;
    uint32_t *bi_sync = nullptr;
    void *bi_state = nullptr;
    hipGraphExec_t bi_graph = nullptr;
    int bi_graph_k = 0;
    void *lam_tmp = nullptr;      // [n] adjoint solution when the caller wants no grad_b

    // iteration driver
    int check_k = 16;
    bool use_graph = true;
    bool profile = false;
    hipStream_t cap_stream = nullptr;
    hipGraphExec_t graph = nullptr;
    int graph_k = 0;
    hipEvent_t ev[2] = {nullptr, nullptr};
    int device = 0;

    std::vector<ProfileRec> pending;
    int64_t prof_launches[SLA_KERNEL_COUNT] = {};
    double prof_ms[SLA_KERNEL_COUNT] = {};

    int64_t bytes = 0;
    std::vector<void *> allocs;
};

// allocation helpers (tracked per handle)
void *dalloc(Handle &h, size_t bytes);
void dfree_all(Handle &h);

// ------------------------------------------------------------------ assembly
void build_from_coo(Handle &h, sla_itype rit, const void *rows, sla_itype cit, const void *cols,
                    const void *values, hipStream_t s);
void build_from_csr(Handle &h, sla_itype rit, const void *row_ptr, sla_itype cit, const void *cols,
                    const void *values, hipStream_t s);
void load_values(Handle &h, const void *values, hipStream_t s);
// seg_rows (host, [nseg+1]) splits tiles at member boundaries (nseg = 0: none)
void build_tiles(Handle &h, hipStream_t s, const int64_t *seg_rows = nullptr, int32_t nseg = 0);
void compute_dinv(Handle &h, hipStream_t s);       // sets h.diag_ok (synchronizes)
bool check_symmetric(Handle &h, hipStream_t s);
// per-workgroup partials the PCG SpMV leaves in spart (the tile grid, or
// the grid of the SpMV by diagonals)
int64_t spmv_blocks(const Handle &h);
void build_dia(Handle &h, hipStream_t s);    // synchronizes
void dia_scatter(Handle &h, hipStream_t s);  // vals -> dia_val    // synchronizes
void gather_to_input(Handle &h, const void *in, void *out, hipStream_t s);
void values_to_batch_major(Handle &h, void *out, hipStream_t s);

// ------------------------------------------------------------------ utilities
void exclusive_scan_i64(const int64_t *in, int64_t *out, int64_t m, hipStream_t s);
void radix_sort_pairs(uint64_t *keys, int64_t *vals, int64_t m, int key_bits, hipStream_t s);
void transpose(const void *in, void *out, int64_t rows, int64_t cols, int vbytes, hipStream_t s);
void iota_i64(int64_t *out, int64_t m, hipStream_t s);

// ------------------------------------------------------------------ SpMV / solve
void spmv(Handle &h, const void *x, void *y, hipStream_t s);
void spmv_from_internal(Handle &h, const void *x_int, void *y, hipStream_t s);
void init_launch_limits(Handle &h);
void init_vector_limits(Handle &h);
void alloc_workspace(Handle &h, hipStream_t s);
void destroy_handle(Handle *h);
// reordering (reorder.hip)
bool want_reorder(const Handle &h);
void build_reordered(Handle &h, hipStream_t s);
void reordered_set_values(Handle &h, hipStream_t s);
void reordered_spmv(Handle &h, const void *x, void *y, hipStream_t s);
void reordered_pcg(Handle &h, const void *b, void *x, double tol, int32_t maxit, sla_info *info,
                   hipStream_t s);
void reordered_adjoint(Handle &h, const void *x, const void *g, void *grad_b, void *grad_vals,
                       double tol, int32_t maxit, sla_info *info, hipStream_t s);
void reordered_bicgstab(Handle &h, const void *b, void *x, double tol, int32_t maxit,
                        sla_info *info, hipStream_t s);
void reordered_spmv_backward(Handle &h, const void *x, const void *g, void *grad_x,
                             void *grad_vals_out, hipStream_t s);
Handle &reordered_bicgstab_adjoint(Handle &h, const void *x, const void *g, void *grad_b,
                                   void *grad_vals_out, double tol, int32_t maxit,
                                   sla_info *info, hipStream_t s);
// BiCGStab on one system (bicgstab.hip); b, x device vectors of n elements
void bicgstab(Handle &h, const void *b, void *x, double tol, int32_t maxit, sla_info *info,
              hipStream_t s, bool keep_internal);
// BiCGStab for any single-system handle (reordered or not), caller's order
void any_bicgstab(Handle &h, const void *b, void *x, double tol, int32_t maxit, sla_info *info,
                  hipStream_t s);
Handle *make_child(Handle &h, const std::vector<int64_t> &rp, const std::vector<int32_t> &col,
                   const int64_t *map, uint32_t flags, hipStream_t s);
void child_values(Handle &h, Handle &child, const int64_t *map, hipStream_t s);
void any_spmv(Handle &h, const void *x, void *y, hipStream_t s);
Handle *transpose_for_backward(Handle &h, hipStream_t s);
// segmented handles (seg.hip)
void build_segments(Handle &h, const int64_t *seg_rows, int32_t nseg, hipStream_t s);
void launch_spmv_plain(Handle &h, const void *x, void *y, hipStream_t s);
inline int32_t num_systems(const Handle &h) { return h.nseg > 0 ? h.nseg : h.B; }
int64_t resident_workgroups(const void *kernel, int device, size_t dyn_lds = 0);
int64_t tile_spmv_waves_per_xcd(const Handle &h, bool ring);
void pcg(Handle &h, const void *b_user, void *x_user, double tol, int32_t maxit, sla_info *info,
         hipStream_t s, bool keep_internal_solution);
// grad[b][k] = sign * a[row k][b] * x[b][col k]: a in the internal layout
// [n][B], x in the caller's [B][n], grad [B][nnz] in CSR order
void grad_vals(Handle &h, const void *a_internal, const void *x_user, void *grad, hipStream_t s,
               double sign = -1.0);
bool resident_ready(Handle &h, hipStream_t s);   // builds the plan on first use
// false (nothing launched) when the cooperative launch is refused
bool resident_solve(Handle &h, const void *b, void *x, double tol, int32_t maxit, hipStream_t s);
void flush_profile(Handle &h);

// hipEvents around kernel launches of a call (profiling on)
struct Launcher {
    Handle &h;
    hipStream_t s;
    bool prof;
    void begin(int kind, hipEvent_t *a) {
        (void)kind;
        if (prof) {
            SLA_HIP(hipEventCreate(a));
            SLA_HIP(hipEventRecord(*a, s));
        }
    }
    void end(int kind, hipEvent_t a) {
        if (prof) {
            hipEvent_t b;
            SLA_HIP(hipEventCreate(&b));
            SLA_HIP(hipEventRecord(b, s));
            h.pending.push_back({kind, a, b});
        }
    }
};

void seg_init(Handle &h, const void *b, hipStream_t s, Launcher *lp);
void seg_iter_kernels(Handle &h, hipStream_t s, Launcher *lp);

// ------------------------------------------------------------------ device helpers

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Deterministic sum over the 256 threads of a block (fixed shuffle tree inside
// each wave, then the 4 wave sums in order). Result valid in every thread.
__device__ __forceinline__ double block_sum(double v, double *lds4) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds4[w] = v;
    __syncthreads();
    double s = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
    __syncthreads();
    return s;
}

// Rows of a batched layout handled by one block pass: lanes t < J*B, system
// b = t % B, row offset t / B. J = kBlock / B.
struct Lanes {
    int B, J, b, jr;
    bool on;
    __device__ Lanes(int B_) : B(B_) {
        J = kBlock / B;
        const int t = threadIdx.x;
        on = t < J * B;
        b = on ? t % B : 0;
        jr = on ? t / B : 0;
    }
};

// Per-system block reduction of one value per lane (lanes with the same b are
// summed in a fixed order). Writes out[b] for b < B from threads t < B.
// tmp must hold kBlock doubles. Ends with a barrier.
__device__ __forceinline__ void block_sum_per_system(double v, const Lanes &L, double *tmp,
                                                      double *out) {
    const int t = threadIdx.x;
    if ((L.B & (L.B - 1)) == 0 && L.B <= 64) {
        // power-of-two B: xor offsets >= B keep the system index
        for (int off = 32; off >= L.B; off >>= 1) v += __shfl_xor(v, off, 64);
        const int w = t >> 6;
        if ((t & 63) < L.B) tmp[w * 64 + (t & 63)] = v;
        __syncthreads();
        if (t < L.B) {
            const int nw = (L.J * L.B + 63) / 64;
            double s = 0.0;
            for (int k = 0; k < nw; ++k) s += tmp[k * 64 + t];
            out[t] = s;
        }
    } else {
        tmp[t] = L.on ? v : 0.0;
        __syncthreads();
        if (t < L.B) {
            double s = 0.0;
            for (int j = 0; j < L.J; ++j) s += tmp[j * L.B + t];
            out[t] = s;
        }
    }
    __syncthreads();
}

// Cross-block partials go through device-scope atomic stores and loads
// (written through to the device coherence point), so no L2 writeback is
// needed: a block stores its partials with store_partial(), every thread
// waits for its own stores to complete, then one thread bumps the arrival
// counter. The block that arrives last reads all partials back with
// device-scope loads.
__device__ __forceinline__ void store_partial(double *p, double v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ double load_partial(const double *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Column sums of rows [j0, j1) of a [rows][C] partial table, in row order,
// read with device-scope loads (4 in flight per lane). Result in out[0..C).
__device__ __forceinline__ void sum_rows(const double *part, int64_t j0, int64_t j1, int C,
                                         double *tmp, double *out) {
    const int t = threadIdx.x;
    const int Cc = C < kBlock ? C : kBlock;
    const int J = kBlock / Cc;
    for (int cb = 0; cb < C; cb += Cc) {
        const int c = cb + t % Cc;
        const int r0 = t / Cc;
        double s = 0.0;
        if (c < C && r0 < J) {
            for (int64_t j = j0 + r0; j < j1; j += 4 * (int64_t)J) {
                double v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t jj = j + (int64_t)u * J;
                    v[u] = jj < j1 ? load_partial(part + jj * C + c) : 0.0;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) s += v[u];
            }
        }
        tmp[t] = s;
        __syncthreads();
        if (t < Cc && cb + t < C) {
            double a = 0.0;
            for (int k = 0; k < J; ++k) a += tmp[k * Cc + t];
            out[cb + t] = a;
        }
        __syncthreads();
    }
}

// Arrive at a device-scope counter after this block's partial stores have
// completed; true in the block whose arrival is number `expected`.
__device__ __forceinline__ bool arrive(uint32_t *counter, uint32_t expected) {
    __shared__ int s_last;
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == expected - 1);
        if (s_last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return s_last;
}

// Grid-wide combination of per-block partials part[blk][C] (C <= 2*kMaxBatch).
// Every block calls it after its threads stored the block's C values with
// store_partial(). Blocks are split into kGroups contiguous groups; the last
// block of a group sums the group's rows (block order) into gpart[g][C]; the
// last group to finish sums the group rows (group order) into tot[0..C)
// (shared) and returns true. The summation tree depends only on nblk, so the
// result is deterministic. Counters are reset for the next launch.
__device__ __forceinline__ bool last_block_sums(double *part, double *gpart, uint32_t *counters,
                                                int64_t nblk, int C, double *tmp, double *tot) {
    const int64_t gb = (nblk + kGroups - 1) / kGroups;   // blocks per group
    const int64_t ngroups = (nblk + gb - 1) / gb;
    const int64_t g = blockIdx.x / gb;
    const int64_t j0 = g * gb;
    const int64_t j1 = (j0 + gb < nblk) ? j0 + gb : nblk;
    if (!arrive(counters + g * kCounterStride, (uint32_t)(j1 - j0))) return false;
    sum_rows(part, j0, j1, C, tmp, tot);
    for (int c = threadIdx.x; c < C; c += kBlock) store_partial(gpart + g * C + c, tot[c]);
    if (!arrive(counters + kGroups * kCounterStride, (uint32_t)ngroups)) return false;
    sum_rows(gpart, 0, ngroups, C, tmp, tot);
    return true;
}

// The group level of last_block_sums alone: the last block of each group
// sums the group's rows (block order) into gpart[g][C]. The next kernel
// finishes the sum with group_total(), in every block, with the tree
// last_block_sums uses, so that the grid-wide serial tail (a second arrival
// and the final sum) leaves the producing kernel.
__device__ __forceinline__ void last_group_sums(double *part, double *gpart, uint32_t *counters,
                                                int64_t nblk, int C, double *tmp, double *tot) {
    const int64_t gb = (nblk + kGroups - 1) / kGroups;
    const int64_t g = blockIdx.x / gb;
    const int64_t j0 = g * gb;
    const int64_t j1 = (j0 + gb < nblk) ? j0 + gb : nblk;
    if (!arrive(counters + g * kCounterStride, (uint32_t)(j1 - j0))) return;
    sum_rows(part, j0, j1, C, tmp, tot);
    for (int c = threadIdx.x; c < C; c += kBlock) store_partial(gpart + g * C + c, tot[c]);
}
// tot[0..C) = the sum of the group rows that last_group_sums left for a
// launch of nblk blocks (group order)
__device__ __forceinline__ void group_total(const double *gpart, int64_t nblk, int C, double *tmp,
                                            double *tot) {
    const int64_t gb = (nblk + kGroups - 1) / kGroups;
    const int64_t ngroups = (nblk + gb - 1) / gb;
    sum_rows(gpart, 0, ngroups, C, tmp, tot);
}

// Last-block epilogue of a fused SpMV: sigma = p.q per system in tot[0..B);
// alpha = rho / sigma, or a breakdown when sigma is not > 0 or not finite.
__device__ __forceinline__ void finish_alpha(const double *tot, int B, Ctl *ctl, SysState *st,
                                             int32_t *h_running);

// 16-byte vector access: W = 16 / sizeof(T) consecutive elements per lane
template <typename T>
struct VecW {
    static constexpr int W = 16 / sizeof(T);
};
template <typename T>
__device__ __forceinline__ void vload(const T *p, T (&o)[VecW<T>::W]) {
    const int4 a = *reinterpret_cast<const int4 *>(p);
    __builtin_memcpy(o, &a, 16);
}
template <typename T>
__device__ __forceinline__ void vstore(T *p, const T (&o)[VecW<T>::W]) {
    int4 a;
    __builtin_memcpy(&a, o, 16);
    *reinterpret_cast<int4 *>(p) = a;
}
// The same with the non-temporal hint, for vectors far larger than the
// caches (they are not re-read before they are evicted, and keeping them out
// of the Infinity Cache leaves it to the matrix stream)
typedef int nt_v4i __attribute__((ext_vector_type(4)));
template <bool NT, typename T>
__device__ __forceinline__ void vload_h(const T *p, T (&o)[VecW<T>::W]) {
    if constexpr (NT) {
        const nt_v4i a = __builtin_nontemporal_load(reinterpret_cast<const nt_v4i *>(p));
        __builtin_memcpy(o, &a, 16);
    } else {
        vload(p, o);
    }
}
template <bool NT, typename T>
__device__ __forceinline__ void vstore_h(T *p, const T (&o)[VecW<T>::W]) {
    if constexpr (NT) {
        nt_v4i a;
        __builtin_memcpy(&a, o, 16);
        __builtin_nontemporal_store(a, reinterpret_cast<nt_v4i *>(p));
    } else {
        vstore(p, o);
    }
}
// vectors of at least this many bytes take the non-temporal accesses
constexpr int64_t kNtVectorBytes = (int64_t)128 << 20;

// Four consecutive elements through 16-byte loads (p 16-byte aligned)
__device__ __forceinline__ void load4(const double *p, double (&o)[4]) {
    const double2 a = *reinterpret_cast<const double2 *>(p);
    const double2 b = *reinterpret_cast<const double2 *>(p + 2);
    o[0] = a.x; o[1] = a.y; o[2] = b.x; o[3] = b.y;
}
__device__ __forceinline__ void load4(const float *p, float (&o)[4]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void load4(const int32_t *p, int32_t (&o)[4]) {
    const int4 a = *reinterpret_cast<const int4 *>(p);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}

// Per-system block sums when lane t carries the W systems (t % Q) * W + w,
// w < W (Q = B / W a power of two dividing kBlock): a fixed shuffle tree
// inside each wavefront, then the wavefront (or lane) rows in order. Writes
// out[s] for s < B. tmp must hold 4 * kMaxBatch doubles. Ends with a barrier.
template <int W>
__device__ __forceinline__ void block_sum_systems(const double (&v)[W], int Q, double *tmp,
                                                  double *out) {
    const int t = threadIdx.x;
    const int B = Q * W;
    double a[W];
#pragma unroll
    for (int w = 0; w < W; ++w) a[w] = v[w];
    int R;
    if (Q < 64) {
        for (int off = 32; off >= Q; off >>= 1) {
#pragma unroll
            for (int w = 0; w < W; ++w) a[w] += __shfl_xor(a[w], off, 64);
        }
        const int l = t & 63;
        if (l < Q) {
#pragma unroll
            for (int w = 0; w < W; ++w) tmp[((t >> 6) * Q + l) * W + w] = a[w];
        }
        R = kWaves;
    } else {
#pragma unroll
        for (int w = 0; w < W; ++w) tmp[t * W + w] = a[w];
        R = kBlock / Q;
    }
    __syncthreads();
    for (int s = t; s < B; s += kBlock) {
        double sum = 0.0;
        for (int j = 0; j < R; ++j) sum += tmp[j * B + s];
        out[s] = sum;
    }
    __syncthreads();
}

// Where a kernel's grid reduction keeps its partials and counters.
struct Red {
    double *part;
    double *gpart;
    uint32_t *sync;  // this kernel kind's kCountersPerKind counters
};
// the general per-step kernels on caller-given buffers (allocation-free solve)
void launch_init_raw(int64_t n, const double *b, double *x, double *r, double *p,
                     const double *dinv, Red red, Ctl *ctl, SysState *st, int32_t *running,
                     hipStream_t s);
void launch_update_raw(int64_t n, double *x, double *r, const double *p, const double *q,
                       const double *dinv, Red red, Ctl *ctl, SysState *st, int32_t *running,
                       hipStream_t s);
void launch_direction_raw(int64_t n, const double *r, double *p, const double *dinv,
                          const Ctl *ctl, const SysState *st, hipStream_t s);
int64_t raw_vec_grid(int64_t n);
bool fold_possible(const Handle &h);
int64_t bvec_fold_grid(const Handle &h, int64_t *rows_block_out);
int64_t bvec_spmv_blocks(const Handle &h);
void launch_spmv_fold(Handle &h, hipStream_t s);
void launch_spmv_csr_dot_raw(int64_t n, const int32_t *row_ptr, const int32_t *col,
                             const double *val, const double *p, double *q, Red red, Ctl *ctl,
                             SysState *st, int32_t *running, hipStream_t s);
// the allocation-free solve (noalloc.hip)
void pcg_noalloc(int64_t n, int64_t nnz, const int32_t *row_ptr, const int32_t *col,
                 const double *val, const double *b, double *x, double tol, int32_t maxit,
                 uint32_t spin_limit, sla_info *info, hipStream_t s);

__device__ __forceinline__ void publish_running(Ctl *ctl, int32_t *h_running, int32_t v) {
    ctl->n_running = v;
    __hip_atomic_store(h_running, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Sum of one integer per thread over the block (integer LDS atomics: exact
// in any order). Every thread of the block calls it; ends with a barrier.
__device__ __forceinline__ int block_count(int v) {
    __shared__ int s_cnt;
    if (threadIdx.x == 0) s_cnt = 0;
    __syncthreads();
    if (v) atomicAdd(&s_cnt, v);
    __syncthreads();
    const int r = s_cnt;
    __syncthreads();
    return r;
}

// Last block of a fused SpMV (every thread of it calls this), one thread per
// system: alpha = rho / sigma, or a breakdown; then the number still running.
// (A loop over the systems in one thread makes a dependent round trip to
// memory per system: 16 us for 32 systems.)
__device__ __forceinline__ void finish_alpha(const double *tot, int B, Ctl *ctl, SysState *st,
                                             int32_t *h_running) {
    int running = 0;
    for (int b = threadIdx.x; b < B; b += kBlock) {
        SysState &s = st[b];
        if (s.status != kRunning) continue;
        const double sigma = tot[b];
        if (!(sigma > 0.0) || !isfinite(sigma)) {
            s.status = SLA_BREAKDOWN;
            s.iter += 1;
            s.alpha = 0.0;   // no step (a folded solve applies alpha to x later)
        } else {
            s.alpha = s.rho / sigma;
            ++running;
        }
    }
    running = block_count(running);
    if (threadIdx.x == 0) publish_running(ctl, h_running, running);
}

template <typename T>
__device__ __forceinline__ T from_double(double v) {
    return static_cast<T>(v);
}

}  // namespace sla

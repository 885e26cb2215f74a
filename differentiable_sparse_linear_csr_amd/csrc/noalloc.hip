// Jacobi-PCG for one fp64 system given as caller CSR arrays, for callers that
// cannot allocate device memory: code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc. No handle and no allocation: the
// workspace (r, p, q and the Jacobi reciprocal, the reductions' partials and
// arrival counters, the control block and the per-system scalars) is one
// file-scope device array, `scratch`, which each GPU holds until the process
// ends. The recurrence and the kernels are those of the per-step solve
// (init, fused SpMV with p.q and alpha, fused update with r.z, r.r, the test
// and beta, direction); the SpMV is the general one-lane-per-row form, since
// the tiled form needs tile tables built (and allocated) per matrix.
#include <mutex>

#include "common.h"

namespace sla {
namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 21;   // SLA_NOALLOC_MAX_ROWS
constexpr size_t align256(size_t b) { return (b + 255) / 256 * 256; }
constexpr size_t kVecBytes = (size_t)kMaxRows * sizeof(double);
// byte offsets inside the array
constexpr size_t kOffR = 0;
constexpr size_t kOffP = kOffR + kVecBytes;
constexpr size_t kOffQ = kOffP + kVecBytes;
constexpr size_t kOffDinv = kOffQ + kVecBytes;
constexpr size_t kOffPart = kOffDinv + kVecBytes;                 // [kMaxGrid][2] doubles
constexpr size_t kOffGpart = kOffPart + align256((size_t)kMaxGrid * 2 * sizeof(double));
constexpr size_t kOffSync = kOffGpart + align256((size_t)kGroups * 2 * sizeof(double));
constexpr size_t kSyncWords = (size_t)kCntKinds * kCountersPerKind;
constexpr size_t kOffState = kOffSync + align256(kSyncWords * sizeof(uint32_t));
constexpr size_t kOffCtl = kOffState + align256(sizeof(SysState));
constexpr size_t kOffFlags = kOffCtl + align256(sizeof(Ctl));     // [0] running, [1] checks
constexpr size_t kScratchBytes = kOffFlags + 256;
static_assert(kScratchBytes <= ((size_t)64 << 20) + ((size_t)58 << 10),
              "the workspace size stated in sla.h");

// The workspace. In host code this name stands for the array but is not its
// device address: host code uses only the address hipGetSymbolAddress gives
// for the current device (scratch_base).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
unsigned char *g_base[kMaxDevices] = {};

// the array's address on the current device, looked up once per device
unsigned char *scratch_base() {
    int dev = 0;
    SLA_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) fail(SLA_ERR_INVALID_ARG, "device index out of range");
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_base[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            fail(SLA_ERR_HIP, std::string("hipGetSymbolAddress of the solve workspace: ") +
                                  hipGetErrorString(e));
        }
        g_base[dev] = (unsigned char *)p;
    }
    return g_base[dev];
}

constexpr int kBadCsr = 1, kBadIndex = 2, kBadDiagonal = 4;

// zero n words (the arrival counters and the flags start at zero)
__global__ __launch_bounds__(kBlock) void k_zero_words(uint32_t *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        p[i] = 0u;
}

__global__ void k_set_ctl(Ctl *ctl, double tol, int32_t maxit, uint32_t spin_limit) {
    Ctl c;
    c.tol = tol;
    c.maxit = maxit;
    c.n_running = 0;
    c.epoch = 0;
    c.error = 0;
    c.spin_limit = spin_limit;
    c.fold_iter = 0;
    *ctl = c;
}

// Validation of the caller's CSR and the Jacobi reciprocal, one lane per row:
// row_ptr runs from 0 to nnz without decreasing, columns lie in [0, n) and
// increase strictly inside a row, the diagonal is present, positive and
// finite. No entry outside [0, nnz) is read: a row whose bounds are not
// inside it is only flagged.
__global__ __launch_bounds__(kBlock) void k_check_dinv(int64_t n, int64_t nnz,
                                                       const int32_t *__restrict__ row_ptr,
                                                       const int32_t *__restrict__ col,
                                                       const double *__restrict__ val,
                                                       double *__restrict__ dinv,
                                                       int32_t *__restrict__ flags) {
    int f = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t lo = row_ptr[i], hi = row_ptr[i + 1];
        if (i == 0 && lo != 0) f |= kBadCsr;
        if (i == n - 1 && hi != nnz) f |= kBadCsr;
        if (lo < 0 || hi < lo || hi > nnz) {
            f |= kBadCsr;
            dinv[i] = 0.0;
            continue;
        }
        double d = 0.0;
        bool found = false;
        int64_t prev = -1;
        for (int64_t k = lo; k < hi; ++k) {
            const int64_t c = col[k];
            if (c < 0 || c >= n) f |= kBadIndex;
            if (c <= prev) f |= kBadCsr;
            prev = c;
            if (c == i) {
                d = val[k];
                found = true;
            }
        }
        const bool ok = found && d > 0.0 && isfinite(d);
        if (!ok) f |= kBadDiagonal;
        dinv[i] = ok ? 1.0 / d : 0.0;
    }
    if (f) atomicOr(flags, f);
}

unsigned grid_of(int64_t work) {
    int64_t g = (work + kBlock - 1) / kBlock;
    if (g > 4 * kMaxGrid) g = 4 * kMaxGrid;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

void pcg_noalloc(int64_t n, int64_t nnz, const int32_t *row_ptr, const int32_t *col,
                 const double *val, const double *b, double *x, double tol, int32_t maxit,
                 uint32_t spin_limit, sla_info *info, hipStream_t s) {
    if (n < 1 || n > kMaxRows)
        fail(SLA_ERR_INVALID_ARG, "the allocation-free solve takes 1 <= n <= 2^21 rows (n = " +
                                      std::to_string(n) + ")");
    if (nnz < 0 || nnz >= ((int64_t)1 << 31)) fail(SLA_ERR_INVALID_ARG, "need 0 <= nnz < 2^31");
    unsigned char *base = scratch_base();
    double *r = (double *)(base + kOffR);
    double *p = (double *)(base + kOffP);
    double *q = (double *)(base + kOffQ);
    double *dinv = (double *)(base + kOffDinv);
    double *part = (double *)(base + kOffPart);
    double *gpart = (double *)(base + kOffGpart);
    uint32_t *sync = (uint32_t *)(base + kOffSync);
    SysState *st = (SysState *)(base + kOffState);
    Ctl *ctl = (Ctl *)(base + kOffCtl);
    int32_t *running = (int32_t *)(base + kOffFlags);
    int32_t *checks = running + 1;

    // what must start at zero: the arrival counters (they return to zero
    // after every complete reduction, but an earlier call may have stopped
    // between two) and the flags
    hipLaunchKernelGGL(k_zero_words, dim3(grid_of((int64_t)kSyncWords)), dim3(kBlock), 0, s, sync,
                       (int64_t)kSyncWords);
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(kBlock), 0, s, (uint32_t *)running, (int64_t)2);
    hipLaunchKernelGGL(k_set_ctl, dim3(1), dim3(1), 0, s, ctl, tol, maxit, spin_limit);
    hipLaunchKernelGGL(k_check_dinv, dim3(grid_of(n)), dim3(kBlock), 0, s, n, nnz, row_ptr, col, val,
                       dinv, checks);
    SLA_HIP(hipGetLastError());
    int32_t flags = 0;
    SLA_HIP(hipMemcpyAsync(&flags, checks, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    if (flags & kBadIndex) fail(SLA_ERR_INDEX_RANGE, "a column index lies outside [0, n)");
    if (flags & kBadCsr)
        fail(SLA_ERR_INVALID_CSR,
             "row_ptr must run from 0 to nnz without decreasing, columns increase in a row");
    if (flags & kBadDiagonal)
        fail(SLA_ERR_BAD_DIAGONAL,
             "Jacobi preconditioning needs every diagonal entry present, positive and finite");

    const Red red_init{part, gpart, sync + kCntInit * kCountersPerKind};
    const Red red_spmv{part, gpart, sync + kCntSpmv * kCountersPerKind};
    const Red red_upd{part, gpart, sync + kCntUpdate * kCountersPerKind};
    launch_init_raw(n, b, x, r, p, dinv, red_init, ctl, st, running, s);
    // blocks of 16 iterations; finished systems make every later kernel a
    // no-op, so the count does not depend on where the host looks
    constexpr int kPoll = 16;
    const int64_t chunks = maxit <= 0 ? 0 : (maxit + kPoll - 1) / kPoll;
    for (int64_t ch = 0; ch < chunks; ++ch) {
        for (int j = 0; j < kPoll; ++j) {
            launch_spmv_csr_dot_raw(n, row_ptr, col, val, p, q, red_spmv, ctl, st, running, s);
            launch_update_raw(n, x, r, p, q, dinv, red_upd, ctl, st, running, s);
            launch_direction_raw(n, r, p, dinv, ctl, st, s);
        }
        int32_t still = 0;
        SLA_HIP(hipMemcpyAsync(&still, running, sizeof(int32_t), hipMemcpyDeviceToHost, s));
        SLA_HIP(hipStreamSynchronize(s));
        if (still == 0) break;
    }
    SysState hs;
    SLA_HIP(hipMemcpyAsync(&hs, st, sizeof(SysState), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    info->iterations = hs.iter;
    info->status = hs.status == kRunning ? SLA_MAXIT : hs.status;
    info->rel_residual = hs.bb == 0.0 ? 0.0 : sqrt(hs.rr / hs.bb);
}

}  // namespace sla

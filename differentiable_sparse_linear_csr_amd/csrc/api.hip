// extern "C" entry points declared in include/sla.h: argument checks, handle
// lifetime, error reporting. Every call runs its work in this library's
// kernels on the caller's stream.
#include <cstring>
#include <new>

#include "common.h"

#include <algorithm>

namespace sla {

namespace {
thread_local std::string g_last_error;

int64_t spmv_grid_count(const Handle &h);
}  // namespace

int64_t spmv_grid(const Handle &h);

[[noreturn]] void fail(sla_status st, const std::string &msg) { throw Error{st, msg}; }

void *dalloc(Handle &h, size_t bytes) {
    void *p = nullptr;
    if (bytes == 0) bytes = 1;
    const hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        fail(SLA_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " +
                              hipGetErrorString(e));
    }
    h.allocs.push_back(p);
    h.bytes += (int64_t)bytes;
    return p;
}

void dfree_all(Handle &h) {
    for (void *p : h.allocs) (void)hipFree(p);
    h.allocs.clear();
    h.bytes = 0;
}

namespace {

int64_t spmv_grid_count(const Handle &h) { return spmv_grid(h); }

template <typename F>
sla_status guard(F &&f) {
    try {
        f();
        g_last_error.clear();
        return SLA_OK;
    } catch (const Error &e) {
        g_last_error = e.msg;
        return e.st;
    } catch (const std::bad_alloc &) {
        g_last_error = "host allocation failed";
        return SLA_ERR_OOM;
    } catch (...) {
        g_last_error = "unexpected internal error";
        return SLA_ERR_HIP;
    }
}

}  // namespace

void destroy_handle(Handle *h) {
    if (!h) return;
    (void)hipSetDevice(h->device);
    if (h->inner) destroy_handle(h->inner);
    if (h->tr) destroy_handle(h->tr);
    if (h->graph) (void)hipGraphExecDestroy(h->graph);
    if (h->bi_graph) (void)hipGraphExecDestroy(h->bi_graph);
    for (auto &rec : h->pending) {
        (void)hipEventDestroy(rec.a);
        (void)hipEventDestroy(rec.b);
    }
    for (hipEvent_t e : h->ev)
        if (e) (void)hipEventDestroy(e);
    if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
    if (h->h_running) (void)hipHostFree(h->h_running);
    if (h->h_state) (void)hipHostFree(h->h_state);
    if (h->h_ctl) (void)hipHostFree(h->h_ctl);
    dfree_all(*h);
    delete h;
}

void alloc_workspace(Handle &h, hipStream_t s) {
    const size_t vec = (size_t)h.n * h.B * h.vbytes;
    h.dinv = dalloc(h, vec);
    h.x = dalloc(h, vec);
    h.r = dalloc(h, vec);
    h.p = dalloc(h, vec);
    h.q = dalloc(h, vec);
    int64_t plen = spmv_grid_count(h) * h.B;
    const int64_t vec_part = (int64_t)kMaxGrid * 2 * h.B;
    if (vec_part > plen) plen = vec_part;
    h.part_len = plen;
    h.part = (double *)dalloc(h, (size_t)plen * sizeof(double));
    h.gpart = (double *)dalloc(h, (size_t)kGroups * 2 * kMaxBatch * sizeof(double));
    h.spart = (double *)dalloc(h, (size_t)std::max(kMaxGrid, kDiaGridMax) * sizeof(double));
    h.gpart_spmv = (double *)dalloc(h, (size_t)kGroups * kMaxBatch * sizeof(double));
    h.sync = (uint32_t *)dalloc(h, (size_t)kCntKinds * kCountersPerKind * sizeof(uint32_t));
    SLA_HIP(hipMemsetAsync(h.sync, 0, (size_t)kCntKinds * kCountersPerKind * sizeof(uint32_t), s));
    h.st = (SysState *)dalloc(h, sizeof(SysState) * num_systems(h));
    h.ctl = (Ctl *)dalloc(h, sizeof(Ctl));
    SLA_HIP(hipMemsetAsync(h.ctl, 0, sizeof(Ctl), s));
    h.bcast = (Bcast *)dalloc(h, sizeof(Bcast));
    SLA_HIP(hipMemsetAsync(h.bcast, 0, sizeof(Bcast), s));
    h.bcast_bv = (double *)dalloc(h, sizeof(double) * 2 * kMaxBatch);
    SLA_HIP(hipMemsetAsync(h.st, 0, sizeof(SysState) * num_systems(h), s));
    if (hipHostMalloc((void **)&h.h_running, sizeof(int32_t), hipHostMallocMapped) != hipSuccess)
        fail(SLA_ERR_OOM, "pinned host allocation failed");
    *h.h_running = 0;
    SLA_HIP(hipHostGetDevicePointer((void **)&h.d_running, h.h_running, 0));
    if (hipHostMalloc((void **)&h.h_state, sizeof(SysState) * num_systems(h), hipHostMallocDefault) !=
        hipSuccess)
        fail(SLA_ERR_OOM, "pinned host allocation failed");
    if (hipHostMalloc((void **)&h.h_ctl, sizeof(Ctl), hipHostMallocDefault) != hipSuccess)
        fail(SLA_ERR_OOM, "pinned host allocation failed");
    std::memset(h.h_ctl, 0, sizeof(Ctl));
    SLA_HIP(hipEventCreateWithFlags(&h.ev[0], hipEventDisableTiming));
    SLA_HIP(hipEventCreateWithFlags(&h.ev[1], hipEventDisableTiming));
    SLA_HIP(hipStreamCreateWithFlags(&h.cap_stream, hipStreamNonBlocking));
}

namespace {

void destroy(Handle *h) { destroy_handle(h); }

Handle *checked(sla_csr h) {
    if (!h) fail(SLA_ERR_INVALID_ARG, "null handle");
    Handle *hh = reinterpret_cast<Handle *>(h);
    SLA_HIP(hipSetDevice(hh->device));
    return hh;
}

}  // namespace
}  // namespace sla

using namespace sla;

namespace sla {
namespace {
sla_status create_impl(sla_csr *out, sla_format fmt, int64_t n, int64_t nnz_in, int32_t batch,
                       sla_itype row_itype, const void *rows_or_row_ptr, sla_itype col_itype,
                       const void *cols, sla_dtype vtype, const void *values, uint32_t flags,
                       int32_t nseg, const int64_t *seg_rows, void *stream) {
    Handle *h = nullptr;
    const sla_status st = guard([&] {
        if (!out) fail(SLA_ERR_INVALID_ARG, "out is null");
        *out = nullptr;
        if (fmt != SLA_INPUT_COO && fmt != SLA_INPUT_CSR) fail(SLA_ERR_INVALID_ARG, "bad format");
        if (n < 1 || n >= (int64_t(1) << 31)) fail(SLA_ERR_INVALID_ARG, "n must be in [1, 2^31)");
        if (nnz_in < 0 || nnz_in >= (int64_t(1) << 62)) fail(SLA_ERR_INVALID_ARG, "bad nnz");
        if (batch < 1 || batch > kMaxBatch) fail(SLA_ERR_INVALID_ARG, "batch must be in [1, 256]");
        if ((row_itype != SLA_I32 && row_itype != SLA_I64) ||
            (col_itype != SLA_I32 && col_itype != SLA_I64))
            fail(SLA_ERR_INVALID_ARG, "bad index type");
        if (vtype != SLA_F32 && vtype != SLA_F64) fail(SLA_ERR_INVALID_ARG, "bad value type");
        if (flags & ~(uint32_t)(SLA_FLAG_CHECK_SYMMETRIC | SLA_FLAG_REORDER | SLA_FLAG_NO_REORDER))
            fail(SLA_ERR_INVALID_ARG, "unknown flag");
        if ((flags & SLA_FLAG_REORDER) && (flags & SLA_FLAG_NO_REORDER))
            fail(SLA_ERR_INVALID_ARG, "SLA_FLAG_REORDER and SLA_FLAG_NO_REORDER exclude each other");
        if (fmt == SLA_INPUT_CSR && !rows_or_row_ptr) fail(SLA_ERR_INVALID_ARG, "row_ptr is null");
        if (nnz_in > 0 && (!rows_or_row_ptr || !cols || !values))
            fail(SLA_ERR_INVALID_ARG, "null index or value pointer");
        if (fmt == SLA_INPUT_CSR && row_itype == SLA_I32 && nnz_in >= (int64_t(1) << 31))
            fail(SLA_ERR_INVALID_ARG, "int32 row_ptr cannot address nnz >= 2^31");
        if (nseg > 0) {
            if (!seg_rows) fail(SLA_ERR_INVALID_ARG, "seg_rows is null");
            if (batch != 1) fail(SLA_ERR_INVALID_ARG, "a segmented handle has batch 1");
            if (flags & SLA_FLAG_REORDER)
                fail(SLA_ERR_INVALID_ARG, "a segmented handle is not reordered");
            if (seg_rows[0] != 0 || seg_rows[nseg] != n)
                fail(SLA_ERR_INVALID_ARG, "seg_rows must run from 0 to n");
            for (int32_t q = 0; q < nseg; ++q)
                if (seg_rows[q + 1] <= seg_rows[q])
                    fail(SLA_ERR_INVALID_ARG, "segments must be non-empty and in order");
            flags |= SLA_FLAG_NO_REORDER;
        }
        hipStream_t s = (hipStream_t)stream;
        h = new Handle();
        SLA_HIP(hipGetDevice(&h->device));
        h->n = n;
        h->nnz_in = nnz_in;
        h->B = batch;
        h->vt = vtype;
        h->vbytes = vtype == SLA_F64 ? 8 : 4;
        h->flags = flags;
        if (fmt == SLA_INPUT_COO)
            build_from_coo(*h, row_itype, rows_or_row_ptr, col_itype, cols, values, s);
        else
            build_from_csr(*h, row_itype, rows_or_row_ptr, col_itype, cols, values, s);
        build_tiles(*h, s, nseg > 0 ? seg_rows : nullptr, nseg);
        init_launch_limits(*h);
        init_vector_limits(*h);
        if (nseg > 0) build_segments(*h, seg_rows, nseg, s);
        alloc_workspace(*h, s);
        compute_dinv(*h, s);
        if ((flags & SLA_FLAG_CHECK_SYMMETRIC) && !check_symmetric(*h, s))
            fail(SLA_ERR_NOT_SYMMETRIC, "matrix is not symmetric (bitwise)");
        if (want_reorder(*h)) build_reordered(*h, s);
        SLA_HIP(hipStreamSynchronize(s));
        *out = reinterpret_cast<sla_csr>(h);
    });
    if (st != SLA_OK && h) destroy(h);
    return st;
}
}  // namespace
}  // namespace sla

extern "C" {

sla_status sla_csr_create(sla_csr *out, sla_format fmt, int64_t n, int64_t nnz_in, int32_t batch,
                          sla_itype row_itype, const void *rows_or_row_ptr, sla_itype col_itype,
                          const void *cols, sla_dtype vtype, const void *values, uint32_t flags,
                          void *stream) {
    return create_impl(out, fmt, n, nnz_in, batch, row_itype, rows_or_row_ptr, col_itype, cols,
                       vtype, values, flags, 0, nullptr, stream);
}

sla_status sla_csr_create_segmented(sla_csr *out, sla_format fmt, int64_t n, int64_t nnz_in,
                                    sla_itype row_itype, const void *rows_or_row_ptr,
                                    sla_itype col_itype, const void *cols, sla_dtype vtype,
                                    const void *values, int32_t nseg, const int64_t *seg_rows,
                                    uint32_t flags, void *stream) {
    if (nseg < 1) {
        g_last_error = "nseg must be >= 1";
        return SLA_ERR_INVALID_ARG;
    }
    return create_impl(out, fmt, n, nnz_in, 1, row_itype, rows_or_row_ptr, col_itype, cols, vtype,
                       values, flags, nseg, seg_rows, stream);
}

sla_status sla_csr_get_segments(sla_csr hd, int32_t *nseg, int64_t *seg_rows) {
    return guard([&] {
        Handle *h = checked(hd);
        if (nseg) *nseg = h->nseg;
        if (seg_rows && h->nseg > 0)
            SLA_HIP(hipMemcpy(seg_rows, h->seg_rows, sizeof(int64_t) * ((size_t)h->nseg + 1),
                              hipMemcpyDeviceToHost));
    });
}

sla_status sla_csr_set_values(sla_csr hd, const void *values, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (h->nnz_in > 0 && !values) fail(SLA_ERR_INVALID_ARG, "values is null");
        hipStream_t s = (hipStream_t)stream;
        load_values(*h, values, s);
        compute_dinv(*h, s);
        if ((h->flags & SLA_FLAG_CHECK_SYMMETRIC) && !check_symmetric(*h, s))
            fail(SLA_ERR_NOT_SYMMETRIC, "matrix is not symmetric (bitwise)");
        if (h->inner) reordered_set_values(*h, s);
        h->tr_stale = h->tr != nullptr;
    });
}

sla_status sla_csr_get(sla_csr hd, int64_t *n, int64_t *nnz, int64_t *nnz_in, int32_t *batch,
                       int32_t *vtype, int32_t *row_itype, const void **row_ptr,
                       const void **col_idx, const int64_t **slot) {
    return guard([&] {
        if (!hd) fail(SLA_ERR_INVALID_ARG, "null handle");
        const Handle *h = reinterpret_cast<const Handle *>(hd);
        if (n) *n = h->n;
        if (nnz) *nnz = h->nnz;
        if (nnz_in) *nnz_in = h->nnz_in;
        if (batch) *batch = h->B;
        if (vtype) *vtype = h->vt;
        if (row_itype) *row_itype = h->rp64 ? SLA_I64 : SLA_I32;
        if (row_ptr) *row_ptr = h->row_ptr;
        if (col_idx) *col_idx = h->col;
        if (slot) *slot = h->slot;
    });
}

sla_status sla_csr_get_pattern(sla_csr hd, void *row_ptr_out, void *col_idx_out,
                               int64_t *slot_out, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        hipStream_t s = (hipStream_t)stream;
        if (row_ptr_out)
            SLA_HIP(hipMemcpyAsync(row_ptr_out, h->row_ptr, (size_t)(h->n + 1) * (h->rp64 ? 8 : 4),
                                   hipMemcpyDeviceToDevice, s));
        if (col_idx_out && h->nnz > 0)
            SLA_HIP(hipMemcpyAsync(col_idx_out, h->col, (size_t)h->nnz * 4, hipMemcpyDeviceToDevice,
                                   s));
        if (slot_out && h->nnz_in > 0) {
            if (h->slot)
                SLA_HIP(hipMemcpyAsync(slot_out, h->slot, (size_t)h->nnz_in * 8,
                                       hipMemcpyDeviceToDevice, s));
            else
                iota_i64(slot_out, h->nnz_in, s);
        }
    });
}

sla_status sla_csr_get_values(sla_csr hd, void *values_out, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!values_out) fail(SLA_ERR_INVALID_ARG, "values_out is null");
        values_to_batch_major(*h, values_out, (hipStream_t)stream);
    });
}

sla_status sla_csr_gather_to_input(sla_csr hd, const void *csr_order, void *input_order,
                                   void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!csr_order || !input_order) fail(SLA_ERR_INVALID_ARG, "null pointer");
        gather_to_input(*h, csr_order, input_order, (hipStream_t)stream);
    });
}

namespace sla {
namespace {
// a solve of `caller` ran on `ran` (the reordered or transposed handle, or
// caller itself): record on the caller how it ran
void record_path(Handle &caller, const Handle &ran) {
    const Handle &r = ran.inner ? *ran.inner : ran;
    caller.last_path = r.last_path;
    caller.last_fallback = r.last_fallback;
}

// the captured iteration graphs hold the kernels of the options they were
// captured under
void drop_graphs(Handle &h) {
    if (h.graph) (void)hipGraphExecDestroy(h.graph);
    if (h.bi_graph) (void)hipGraphExecDestroy(h.bi_graph);
    h.graph = nullptr;
    h.bi_graph = nullptr;
    h.graph_k = h.bi_graph_k = 0;
}

void set_option(Handle *h, int32_t key, int64_t value) {
    switch (key) {
        case SLA_OPT_CHECK_INTERVAL:
            if (value < 1 || value > 4096) fail(SLA_ERR_INVALID_ARG, "check interval in [1, 4096]");
            h->check_k = (int)value;
            break;
        case SLA_OPT_USE_GRAPH:
            h->use_graph = value != 0;
            break;
        case SLA_OPT_PROFILE:
            h->profile = value != 0;
            break;
        case SLA_OPT_RESIDENT:
            if (value < 0 || value > 2) fail(SLA_ERR_INVALID_ARG, "resident mode in [0, 2]");
            h->res_mode = (int)value;
            break;
        case SLA_OPT_COOPERATIVE:
            h->res_coop = value != 0;
            break;
        case SLA_OPT_SPIN_LIMIT:
            if (value < 0 || value > (int64_t)0xffffffffu)
                fail(SLA_ERR_INVALID_ARG, "spin limit in [0, 2^32)");
            h->spin_limit = (uint32_t)value;
            break;
        case SLA_OPT_SPMV_RING:
            if (h->spmv_ring != (value != 0)) drop_graphs(*h);
            h->spmv_ring = value != 0;
            break;
        case SLA_OPT_FOLD_DIRECTION:
            if (h->fold_direction != (value != 0)) drop_graphs(*h);
            h->fold_direction = value != 0;
            break;
        case SLA_OPT_FUSED_UPDATE:
            if (h->fuse_update != (value != 0)) drop_graphs(*h);
            h->fuse_update = value != 0;
            break;
        case SLA_OPT_RESIDENT_WALK:
            if (value < 0 || value > 2) fail(SLA_ERR_INVALID_ARG, "resident walk in [0, 2]");
            h->res_walk = (int)value;
            break;
        case SLA_OPT_RESIDENT_DIA:
            h->res_dia_on = value != 0;
            break;
        case SLA_OPT_SPMV_DIA:
            if (h->spmv_dia != (value != 0)) drop_graphs(*h);
            h->spmv_dia = value != 0;
            break;
        default:
            fail(SLA_ERR_INVALID_ARG, "unknown option");
    }
    if (h->inner) set_option(h->inner, key, value);
    // A^T (the matvec backward, the BiCGStab adjoint) runs under A's options;
    // its launches are not profiled, so A's per-kernel figures stay A's
    if (h->tr && key != SLA_OPT_PROFILE) set_option(h->tr, key, value);
}
}  // namespace
}  // namespace sla

sla_status sla_csr_set_option(sla_csr hd, int32_t key, int64_t value) {
    return guard([&] { set_option(checked(hd), key, value); });
}

sla_status sla_spmv(sla_csr hd, const void *x, void *y, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!x || !y) fail(SLA_ERR_INVALID_ARG, "null vector");
        if (x == y) fail(SLA_ERR_INVALID_ARG, "x and y must not alias");
        if (h->inner) reordered_spmv(*h, x, y, (hipStream_t)stream);
        else spmv(*h, x, y, (hipStream_t)stream);
    });
}

sla_status sla_spmv_backward(sla_csr hd, const void *x, const void *grad_y, void *grad_x,
                             void *grad_vals_out, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!x || !grad_y) fail(SLA_ERR_INVALID_ARG, "null pointer");
        if (grad_x && (grad_x == grad_y || grad_x == x))
            fail(SLA_ERR_INVALID_ARG, "grad_x must not alias x or grad_y");
        hipStream_t s = (hipStream_t)stream;
        if (h->inner) {
            reordered_spmv_backward(*h, x, grad_y, grad_x, grad_vals_out, s);
            if (h->profile) {
                SLA_HIP(hipStreamSynchronize(s));
                flush_profile(*h->inner);
            }
            return;
        }
        Handle *t = grad_x ? transpose_for_backward(*h, s) : nullptr;
        const bool want_vals = grad_vals_out && h->nnz > 0;
        // a batch's grad_y in the internal layout [n][B] (the workspace q
        // holds it), made once for A^T g (when neither handle is reordered)
        // and the value gradient
        const bool shared = h->B > 1 && t && !t->inner && want_vals;
        const void *g_int = grad_y;
        if (h->B > 1 && (shared || want_vals)) {
            transpose(grad_y, h->q, h->B, h->n, h->vbytes, s);
            g_int = h->q;
        }
        if (t) {
            if (shared) spmv_from_internal(*t, g_int, grad_x, s);
            else any_spmv(*t, grad_y, grad_x, s);
        }
        if (want_vals) grad_vals(*h, g_int, x, grad_vals_out, s, 1.0);
        if (h->profile) {
            SLA_HIP(hipStreamSynchronize(s));
            flush_profile(*h);
        }
    });
}

sla_status sla_pcg_solve(sla_csr hd, const void *b, void *x, double tol, int32_t maxit,
                         sla_info *info, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!b || !x || !info) fail(SLA_ERR_INVALID_ARG, "null pointer");
        if (!(tol >= 0.0) || maxit < 0) fail(SLA_ERR_INVALID_ARG, "need tol >= 0 and maxit >= 0");
        if (!h->diag_ok)
            fail(SLA_ERR_BAD_DIAGONAL,
                 "Jacobi preconditioning needs every diagonal entry present, positive and finite");
        if (h->inner) reordered_pcg(*h, b, x, tol, maxit, info, (hipStream_t)stream);
        else pcg(*h, b, x, tol, maxit, info, (hipStream_t)stream, false);
        record_path(*h, *h);
    });
}

sla_status sla_adjoint_backward(sla_csr hd, const void *x, const void *grad_x, void *grad_b,
                                void *grad_vals_out, double tol, int32_t maxit, sla_info *info,
                                void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!x || !grad_x || !info) fail(SLA_ERR_INVALID_ARG, "null pointer");
        if (!(tol >= 0.0) || maxit < 0) fail(SLA_ERR_INVALID_ARG, "need tol >= 0 and maxit >= 0");
        if (!h->diag_ok)
            fail(SLA_ERR_BAD_DIAGONAL,
                 "Jacobi preconditioning needs every diagonal entry present, positive and finite");
        hipStream_t s = (hipStream_t)stream;
        if (h->inner) {
            reordered_adjoint(*h, x, grad_x, grad_b, grad_vals_out, tol, maxit, info, s);
            record_path(*h, *h);
            return;
        }
        pcg(*h, grad_x, nullptr, tol, maxit, info, s, true);  // lambda stays in the workspace
        if (grad_b) {
            if (h->B == 1)
                SLA_HIP(hipMemcpyAsync(grad_b, h->x, (size_t)h->n * h->vbytes,
                                       hipMemcpyDeviceToDevice, s));
            else
                transpose(h->x, grad_b, h->n, h->B, h->vbytes, s);
        }
        if (grad_vals_out) grad_vals(*h, h->x, x, grad_vals_out, s);
        SLA_HIP(hipStreamSynchronize(s));
        if (h->profile) flush_profile(*h);
    });
}

sla_status sla_pcg_solve_noalloc(int64_t n, int64_t nnz, const int32_t *row_ptr,
                                 const int32_t *col_idx, const double *values, const double *b,
                                 double *x, double tol, int32_t maxit, sla_info *info,
                                 void *stream) {
    return guard([&] {
        if (!row_ptr || !b || !x || !info || (nnz > 0 && (!col_idx || !values)))
            fail(SLA_ERR_INVALID_ARG, "null pointer");
        if (!(tol >= 0.0) || maxit < 0) fail(SLA_ERR_INVALID_ARG, "need tol >= 0 and maxit >= 0");
        if ((const void *)x == (const void *)b) fail(SLA_ERR_INVALID_ARG, "x and b must not alias");
        pcg_noalloc(n, nnz, row_ptr, col_idx, values, b, x, tol, maxit, kDefaultSpinLimit, info,
                    (hipStream_t)stream);
    });
}

sla_status sla_bicgstab_solve(sla_csr hd, const void *b, void *x, double tol, int32_t maxit,
                              sla_info *info, void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!b || !x || !info) fail(SLA_ERR_INVALID_ARG, "null pointer");
        if (!(tol >= 0.0) || maxit < 0) fail(SLA_ERR_INVALID_ARG, "need tol >= 0 and maxit >= 0");
        if (h->B != 1 || h->nseg > 0)
            fail(SLA_ERR_INVALID_ARG, "BiCGStab solves one system: batch 1, not segmented");
        if (!h->diag_nonzero)
            fail(SLA_ERR_BAD_DIAGONAL,
                 "Jacobi preconditioning needs every diagonal entry present, non-zero and finite");
        any_bicgstab(*h, b, x, tol, maxit, info, (hipStream_t)stream);
        record_path(*h, *h);
    });
}

sla_status sla_bicgstab_adjoint(sla_csr hd, const void *x, const void *grad_x, void *grad_b,
                                void *grad_vals_out, double tol, int32_t maxit, sla_info *info,
                                void *stream) {
    return guard([&] {
        Handle *h = checked(hd);
        if (!x || !grad_x || !info) fail(SLA_ERR_INVALID_ARG, "null pointer");
        if (!(tol >= 0.0) || maxit < 0) fail(SLA_ERR_INVALID_ARG, "need tol >= 0 and maxit >= 0");
        if (h->B != 1 || h->nseg > 0)
            fail(SLA_ERR_INVALID_ARG, "BiCGStab solves one system: batch 1, not segmented");
        if (!h->diag_nonzero)
            fail(SLA_ERR_BAD_DIAGONAL,
                 "Jacobi preconditioning needs every diagonal entry present, non-zero and finite");
        if (grad_b && (grad_b == x || grad_b == grad_x))
            fail(SLA_ERR_INVALID_ARG, "grad_b must not alias x or grad_x");
        hipStream_t s = (hipStream_t)stream;
        if (h->inner) {
            Handle &t = reordered_bicgstab_adjoint(*h, x, grad_x, grad_b, grad_vals_out, tol, maxit,
                                                   info, s);
            record_path(*h, t);
            SLA_HIP(hipStreamSynchronize(s));
            if (h->inner->profile) flush_profile(*h->inner);
            return;
        }
        // A^T lambda = grad_x by BiCGStab on A^T (the handle itself when it was
        // checked symmetric)
        Handle &at = *transpose_for_backward(*h, s);
        void *lam = grad_b;
        if (!lam) {
            if (!h->lam_tmp) h->lam_tmp = dalloc(*h, (size_t)h->n * h->vbytes);
            lam = h->lam_tmp;
        }
        any_bicgstab(at, grad_x, lam, tol, maxit, info, s);
        record_path(*h, at);
        if (grad_vals_out) grad_vals(*h, lam, x, grad_vals_out, s);
        SLA_HIP(hipStreamSynchronize(s));
        if (h->profile) flush_profile(*h);
    });
}

sla_status sla_profile_get(sla_csr hd, int32_t kind, int64_t *launches, double *total_ms) {
    return guard([&] {
        if (!hd) fail(SLA_ERR_INVALID_ARG, "null handle");
        if (kind < 0 || kind >= SLA_KERNEL_COUNT) fail(SLA_ERR_INVALID_ARG, "bad kernel kind");
        const Handle *h = reinterpret_cast<const Handle *>(hd);
        if (h->inner) h = h->inner;  // kernels run on the reordered handle
        if (launches) *launches = h->prof_launches[kind];
        if (total_ms) *total_ms = h->prof_ms[kind];
    });
}

sla_status sla_profile_reset(sla_csr hd) {
    return guard([&] {
        if (!hd) fail(SLA_ERR_INVALID_ARG, "null handle");
        for (Handle *h = reinterpret_cast<Handle *>(hd); h; h = h->inner)
            for (int k = 0; k < SLA_KERNEL_COUNT; ++k) {
                h->prof_launches[k] = 0;
                h->prof_ms[k] = 0.0;
            }
    });
}

sla_status sla_csr_memory(sla_csr hd, int64_t *bytes) {
    return guard([&] {
        if (!hd || !bytes) fail(SLA_ERR_INVALID_ARG, "null pointer");
        const Handle *h = reinterpret_cast<const Handle *>(hd);
        int64_t b = 0;
        for (const Handle *c : {h, (const Handle *)h->inner, (const Handle *)h->tr,
                                h->tr ? (const Handle *)h->tr->inner : nullptr,
                                h->inner ? (const Handle *)h->inner->tr : nullptr})
            if (c) b += c->bytes;
        *bytes = b;
    });
}

sla_status sla_csr_get_layout(sla_csr hd, int32_t *reordered, int32_t *narrow_columns,
                              int64_t *tiles, int64_t *long_rows) {
    return guard([&] {
        if (!hd) fail(SLA_ERR_INVALID_ARG, "null handle");
        const Handle *h = reinterpret_cast<const Handle *>(hd);
        if (reordered) *reordered = h->inner ? 1 : 0;
        const Handle *sv = h->inner ? h->inner : h;
        if (narrow_columns) *narrow_columns = sv->all_narrow ? (sv->ring_tiles ? 2 : 1) : 0;
        if (tiles) *tiles = sv->ntiles;
        if (long_rows) *long_rows = sv->nlong;
    });
}

sla_status sla_csr_get_last_path(sla_csr hd, int32_t *path, uint32_t *fallbacks) {
    return guard([&] {
        if (!hd) fail(SLA_ERR_INVALID_ARG, "null handle");
        const Handle *h = reinterpret_cast<const Handle *>(hd);
        if (path) *path = h->last_path;
        if (fallbacks) *fallbacks = h->last_fallback;
    });
}

sla_status sla_csr_get_diagonals(sla_csr hd, int32_t *ndiag, int32_t *per_step) {
    return guard([&] {
        const Handle *h = checked(hd);
        if (h->inner) h = h->inner;
        if (ndiag) *ndiag = (h->res_state > 0 && h->res_dia_on && h->res_dia_fits) ? h->dia_m : 0;
        if (per_step) *per_step = (h->spmv_dia && h->B == 1 && h->nseg == 0) ? h->dia_m : 0;
    });
}

void sla_csr_destroy(sla_csr hd) { destroy(reinterpret_cast<Handle *>(hd)); }

const char *sla_last_error(void) { return g_last_error.c_str(); }

const char *sla_version(void) { return "sla 0.1.0 (gfx950)"; }

}  // extern "C"

// Symmetric reordering for locality. A matrix whose rows gather from far
// apart (a graph of random points, say) makes every 8-byte gather of the SpMV
// fetch its own cache line. Reverse Cuthill-McKee on the pattern gives a
// permutation P with P A P^T banded; the solver then runs on a second handle
// holding P A P^T, and this handle maps vectors (b, x, lambda: permuted
// gathers), values (CSR position maps) and the value gradient between the
// caller's order and the solver's.
//
// Jacobi-PCG is invariant under symmetric permutation in exact arithmetic:
// diag(P A P^T) = P diag(A) P^T, and CG on (P A P^T, P b) produces P x_k at
// every step. Only the order of the terms inside each row sum changes (the
// columns of a row are sorted in the new numbering), so results agree with
// the unpermuted solve to rounding.
#include "common.h"

#include <algorithm>
#include <thread>
#include <vector>

namespace sla {

namespace {

// Reverse Cuthill-McKee order (new -> old) of the graph of the pattern
// (row_ptr, col). Components are started from a pseudo-peripheral node (two
// breadth-first sweeps from a node of least degree); each node's unvisited
// neighbours are appended in order of increasing degree.
void rcm_order(int64_t n, const std::vector<int64_t> &rp, const std::vector<int32_t> &col,
               std::vector<int32_t> &order) {
    std::vector<int32_t> deg((size_t)n);
    for (int64_t i = 0; i < n; ++i) deg[(size_t)i] = (int32_t)(rp[(size_t)i + 1] - rp[(size_t)i]);
    std::vector<int32_t> by_deg((size_t)n);
    for (int64_t i = 0; i < n; ++i) by_deg[(size_t)i] = (int32_t)i;
    std::stable_sort(by_deg.begin(), by_deg.end(),
                     [&](int32_t a, int32_t b) { return deg[(size_t)a] < deg[(size_t)b]; });
    std::vector<char> done((size_t)n, 0);
    std::vector<int32_t> stamp((size_t)n, -1);
    std::vector<int32_t> queue;
    queue.reserve((size_t)n);
    order.clear();
    order.reserve((size_t)n);
    std::vector<int32_t> nb;
    int32_t sweep = 0;
    // last level of a breadth-first sweep from r (nodes not yet ordered)
    auto last_level_min = [&](int32_t r) {
        ++sweep;
        queue.clear();
        queue.push_back(r);
        stamp[(size_t)r] = sweep;
        size_t head = 0, level_start = 0;
        while (head < queue.size()) {
            level_start = head;
            const size_t level_end = queue.size();
            for (; head < level_end; ++head) {
                const int32_t u = queue[head];
                for (int64_t k = rp[(size_t)u]; k < rp[(size_t)u + 1]; ++k) {
                    const int32_t v = col[(size_t)k];
                    if (!done[(size_t)v] && stamp[(size_t)v] != sweep) {
                        stamp[(size_t)v] = sweep;
                        queue.push_back(v);
                    }
                }
            }
        }
        int32_t best = queue[level_start];
        for (size_t i = level_start; i < queue.size(); ++i)
            if (deg[(size_t)queue[i]] < deg[(size_t)best]) best = queue[i];
        return best;
    };
    size_t next = 0;
    while ((int64_t)order.size() < n) {
        while (done[(size_t)by_deg[next]]) ++next;
        int32_t root = by_deg[next];
        root = last_level_min(root);
        root = last_level_min(root);
        size_t head = order.size();
        order.push_back(root);
        done[(size_t)root] = 1;
        while (head < order.size()) {
            const int32_t u = order[head++];
            nb.clear();
            for (int64_t k = rp[(size_t)u]; k < rp[(size_t)u + 1]; ++k) {
                const int32_t v = col[(size_t)k];
                if (!done[(size_t)v]) {
                    done[(size_t)v] = 1;
                    nb.push_back(v);
                }
            }
            std::sort(nb.begin(), nb.end(), [&](int32_t a, int32_t b) {
                return deg[(size_t)a] != deg[(size_t)b] ? deg[(size_t)a] < deg[(size_t)b] : a < b;
            });
            order.insert(order.end(), nb.begin(), nb.end());
        }
    }
    std::reverse(order.begin(), order.end());
}

template <typename F>
void parallel_rows(int64_t n, F &&f) {
    unsigned nt = std::thread::hardware_concurrency();
    if (nt < 1) nt = 1;
    if (nt > 16) nt = 16;
    if (n < 65536) nt = 1;
    std::vector<std::thread> th;
    for (unsigned t = 0; t < nt; ++t)
        th.emplace_back([&, t] {
            const int64_t a = n * t / nt, b = n * (t + 1) / nt;
            f(a, b);
        });
    for (auto &x : th) x.join();
}

// out[b][i] = in[b][new2old[i]]   (caller order -> solver order)
template <typename T>
__global__ __launch_bounds__(kBlock) void k_to_inner(const T *__restrict__ in, T *__restrict__ out,
                                                     const int32_t *__restrict__ new2old, int64_t n,
                                                     int B) {
    const int64_t total = n * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t b = f / n, i = f - b * n;
        out[f] = in[b * n + new2old[i]];
    }
}

// out[b][new2old[i]] = in[b][i]   (solver order -> caller order)
template <typename T>
__global__ __launch_bounds__(kBlock) void k_to_outer(const T *__restrict__ in, T *__restrict__ out,
                                                     const int32_t *__restrict__ new2old, int64_t n,
                                                     int B) {
    const int64_t total = n * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t b = f / n, i = f - b * n;
        out[b * n + new2old[i]] = in[f];
    }
}

// inner values [nnz][B] from this handle's [nnz][B]: row k of the inner CSR
// is row map_in[k] here
template <typename T>
__global__ __launch_bounds__(kBlock) void k_vals_to_inner(const T *__restrict__ vals,
                                                          T *__restrict__ inner,
                                                          const int64_t *__restrict__ map_in,
                                                          int64_t nnz, int B) {
    const int64_t total = nnz * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t k = f / B, b = f - k * B;
        inner[f] = vals[map_in[k] * B + b];
    }
}

// the same, written batch-major [B][nnz] (the layout create takes)
template <typename T>
__global__ __launch_bounds__(kBlock) void k_vals_to_inner_bm(const T *__restrict__ vals,
                                                             T *__restrict__ inner,
                                                             const int64_t *__restrict__ map_in,
                                                             int64_t nnz, int B) {
    const int64_t total = nnz * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t b = f / nnz, k = f - b * nnz;
        inner[f] = vals[map_in[k] * B + b];
    }
}

// gradient [B][nnz] in this handle's CSR order from the inner one's
template <typename T>
__global__ __launch_bounds__(kBlock) void k_grad_to_outer(const T *__restrict__ in,
                                                          T *__restrict__ out,
                                                          const int64_t *__restrict__ map_out,
                                                          int64_t nnz, int B) {
    const int64_t total = nnz * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t b = f / nnz, k = f - b * nnz;
        out[f] = in[b * nnz + map_out[k]];
    }
}

unsigned grid_of(int64_t total) {
    int64_t g = (total + kBlock - 1) / kBlock;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return (unsigned)g;
}

void to_inner(Handle &h, const void *in, void *out, hipStream_t s) {
    const int64_t total = h.n * h.B;
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_to_inner<double>, dim3(grid_of(total)), dim3(kBlock), 0, s,
                           (const double *)in, (double *)out, (const int32_t *)h.new2old, h.n, h.B);
    else
        hipLaunchKernelGGL(k_to_inner<float>, dim3(grid_of(total)), dim3(kBlock), 0, s,
                           (const float *)in, (float *)out, (const int32_t *)h.new2old, h.n, h.B);
    SLA_HIP(hipGetLastError());
}

void to_outer(Handle &h, const void *in, void *out, hipStream_t s) {
    const int64_t total = h.n * h.B;
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_to_outer<double>, dim3(grid_of(total)), dim3(kBlock), 0, s,
                           (const double *)in, (double *)out, (const int32_t *)h.new2old, h.n, h.B);
    else
        hipLaunchKernelGGL(k_to_outer<float>, dim3(grid_of(total)), dim3(kBlock), 0, s,
                           (const float *)in, (float *)out, (const int32_t *)h.new2old, h.n, h.B);
    SLA_HIP(hipGetLastError());
}

// the value gradient in the inner CSR order (h.rtmp_grad) to this handle's
void grad_to_outer(Handle &h, void *grad_vals_out, hipStream_t s) {
    if (h.nnz == 0) return;
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_grad_to_outer<double>, dim3(grid_of(h.nnz * h.B)), dim3(kBlock), 0, s,
                           (const double *)h.rtmp_grad, (double *)grad_vals_out,
                           (const int64_t *)h.map_out, h.nnz, h.B);
    else
        hipLaunchKernelGGL(k_grad_to_outer<float>, dim3(grid_of(h.nnz * h.B)), dim3(kBlock), 0, s,
                           (const float *)h.rtmp_grad, (float *)grad_vals_out,
                           (const int64_t *)h.map_out, h.nnz, h.B);
    SLA_HIP(hipGetLastError());
}

}  // namespace

// Handles for a matrix with the same entries as h in another arrangement
// (P A P^T, A^T): a CSR pattern and map[k] = position in h's CSR of entry k
// (device array, kept by the caller); values are gathered from h's.
namespace {

// keys[k] = col[k] (the sort key), pos[k] = k (what the sort carries)
__global__ __launch_bounds__(kBlock) void k_keys_by_column(const int32_t *__restrict__ col,
                                                           int64_t nnz, uint64_t *__restrict__ keys,
                                                           int64_t *__restrict__ pos) {
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz;
         k += (int64_t)gridDim.x * kBlock) {
        keys[k] = (uint64_t)(uint32_t)col[k];
        pos[k] = k;
    }
}

// row of each stored entry: the last row whose first entry is at or before
// it (binary search in row_ptr, so long rows cost nothing extra)
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_row_of_entry(const RP *__restrict__ row_ptr, int64_t n,
                                                         int64_t nnz, int32_t *__restrict__ rowof) {
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz;
         k += (int64_t)gridDim.x * kBlock) {
        int64_t lo = 0, hi = n - 1;   // row_ptr[lo] <= k < row_ptr[hi + 1]
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if ((int64_t)row_ptr[mid] <= k) lo = mid;
            else hi = mid - 1;
        }
        rowof[k] = (int32_t)lo;
    }
}

__global__ __launch_bounds__(kBlock) void k_gather_i32(const int32_t *__restrict__ src,
                                                       const int64_t *__restrict__ idx, int64_t m,
                                                       int32_t *__restrict__ out) {
    for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < m;
         j += (int64_t)gridDim.x * kBlock)
        out[j] = src[idx[j]];
}

// trp[c] = first position whose key is >= c, c = 0..n (keys sorted)
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_column_starts(const uint64_t *__restrict__ keys,
                                                          int64_t nnz, int64_t n,
                                                          RP *__restrict__ trp) {
    for (int64_t c = (int64_t)blockIdx.x * kBlock + threadIdx.x; c <= n;
         c += (int64_t)gridDim.x * kBlock) {
        int64_t lo = 0, hi = nnz;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (keys[mid] < (uint64_t)c) lo = mid + 1;
            else hi = mid;
        }
        trp[c] = (RP)lo;
    }
}

}  // namespace

// A handle of the matrix whose CSR pattern is (d_rp, d_col) (device arrays,
// d_rp int64 when rp64 else int32, [n+1]; d_col int32 [nnz]) and whose entry
// j takes h's value at CSR position map[j] (device, kept by the caller).
Handle *make_child_dev(Handle &h, int64_t n, int64_t nnz, const void *d_rp, bool rp64,
                       const int32_t *d_col, const int64_t *map, uint32_t flags, hipStream_t s) {
    void *d_vals = nullptr;
    SLA_HIP(hipMalloc(&d_vals, (size_t)(nnz + 1) * h.B * h.vbytes));
    Handle *in = nullptr;
    try {
        if (nnz > 0) {
            if (h.vt == SLA_F64)
                hipLaunchKernelGGL(k_vals_to_inner_bm<double>, dim3(grid_of(nnz * h.B)), dim3(kBlock),
                                   0, s, (const double *)h.vals, (double *)d_vals, map, nnz, h.B);
            else
                hipLaunchKernelGGL(k_vals_to_inner_bm<float>, dim3(grid_of(nnz * h.B)), dim3(kBlock),
                                   0, s, (const float *)h.vals, (float *)d_vals, map, nnz, h.B);
            SLA_HIP(hipGetLastError());
        }
        in = new Handle();
        in->device = h.device;
        in->n = n;
        in->nnz_in = nnz;
        in->B = h.B;
        in->vt = h.vt;
        in->vbytes = h.vbytes;
        in->flags = flags;
        build_from_csr(*in, rp64 ? SLA_I64 : SLA_I32, d_rp, SLA_I32, d_col, d_vals, s);
        build_tiles(*in, s);
        init_launch_limits(*in);
        init_vector_limits(*in);
        alloc_workspace(*in, s);
        compute_dinv(*in, s);
        if (want_reorder(*in)) build_reordered(*in, s);
        SLA_HIP(hipStreamSynchronize(s));
    } catch (...) {
        (void)hipFree(d_vals);
        if (in) destroy_handle(in);
        throw;
    }
    SLA_HIP(hipFree(d_vals));
    return in;
}

// the same from host pattern arrays
Handle *make_child(Handle &h, const std::vector<int64_t> &rp, const std::vector<int32_t> &col,
                   const int64_t *map, uint32_t flags, hipStream_t s) {
    const int64_t n = (int64_t)rp.size() - 1, nnz = (int64_t)col.size();
    const bool rp64 = nnz >= ((int64_t)1 << 31);
    void *d_rp = nullptr, *d_col = nullptr;
    SLA_HIP(hipMalloc(&d_rp, (size_t)(n + 1) * (rp64 ? 8 : 4)));
    SLA_HIP(hipMalloc(&d_col, 4 * (size_t)(nnz + 1)));
    Handle *in = nullptr;
    try {
        if (rp64) {
            SLA_HIP(hipMemcpyAsync(d_rp, rp.data(), 8 * (size_t)(n + 1), hipMemcpyHostToDevice, s));
        } else {
            std::vector<int32_t> r32((size_t)n + 1);
            for (int64_t i = 0; i <= n; ++i) r32[(size_t)i] = (int32_t)rp[(size_t)i];
            SLA_HIP(hipMemcpyAsync(d_rp, r32.data(), 4 * (size_t)(n + 1), hipMemcpyHostToDevice, s));
            SLA_HIP(hipStreamSynchronize(s));
        }
        if (nnz > 0)
            SLA_HIP(hipMemcpyAsync(d_col, col.data(), 4 * (size_t)nnz, hipMemcpyHostToDevice, s));
        in = make_child_dev(h, n, nnz, d_rp, rp64, (const int32_t *)d_col, map, flags, s);
    } catch (...) {
        (void)hipFree(d_rp);
        (void)hipFree(d_col);
        throw;
    }
    SLA_HIP(hipFree(d_rp));
    SLA_HIP(hipFree(d_col));
    return in;
}

// values of a child from h's (same map as at make_child)
void child_values(Handle &h, Handle &child, const int64_t *map, hipStream_t s) {
    if (h.nnz > 0) {
        if (h.vt == SLA_F64)
            hipLaunchKernelGGL(k_vals_to_inner<double>, dim3(grid_of(h.nnz * h.B)), dim3(kBlock), 0,
                               s, (const double *)h.vals, (double *)child.vals, map, h.nnz, h.B);
        else
            hipLaunchKernelGGL(k_vals_to_inner<float>, dim3(grid_of(h.nnz * h.B)), dim3(kBlock), 0,
                               s, (const float *)h.vals, (float *)child.vals, map, h.nnz, h.B);
        SLA_HIP(hipGetLastError());
    }
    dia_scatter(child, s);
    compute_dinv(child, s);
    if (child.inner) reordered_set_values(child, s);
}

// y = A x for any handle (reordered or not), vectors in the caller's order
void any_spmv(Handle &h, const void *x, void *y, hipStream_t s) {
    if (h.inner) reordered_spmv(h, x, y, s);
    else spmv(h, x, y, s);
}

// Reorder when asked to, or automatically when most SpMV tiles gather from
// column ranges of 2^16 or more (poor locality) on a matrix large enough for
// it to matter (n >= 2^16) and small enough for the host ordering (nnz < 2^28).
bool want_reorder(const Handle &h) {
    if (h.flags & SLA_FLAG_NO_REORDER) return false;
    if (h.flags & SLA_FLAG_REORDER) return h.n > 1;
    return h.n >= (1 << 16) && h.nnz < ((int64_t)1 << 28) && 2 * h.wide_tiles > h.ntiles;
}

// Build the solver handle of P A P^T from this handle's CSR (already
// assembled, values loaded).
void build_reordered(Handle &h, hipStream_t s) {
    const int64_t n = h.n, nnz = h.nnz;
    std::vector<int64_t> rp((size_t)n + 1);
    std::vector<int32_t> col((size_t)nnz);
    if (h.rp64) {
        SLA_HIP(hipMemcpyAsync(rp.data(), h.row_ptr, 8 * (size_t)(n + 1), hipMemcpyDeviceToHost, s));
    } else {
        std::vector<int32_t> r32((size_t)n + 1);
        SLA_HIP(hipMemcpyAsync(r32.data(), h.row_ptr, 4 * (size_t)(n + 1), hipMemcpyDeviceToHost, s));
        SLA_HIP(hipStreamSynchronize(s));
        for (int64_t i = 0; i <= n; ++i) rp[(size_t)i] = r32[(size_t)i];
    }
    if (nnz > 0)
        SLA_HIP(hipMemcpyAsync(col.data(), h.col, 4 * (size_t)nnz, hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));

    std::vector<int32_t> order;  // new -> old
    rcm_order(n, rp, col, order);
    std::vector<int32_t> old2new((size_t)n);
    for (int64_t i = 0; i < n; ++i) old2new[(size_t)order[(size_t)i]] = (int32_t)i;

    // P A P^T in CSR: row i is row order[i] of A with columns renumbered and
    // sorted; map_in[k'] = position in A's CSR of entry k'
    std::vector<int64_t> irp((size_t)n + 1);
    irp[0] = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t o = order[(size_t)i];
        irp[(size_t)i + 1] = irp[(size_t)i] + (rp[(size_t)o + 1] - rp[(size_t)o]);
    }
    std::vector<int32_t> icol((size_t)nnz);
    std::vector<int64_t> map_in((size_t)nnz), map_out((size_t)nnz);
    parallel_rows(n, [&](int64_t a, int64_t b) {
        std::vector<std::pair<int32_t, int64_t>> e;
        for (int64_t i = a; i < b; ++i) {
            const int32_t o = order[(size_t)i];
            e.clear();
            for (int64_t k = rp[(size_t)o]; k < rp[(size_t)o + 1]; ++k)
                e.emplace_back(old2new[(size_t)col[(size_t)k]], k);
            std::sort(e.begin(), e.end());
            int64_t pos = irp[(size_t)i];
            for (const auto &pr : e) {
                icol[(size_t)pos] = pr.first;
                map_in[(size_t)pos] = pr.second;
                map_out[(size_t)pr.second] = pos;
                ++pos;
            }
        }
    });

    // device copies: maps, permutation, and the solver handle of P A P^T
    h.new2old = (int32_t *)dalloc(h, sizeof(int32_t) * (size_t)n);
    h.map_in = (int64_t *)dalloc(h, sizeof(int64_t) * (size_t)(nnz + 1));
    h.map_out = (int64_t *)dalloc(h, sizeof(int64_t) * (size_t)(nnz + 1));
    const size_t vec = (size_t)n * h.B * h.vbytes;
    h.rtmp[0] = dalloc(h, vec);
    h.rtmp[1] = dalloc(h, vec);
    h.rtmp_grad = dalloc(h, (size_t)(nnz + 1) * h.B * h.vbytes);
    SLA_HIP(hipMemcpyAsync(h.new2old, order.data(), sizeof(int32_t) * (size_t)n,
                           hipMemcpyHostToDevice, s));
    if (nnz > 0) {
        SLA_HIP(hipMemcpyAsync(h.map_in, map_in.data(), 8 * (size_t)nnz, hipMemcpyHostToDevice, s));
        SLA_HIP(hipMemcpyAsync(h.map_out, map_out.data(), 8 * (size_t)nnz, hipMemcpyHostToDevice, s));
    }
    h.inner = make_child(h, irp, icol, h.map_in, SLA_FLAG_NO_REORDER, s);
}

// after this handle's values changed: the inner values and Jacobi diagonal
void reordered_set_values(Handle &h, hipStream_t s) {
    child_values(h, *h.inner, h.map_in, s);
    h.inner->tr_stale = h.inner->tr != nullptr;
}

void reordered_spmv(Handle &h, const void *x, void *y, hipStream_t s) {
    to_inner(h, x, h.rtmp[0], s);
    spmv(*h.inner, h.rtmp[0], h.rtmp[1], s);
    to_outer(h, h.rtmp[1], y, s);
}

void reordered_pcg(Handle &h, const void *b, void *x, double tol, int32_t maxit, sla_info *info,
                   hipStream_t s) {
    to_inner(h, b, h.rtmp[0], s);
    pcg(*h.inner, h.rtmp[0], h.rtmp[1], tol, maxit, info, s, false);
    to_outer(h, h.rtmp[1], x, s);
    SLA_HIP(hipStreamSynchronize(s));
}

void reordered_bicgstab(Handle &h, const void *b, void *x, double tol, int32_t maxit,
                        sla_info *info, hipStream_t s) {
    to_inner(h, b, h.rtmp[0], s);
    bicgstab(*h.inner, h.rtmp[0], h.rtmp[1], tol, maxit, info, s, false);
    to_outer(h, h.rtmp[1], x, s);
    SLA_HIP(hipStreamSynchronize(s));
}

void any_bicgstab(Handle &h, const void *b, void *x, double tol, int32_t maxit, sla_info *info,
                  hipStream_t s) {
    if (h.inner) reordered_bicgstab(h, b, x, tol, maxit, info, s);
    else bicgstab(h, b, x, tol, maxit, info, s, false);
}

void reordered_adjoint(Handle &h, const void *x, const void *g, void *grad_b, void *grad_vals_out,
                       double tol, int32_t maxit, sla_info *info, hipStream_t s) {
    Handle &in = *h.inner;
    to_inner(h, g, h.rtmp[0], s);
    pcg(in, h.rtmp[0], nullptr, tol, maxit, info, s, true);  // lambda stays in in.x
    if (grad_b) {
        if (in.B == 1)
            SLA_HIP(hipMemcpyAsync(h.rtmp[1], in.x, (size_t)in.n * in.vbytes,
                                   hipMemcpyDeviceToDevice, s));
        else
            transpose(in.x, h.rtmp[1], in.n, in.B, in.vbytes, s);
        to_outer(h, h.rtmp[1], grad_b, s);
    }
    if (grad_vals_out) {
        to_inner(h, x, h.rtmp[1], s);
        grad_vals(in, in.x, h.rtmp[1], h.rtmp_grad, s);
        grad_to_outer(h, grad_vals_out, s);
    }
    SLA_HIP(hipStreamSynchronize(s));
    if (in.profile) flush_profile(in);
}

// A^T for a backward on a reordered handle, in the inner order: (P A P^T)^T
// (the inner handle itself when A was checked symmetric)
Handle &inner_transpose(Handle &h, hipStream_t s) {
    Handle &in = *h.inner;
    return (h.flags & SLA_FLAG_CHECK_SYMMETRIC) ? in : *transpose_for_backward(in, s);
}

// The backward of y = A x on a reordered handle, through P A P^T: A^T g =
// P^T (P A P^T)^T P g, and g_i x_j formed on the inner pattern (banded, so
// its gathers stay local) and moved to this handle's CSR order.
void reordered_spmv_backward(Handle &h, const void *x, const void *g, void *grad_x,
                             void *grad_vals_out, hipStream_t s) {
    Handle &in = *h.inner;
    to_inner(h, g, h.rtmp[0], s);
    if (grad_x) {
        spmv(inner_transpose(h, s), h.rtmp[0], h.rtmp[1], s);
        to_outer(h, h.rtmp[1], grad_x, s);
    }
    if (grad_vals_out && h.nnz > 0) {
        to_inner(h, x, h.rtmp[1], s);
        const void *g_int = h.rtmp[0];
        if (in.B > 1) {
            transpose(h.rtmp[0], in.q, in.B, in.n, in.vbytes, s);
            g_int = in.q;
        }
        grad_vals(in, g_int, h.rtmp[1], h.rtmp_grad, s, 1.0);
        grad_to_outer(h, grad_vals_out, s);
    }
}

// The BiCGStab adjoint on a reordered handle: (P A P^T)^T (P lambda) = P g,
// then the value gradient as above. Returns the handle that solved.
Handle &reordered_bicgstab_adjoint(Handle &h, const void *x, const void *g, void *grad_b,
                                   void *grad_vals_out, double tol, int32_t maxit,
                                   sla_info *info, hipStream_t s) {
    Handle &in = *h.inner;
    Handle &t = inner_transpose(h, s);
    to_inner(h, g, h.rtmp[0], s);
    bicgstab(t, h.rtmp[0], h.rtmp[1], tol, maxit, info, s, false);   // P lambda
    if (grad_b) to_outer(h, h.rtmp[1], grad_b, s);
    if (grad_vals_out && h.nnz > 0) {
        to_inner(h, x, h.rtmp[0], s);
        grad_vals(in, h.rtmp[1], h.rtmp[0], h.rtmp_grad, s);
        grad_to_outer(h, grad_vals_out, s);
    }
    return t;
}

// ------------------------------------------------------------------ A^T for the matvec backward
// The backward of y = A x needs A^T g. A handle checked for bitwise symmetry
// uses itself (row i of A^T holds the same values in the same column order as
// row i of A). Otherwise the first backward builds a child handle of A^T on
// the device (rows of A^T list their entries in increasing row of A), values
// gathered from A's through a position map, refreshed after set_values.
Handle *transpose_for_backward(Handle &h, hipStream_t s) {
    if (h.flags & SLA_FLAG_CHECK_SYMMETRIC) return &h;
    if (h.tr) {
        if (h.tr_stale) {
            child_values(h, *h.tr, h.tr_map, s);
            h.tr_stale = false;
        }
        return h.tr;
    }
    // A^T's pattern on the device: a stable sort of the CSR positions by
    // column (rows stay ascending inside each column, since positions are in
    // row order) gives A^T's entries in its CSR order; the sorted positions
    // are the value map, the rows of those positions A^T's columns, and the
    // first sorted position of each column A^T's row pointer.
    const int64_t n = h.n, nnz = h.nnz;
    const bool rp64 = nnz >= ((int64_t)1 << 31);
    h.tr_map = (int64_t *)dalloc(h, sizeof(int64_t) * (size_t)(nnz + 1));
    uint64_t *keys = nullptr;
    int32_t *rowof = nullptr, *tcol = nullptr;
    void *trp = nullptr;
    SLA_HIP(hipMallocAsync((void **)&keys, sizeof(uint64_t) * (size_t)(nnz + 1), s));
    SLA_HIP(hipMallocAsync((void **)&rowof, sizeof(int32_t) * (size_t)(nnz + 1), s));
    SLA_HIP(hipMallocAsync((void **)&tcol, sizeof(int32_t) * (size_t)(nnz + 1), s));
    SLA_HIP(hipMallocAsync(&trp, (size_t)(n + 1) * (rp64 ? 8 : 4), s));
    Handle *tr = nullptr;
    try {
        int bits = 0;
        while (bits < 63 && ((int64_t)1 << bits) < n) ++bits;
        if (nnz > 0) {
            hipLaunchKernelGGL(k_keys_by_column, dim3(grid_of(nnz)), dim3(kBlock), 0, s,
                               (const int32_t *)h.col, nnz, keys, h.tr_map);
            if (h.rp64)
                hipLaunchKernelGGL(k_row_of_entry<int64_t>, dim3(grid_of(nnz)), dim3(kBlock), 0, s,
                                   (const int64_t *)h.row_ptr, n, nnz, rowof);
            else
                hipLaunchKernelGGL(k_row_of_entry<int32_t>, dim3(grid_of(nnz)), dim3(kBlock), 0, s,
                                   (const int32_t *)h.row_ptr, n, nnz, rowof);
            SLA_HIP(hipGetLastError());
            radix_sort_pairs(keys, h.tr_map, nnz, bits, s);
            hipLaunchKernelGGL(k_gather_i32, dim3(grid_of(nnz)), dim3(kBlock), 0, s,
                               (const int32_t *)rowof, (const int64_t *)h.tr_map, nnz, tcol);
            SLA_HIP(hipGetLastError());
        }
        if (rp64)
            hipLaunchKernelGGL(k_column_starts<int64_t>, dim3(grid_of(n + 1)), dim3(kBlock), 0, s,
                               (const uint64_t *)keys, nnz, n, (int64_t *)trp);
        else
            hipLaunchKernelGGL(k_column_starts<int32_t>, dim3(grid_of(n + 1)), dim3(kBlock), 0, s,
                               (const uint64_t *)keys, nnz, n, (int32_t *)trp);
        SLA_HIP(hipGetLastError());
        // (a reordered handle's backward goes through its inner handle, so
        // A^T itself is never reordered)
        tr = make_child_dev(h, n, nnz, trp, rp64, tcol, h.tr_map, SLA_FLAG_NO_REORDER, s);
    } catch (...) {
        (void)hipFreeAsync(keys, s);
        (void)hipFreeAsync(rowof, s);
        (void)hipFreeAsync(tcol, s);
        (void)hipFreeAsync(trp, s);
        throw;
    }
    SLA_HIP(hipFreeAsync(keys, s));
    SLA_HIP(hipFreeAsync(rowof, s));
    SLA_HIP(hipFreeAsync(tcol, s));
    SLA_HIP(hipFreeAsync(trp, s));
    // A^T runs under the options set on A (set_option reaches it from now
    // on), profiling aside
    tr->check_k = h.check_k;
    tr->use_graph = h.use_graph;
    tr->res_mode = h.res_mode;
    tr->res_coop = h.res_coop;
    tr->res_walk = h.res_walk;
    tr->spin_limit = h.spin_limit;
    tr->spmv_ring = h.spmv_ring;
    tr->fold_direction = h.fold_direction;
    tr->fuse_update = h.fuse_update;
    h.tr = tr;
    h.tr_stale = false;
    return h.tr;
}

}  // namespace sla

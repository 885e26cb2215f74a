// CSR assembly on the device: COO validation, stable (row, col) ordering,
// in-order duplicate merge, row pointers, slot map; CSR validation and
// adoption; SpMV tiles; Jacobi reciprocal; bitwise symmetry check.
//
// The storage a SparseTensor needs (one matrix, or a batch of value sets on
// one pattern: torch-sla, tensor-types passage of its API section) is built
// here. Duplicate entries are summed left to right in input order, in the
// value type, so the result is bit-identical for any launch configuration.
#include <type_traits>

#include <algorithm>
#include <cmath>

#include "common.h"

namespace sla {

namespace {

enum : int { kBadIndex = 1, kUnsorted = 2, kBadCsr = 4 };

template <typename I>
__device__ __forceinline__ int64_t ld_idx(const I *p, int64_t k) {
    return (int64_t)p[k];
}

template <typename RI, typename CI>
__global__ __launch_bounds__(kBlock) void k_coo_check(const RI *__restrict__ rows,
                                                      const CI *__restrict__ cols, int64_t m,
                                                      int64_t n, int *__restrict__ flags) {
    int f = 0;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < m;
         e += (int64_t)gridDim.x * kBlock) {
        const int64_t r = ld_idx(rows, e), c = ld_idx(cols, e);
        if (r < 0 || r >= n || c < 0 || c >= n) f |= kBadIndex;
        if (e + 1 < m) {
            const int64_t r2 = ld_idx(rows, e + 1), c2 = ld_idx(cols, e + 1);
            if (!(r < r2 || (r == r2 && c < c2))) f |= kUnsorted;
        }
    }
    if (f) atomicOr(flags, f);
}

// row_ptr of a row-sorted index list: row_ptr[r] = first position with row >= r
template <typename RI, typename RP>
__global__ __launch_bounds__(kBlock) void k_rowptr_sorted(const RI *__restrict__ rows, int64_t m,
                                                          int64_t n, RP *__restrict__ row_ptr) {
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e <= m;
         e += (int64_t)gridDim.x * kBlock) {
        const int64_t prev = e == 0 ? -1 : ld_idx(rows, e - 1);
        const int64_t cur = e == m ? n : ld_idx(rows, e);
        for (int64_t r = prev + 1; r <= cur; ++r) row_ptr[r] = (RP)e;
    }
}

template <typename S, typename D>
__global__ __launch_bounds__(kBlock) void k_convert(const S *__restrict__ in, int64_t m,
                                                    D *__restrict__ out) {
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < m;
         e += (int64_t)gridDim.x * kBlock)
        out[e] = (D)in[e];
}

template <typename RI, typename CI>
__global__ __launch_bounds__(kBlock) void k_make_keys(const RI *__restrict__ rows,
                                                      const CI *__restrict__ cols, int64_t m,
                                                      int64_t n, uint64_t *__restrict__ keys,
                                                      int64_t *__restrict__ idx) {
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < m;
         e += (int64_t)gridDim.x * kBlock) {
        keys[e] = (uint64_t)ld_idx(rows, e) * (uint64_t)n + (uint64_t)ld_idx(cols, e);
        idx[e] = e;
    }
}

__global__ __launch_bounds__(kBlock) void k_heads(const uint64_t *__restrict__ keys, int64_t m,
                                                  int64_t *__restrict__ head) {
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < m;
         t += (int64_t)gridDim.x * kBlock)
        head[t] = (t == 0 || keys[t] != keys[t - 1]) ? 1 : 0;
}

__global__ __launch_bounds__(kBlock) void k_unique(const uint64_t *__restrict__ keys,
                                                   const int64_t *__restrict__ perm,
                                                   const int64_t *__restrict__ excl,
                                                   const int64_t *__restrict__ head, int64_t m,
                                                   int64_t n, int32_t *__restrict__ col,
                                                   int64_t *__restrict__ urow,
                                                   int64_t *__restrict__ run,
                                                   int64_t *__restrict__ slot) {
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < m;
         t += (int64_t)gridDim.x * kBlock) {
        const int64_t u = excl[t] + head[t] - 1;
        if (head[t]) {
            const uint64_t k = keys[t];
            run[u] = t;
            urow[u] = (int64_t)(k / (uint64_t)n);
            col[u] = (int32_t)(k % (uint64_t)n);
        }
        slot[perm[t]] = u;
    }
}

// CSR entry u (of value set b) = v[run[u]] + v[run[u]+1] + ... in sorted
// order, which is input order within one position (stable sort).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_merge(const T *__restrict__ vin,
                                                  const int64_t *__restrict__ perm,
                                                  const int64_t *__restrict__ run, int64_t nnz,
                                                  int64_t nnz_in, int B, T *__restrict__ out) {
    const int64_t total = nnz * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t u = f / B;
        const int b = (int)(f - u * B);
        const T *vb = vin + (int64_t)b * nnz_in;
        const int64_t t0 = run[u], t1 = run[u + 1];
        T acc = vb[perm[t0]];
        for (int64_t t = t0 + 1; t < t1; ++t) acc = acc + vb[perm[t]];
        out[f] = acc;
    }
}

template <typename RI, typename CI>
__global__ __launch_bounds__(kBlock) void k_csr_check(const RI *__restrict__ row_ptr,
                                                      const CI *__restrict__ cols, int64_t n,
                                                      int64_t nnz, int *__restrict__ flags) {
    int f = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t a = ld_idx(row_ptr, i), b = ld_idx(row_ptr, i + 1);
        if (i == 0 && a != 0) f |= kBadCsr;
        if (i == n - 1 && b != nnz) f |= kBadCsr;
        if (a < 0 || b > nnz || b < a) {
            f |= kBadCsr;
            continue;  // never index outside [0, nnz)
        }
        int64_t prevc = -1;
        for (int64_t k = a; k < b; ++k) {
            const int64_t c = ld_idx(cols, k);
            if (c < 0 || c >= n) f |= kBadIndex;
            if (c <= prevc) f |= kBadCsr;
            prevc = c;
        }
    }
    if (f) atomicOr(flags, f);
}

template <typename RP>
__global__ __launch_bounds__(kBlock) void k_tile_flags(const RP *__restrict__ row_ptr, int64_t n,
                                                       int64_t band_n, int64_t band_l,
                                                       int64_t *__restrict__ flag) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t a = row_ptr[i], b = row_ptr[i + 1];
        const bool long_i = (b - a) > kLongRow;
        int64_t f = 1;
        if (i > 0) {
            const int64_t pa = row_ptr[i - 1];
            const bool long_prev = (a - pa) > kLongRow;
            // banded: tile j holds the rows i with floor(i L / N) = j, so tile
            // j + L is tile j moved down by N rows; else runs of kTileUnits
            // rows + entries
            const bool cut = band_l > 0 ? (i * band_l) / band_n != ((i - 1) * band_l) / band_n
                                        : (pa + (i - 1)) / kTileUnits != (a + i) / kTileUnits;
            f = (long_i || long_prev || cut) ? 1 : 0;
        }
        flag[i] = f;
    }
}

// Band test of a pattern: the farthest column to the right of row i is
// i + band for at least 9 rows in 10 (a stencil on a grid: band = the grid's
// largest stride). Counts the rows that match `band` and the longest row.
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_band_count(const RP *__restrict__ row_ptr,
                                                       const int32_t *__restrict__ col, int64_t n,
                                                       int64_t band,
                                                       unsigned long long *__restrict__ match,
                                                       int *__restrict__ maxlen) {
    unsigned long long m = 0;
    int ml = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t a = row_ptr[i], b = row_ptr[i + 1];
        if (b > a && (int64_t)col[b - 1] - i == band) ++m;
        ml = max(ml, (int)min(b - a, (int64_t)1 << 30));
    }
    if (m) atomicAdd(match, m);
    if (ml) atomicMax(maxlen, ml);
}

__global__ __launch_bounds__(kBlock) void k_tile_fill(const int64_t *__restrict__ flag,
                                                      const int64_t *__restrict__ excl, int64_t n,
                                                      int32_t *__restrict__ tile_start) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        if (flag[i]) tile_start[excl[i]] = (int32_t)i;
}

template <typename RP>
__global__ __launch_bounds__(kBlock) void k_tile_k0(const RP *__restrict__ row_ptr,
                                                   const int32_t *__restrict__ tile_start,
                                                   int64_t nt, int64_t *__restrict__ tile_k0) {
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t <= nt;
         t += (int64_t)gridDim.x * kBlock)
        tile_k0[t] = (int64_t)row_ptr[tile_start[t]];
}

// dinv[i][b] = 1 / A_ii (IEEE division; fp32 storage: formed in fp64, rounded
// once) for every present, non-zero, finite diagonal; 0 otherwise. Flags:
// kDiagUnusable for a missing, zero or non-finite diagonal (no Jacobi at
// all), kDiagNegative for a negative one (Jacobi-PCG needs positive ones).
constexpr int kDiagUnusable = 1, kDiagNegative = 2;

template <typename T, typename RP>
__global__ __launch_bounds__(kBlock) void k_dinv(const RP *__restrict__ row_ptr,
                                                 const int32_t *__restrict__ col,
                                                 const T *__restrict__ vals, int64_t n, int B,
                                                 T *__restrict__ dinv, int *__restrict__ bad) {
    int flags = 0;
    const int64_t total = n * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t i = f / B;
        const int b = (int)(f - i * B);
        int64_t lo = row_ptr[i], hi = row_ptr[i + 1];
        while (lo < hi) {  // first column >= i
            const int64_t mid = (lo + hi) >> 1;
            if (col[mid] < i) lo = mid + 1;
            else hi = mid;
        }
        const bool found = lo < (int64_t)row_ptr[i + 1] && col[lo] == i;
        const double d = found ? (double)vals[lo * B + b] : 0.0;
        if (!found || d == 0.0 || !isfinite(d)) {
            flags |= kDiagUnusable;
            dinv[f] = (T)0;
        } else {
            if (d < 0.0) flags |= kDiagNegative;
            dinv[f] = (T)(1.0 / d);
        }
    }
    if (flags) atomicOr(bad, flags);
}

template <typename T>
struct Bits;
template <>
struct Bits<float> {
    using U = uint32_t;
};
template <>
struct Bits<double> {
    using U = uint64_t;
};

template <typename T, typename RP>
__global__ __launch_bounds__(kBlock) void k_symmetric(const RP *__restrict__ row_ptr,
                                                      const int32_t *__restrict__ col,
                                                      const T *__restrict__ vals, int64_t n, int B,
                                                      int *__restrict__ flag) {
    using U = typename Bits<T>::U;
    const U *bits = reinterpret_cast<const U *>(vals);
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        for (int64_t k = row_ptr[i]; k < (int64_t)row_ptr[i + 1]; ++k) {
            const int64_t j = col[k];
            int64_t lo = row_ptr[j], hi = row_ptr[j + 1];
            while (lo < hi) {
                const int64_t mid = (lo + hi) >> 1;
                if (col[mid] < i) lo = mid + 1;
                else hi = mid;
            }
            if (!(lo < (int64_t)row_ptr[j + 1] && col[lo] == i)) {
                bad = 1;
                continue;
            }
            for (int b = 0; b < B; ++b)
                if (bits[k * B + b] != bits[lo * B + b]) bad = 1;
        }
    }
    if (bad) atomicOr(flag, 1);
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_gather(const T *__restrict__ in,
                                                   const int64_t *__restrict__ slot, int64_t nnz,
                                                   int64_t nnz_in, int B, T *__restrict__ out) {
    const int64_t total = nnz_in * B;
    for (int64_t f = (int64_t)blockIdx.x * kBlock + threadIdx.x; f < total;
         f += (int64_t)gridDim.x * kBlock) {
        const int64_t b = f / nnz_in;
        const int64_t e = f - b * nnz_in;
        out[f] = in[b * nnz + slot[e]];
    }
}

inline unsigned grid_for(int64_t work) {
    int64_t g = (work + kBlock - 1) / kBlock;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

template <typename F>
void dispatch_idx(sla_itype it, F &&f) {
    if (it == SLA_I32) f((const int32_t *)nullptr);
    else f((const int64_t *)nullptr);
}

int read_flag(int *dflag, hipStream_t s) {
    int h = 0;
    SLA_HIP(hipMemcpyAsync(&h, dflag, sizeof(int), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    return h;
}

int64_t read_i64(const int64_t *d, hipStream_t s) {
    int64_t h = 0;
    SLA_HIP(hipMemcpyAsync(&h, d, sizeof(int64_t), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    return h;
}

struct Scratch {
    hipStream_t s;
    std::vector<void *> ptrs;
    explicit Scratch(hipStream_t s_) : s(s_) {}
    template <typename T>
    T *get(int64_t count) {
        void *p = nullptr;
        SLA_HIP(hipMallocAsync(&p, (size_t)(count > 0 ? count : 1) * sizeof(T), s));
        ptrs.push_back(p);
        return (T *)p;
    }
    ~Scratch() {
        for (void *p : ptrs) (void)hipFreeAsync(p, s);
    }
};

}  // namespace

// spare entries past nnz: column 0, value 0 (read by grouped loads, never used)
void zero_padding(Handle &h, hipStream_t s) {
    SLA_HIP(hipMemsetAsync(h.col + h.nnz, 0, (size_t)kEntryPad * 4, s));
    SLA_HIP(hipMemsetAsync((char *)h.vals + (size_t)h.nnz * h.B * h.vbytes, 0,
                           (size_t)kEntryPad * h.B * h.vbytes, s));
}

// ------------------------------------------------------------------ COO input

void build_from_coo(Handle &h, sla_itype rit, const void *rows, sla_itype cit, const void *cols,
                    const void *values, hipStream_t s) {
    const int64_t m = h.nnz_in, n = h.n;
    Scratch sc(s);
    int *dflag = sc.get<int>(1);
    SLA_HIP(hipMemsetAsync(dflag, 0, sizeof(int), s));
    if (m > 0) {
        auto launch = [&](auto rtag, auto ctag) {
            using RI = std::remove_const_t<std::remove_pointer_t<decltype(rtag)>>;
            using CI = std::remove_const_t<std::remove_pointer_t<decltype(ctag)>>;
            hipLaunchKernelGGL((k_coo_check<RI, CI>), dim3(grid_for(m)), dim3(kBlock), 0, s,
                               (const RI *)rows, (const CI *)cols, m, n, dflag);
        };
        dispatch_idx(rit, [&](auto r) { dispatch_idx(cit, [&](auto c) { launch(r, c); }); });
        SLA_HIP(hipGetLastError());
    }
    const int flags = read_flag(dflag, s);
    if (flags & kBadIndex) fail(SLA_ERR_INDEX_RANGE, "a COO row or column index is outside [0, n)");

    if (!(flags & kUnsorted)) {
        // sorted, duplicate-free input: the permutation and the slot map are the identity
        h.nnz = m;
        h.rp64 = m >= (int64_t(1) << 31);
        h.row_ptr = dalloc(h, (size_t)(n + 1) * (h.rp64 ? 8 : 4));
        h.col = (int32_t *)dalloc(h, (size_t)(m + kEntryPad) * 4);
        auto launch = [&](auto rtag) {
            using RI = std::remove_const_t<std::remove_pointer_t<decltype(rtag)>>;
            if (h.rp64)
                hipLaunchKernelGGL((k_rowptr_sorted<RI, int64_t>), dim3(grid_for(m + 1)),
                                   dim3(kBlock), 0, s, (const RI *)rows, m, n,
                                   (int64_t *)h.row_ptr);
            else
                hipLaunchKernelGGL((k_rowptr_sorted<RI, int32_t>), dim3(grid_for(m + 1)),
                                   dim3(kBlock), 0, s, (const RI *)rows, m, n,
                                   (int32_t *)h.row_ptr);
        };
        dispatch_idx(rit, launch);
        SLA_HIP(hipGetLastError());
        if (m > 0) {
            if (cit == SLA_I32)
                SLA_HIP(hipMemcpyAsync(h.col, cols, (size_t)m * 4, hipMemcpyDeviceToDevice, s));
            else
                hipLaunchKernelGGL((k_convert<int64_t, int32_t>), dim3(grid_for(m)), dim3(kBlock),
                                   0, s, (const int64_t *)cols, m, h.col);
            SLA_HIP(hipGetLastError());
        }
    } else {
        // general input: stable radix sort of (row*n + col, input index)
        uint64_t *keys = sc.get<uint64_t>(m);
        h.perm = (int64_t *)dalloc(h, (size_t)m * 8);
        auto launch = [&](auto rtag, auto ctag) {
            using RI = std::remove_const_t<std::remove_pointer_t<decltype(rtag)>>;
            using CI = std::remove_const_t<std::remove_pointer_t<decltype(ctag)>>;
            hipLaunchKernelGGL((k_make_keys<RI, CI>), dim3(grid_for(m)), dim3(kBlock), 0, s,
                               (const RI *)rows, (const CI *)cols, m, n, keys, h.perm);
        };
        dispatch_idx(rit, [&](auto r) { dispatch_idx(cit, [&](auto c) { launch(r, c); }); });
        SLA_HIP(hipGetLastError());
        int bits = 0;
        while ((int64_t(1) << bits) < n) ++bits;
        radix_sort_pairs(keys, h.perm, m, 2 * bits, s);

        int64_t *head = sc.get<int64_t>(m);
        int64_t *excl = sc.get<int64_t>(m);
        hipLaunchKernelGGL(k_heads, dim3(grid_for(m)), dim3(kBlock), 0, s, (const uint64_t *)keys,
                           m, head);
        SLA_HIP(hipGetLastError());
        exclusive_scan_i64(head, excl, m, s);
        const int64_t nnz_u = read_i64(excl + (m - 1), s) + read_i64(head + (m - 1), s);
        h.nnz = nnz_u;
        h.rp64 = nnz_u >= (int64_t(1) << 31);
        h.col = (int32_t *)dalloc(h, (size_t)(nnz_u + kEntryPad) * 4);
        h.run = (int64_t *)dalloc(h, (size_t)(nnz_u + 1) * 8);
        h.slot = (int64_t *)dalloc(h, (size_t)m * 8);
        int64_t *urow = sc.get<int64_t>(nnz_u);
        hipLaunchKernelGGL(k_unique, dim3(grid_for(m)), dim3(kBlock), 0, s, (const uint64_t *)keys,
                           (const int64_t *)h.perm, (const int64_t *)excl, (const int64_t *)head,
                           m, n, h.col, urow, h.run, h.slot);
        SLA_HIP(hipGetLastError());
        SLA_HIP(hipMemcpyAsync(h.run + nnz_u, &m, 8, hipMemcpyHostToDevice, s));
        h.row_ptr = dalloc(h, (size_t)(n + 1) * (h.rp64 ? 8 : 4));
        if (h.rp64)
            hipLaunchKernelGGL((k_rowptr_sorted<int64_t, int64_t>), dim3(grid_for(nnz_u + 1)),
                               dim3(kBlock), 0, s, (const int64_t *)urow, nnz_u, n,
                               (int64_t *)h.row_ptr);
        else
            hipLaunchKernelGGL((k_rowptr_sorted<int64_t, int32_t>), dim3(grid_for(nnz_u + 1)),
                               dim3(kBlock), 0, s, (const int64_t *)urow, nnz_u, n,
                               (int32_t *)h.row_ptr);
        SLA_HIP(hipGetLastError());
        SLA_HIP(hipStreamSynchronize(s));  // host value m above must outlive the copy
    }
    h.vals = dalloc(h, (size_t)(h.nnz + kEntryPad) * h.B * h.vbytes);
    zero_padding(h, s);
    load_values(h, values, s);
}

// ------------------------------------------------------------------ CSR input

void build_from_csr(Handle &h, sla_itype rit, const void *row_ptr, sla_itype cit, const void *cols,
                    const void *values, hipStream_t s) {
    const int64_t n = h.n, nnz = h.nnz_in;
    Scratch sc(s);
    int *dflag = sc.get<int>(1);
    SLA_HIP(hipMemsetAsync(dflag, 0, sizeof(int), s));
    auto launch = [&](auto rtag, auto ctag) {
        using RI = std::remove_const_t<std::remove_pointer_t<decltype(rtag)>>;
        using CI = std::remove_const_t<std::remove_pointer_t<decltype(ctag)>>;
        hipLaunchKernelGGL((k_csr_check<RI, CI>), dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const RI *)row_ptr, (const CI *)cols, n, nnz, dflag);
    };
    dispatch_idx(rit, [&](auto r) { dispatch_idx(cit, [&](auto c) { launch(r, c); }); });
    SLA_HIP(hipGetLastError());
    const int flags = read_flag(dflag, s);
    if (flags & kBadCsr)
        fail(SLA_ERR_INVALID_CSR,
             "CSR input: row_ptr must run 0..nnz without decreasing and columns must be strictly "
             "increasing inside each row");
    if (flags & kBadIndex) fail(SLA_ERR_INDEX_RANGE, "a CSR column index is outside [0, n)");

    h.nnz = nnz;
    h.rp64 = (rit == SLA_I64);  // CSR input keeps its row-pointer width
    const size_t rp_bytes = (size_t)(n + 1) * (h.rp64 ? 8 : 4);
    h.row_ptr = dalloc(h, rp_bytes);
    SLA_HIP(hipMemcpyAsync(h.row_ptr, row_ptr, rp_bytes, hipMemcpyDeviceToDevice, s));
    h.col = (int32_t *)dalloc(h, (size_t)(nnz + kEntryPad) * 4);
    if (nnz > 0) {
        if (cit == SLA_I32)
            SLA_HIP(hipMemcpyAsync(h.col, cols, (size_t)nnz * 4, hipMemcpyDeviceToDevice, s));
        else
            hipLaunchKernelGGL((k_convert<int64_t, int32_t>), dim3(grid_for(nnz)), dim3(kBlock), 0,
                               s, (const int64_t *)cols, nnz, h.col);
        SLA_HIP(hipGetLastError());
    }
    h.vals = dalloc(h, (size_t)(nnz + kEntryPad) * h.B * h.vbytes);
    zero_padding(h, s);
    load_values(h, values, s);
}

// values [B][nnz_in] (input order) -> internal [nnz][B]
static void load_values_csr(Handle &h, const void *values, hipStream_t s) {
    if (h.nnz_in == 0) return;
    if (!h.perm) {
        if (h.B == 1)
            SLA_HIP(hipMemcpyAsync(h.vals, values, (size_t)h.nnz * h.vbytes,
                                   hipMemcpyDeviceToDevice, s));
        else
            transpose(values, h.vals, h.B, h.nnz, h.vbytes, s);
        return;
    }
    const unsigned g = grid_for(h.nnz * h.B);
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_merge<double>, dim3(g), dim3(kBlock), 0, s, (const double *)values,
                           (const int64_t *)h.perm, (const int64_t *)h.run, h.nnz, h.nnz_in, h.B,
                           (double *)h.vals);
    else
        hipLaunchKernelGGL(k_merge<float>, dim3(g), dim3(kBlock), 0, s, (const float *)values,
                           (const int64_t *)h.perm, (const int64_t *)h.run, h.nnz, h.nnz_in, h.B,
                           (float *)h.vals);
    SLA_HIP(hipGetLastError());
}

void load_values(Handle &h, const void *values, hipStream_t s) {
    load_values_csr(h, values, s);
    dia_scatter(h, s);
}

// ------------------------------------------------------------------ tiles

// One wavefront per tile: the tile's column range decides whether its
// columns fit 16 bits relative to the smallest one (narrow); narrow tiles get
// col16, every tile gets its row offsets relative to k0 in roff16.
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_tile_compress(TileDesc *__restrict__ tiles,
                                                          int64_t ntiles,
                                                          const RP *__restrict__ row_ptr,
                                                          const int32_t *__restrict__ col,
                                                          uint16_t *__restrict__ col16,
                                                          uint16_t *__restrict__ roff16,
                                                          int *__restrict__ wide) {
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= ntiles) return;  // whole wavefronts; no workgroup barrier below
    const int lane = threadIdx.x & 63;
    const TileDesc d = tiles[t];
    int32_t mn = INT32_MAX, mx = INT32_MIN;
    for (int64_t k = d.k0 + lane; k < d.k1; k += 64) {
        const int32_t c = col[k];
        mn = c < mn ? c : mn;
        mx = c > mx ? c : mx;
    }
    for (int off = 32; off > 0; off >>= 1) {
        const int32_t a = __shfl_xor(mn, off, 64), b = __shfl_xor(mx, off, 64);
        mn = a < mn ? a : mn;
        mx = b > mx ? b : mx;
    }
    const bool empty = d.k1 == d.k0;
    const bool narrow = empty || (int64_t)mx - (int64_t)mn < 65536;
    const int32_t cbase = empty ? 0 : mn;
    if (narrow)
        for (int64_t k = d.k0 + lane; k < d.k1; k += 64) col16[k] = (uint16_t)(col[k] - cbase);
    const int nr = d.re - d.rs;
    for (int j = lane; j <= nr; j += 64) roff16[d.rpos + j] = (uint16_t)(row_ptr[d.rs + j] - d.k0);
    if (lane == 0) {
        tiles[t].cbase = cbase;
        tiles[t].narrow = narrow ? 1 : 0;
        if (!narrow) atomicAdd(wide, 1);
    }
}

template <typename RP>
__global__ __launch_bounds__(kBlock) void k_gather_rp(const RP *__restrict__ row_ptr,
                                                      const int64_t *__restrict__ rows, int64_t m,
                                                      int64_t *__restrict__ out) {
    const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (j < m) out[j] = (int64_t)row_ptr[rows[j]];
}

// Band-aligned tiles for a large single stencil-like matrix: with band N
// (the farthest column right of most rows is row + N) and L tiles per N rows,
// tile j + L holds the rows of tile j moved by N, so the p values tile j
// gathers from rows near +N are the ones tile j + L owns and tile j + 2L
// gathers near -N. The SpMV walks tiles j, j + L, j + 2L, ... in one
// wavefront, one step apart, so those p lines are reused from the L2 whatever
// the pace of the other wavefronts (with the usual tiles the three uses fall
// to different wavefronts, which drift apart: at 133M rows each p line was
// fetched about three times). L = the SpMV's wavefronts per XCD divided by a
// panel count P, picked so that a tile has 36 to 64 rows (at most 63 rows and
// 253 entries for the ring form of the SpMV), nearest 45. On the 133M-row
// Poisson matrix: one-tile-ahead SpMV (768 wavefronts per XCD), 3 panels of
// 256 columns and 45-row tiles took it from 2.28 to 2.14 ms (HBM fetches
// 10.7 -> 8.4 GB), 30-row tiles were slower than the usual ones (2.69 ms),
// 60-row ones 2.22 ms; ring SpMV (512 wavefronts), 2 panels of 256 columns
// and 45-row tiles 2.05 ms against 2.40 with the usual tiles. Bands under
// 4096 rows keep the usual tiles: their p lines are reused by neighbouring
// wavefronts anyway.
void choose_band(Handle &h, hipStream_t s) {
    h.band_n = h.band_l = 0;
    h.band_p = 0;
    const int64_t n = h.n;
    if (h.B != 1 || n < ((int64_t)1 << 20) || h.nnz == 0) return;
    Scratch sc(s);
    unsigned long long *match = sc.get<unsigned long long>(1);
    int *maxlen = sc.get<int>(1);
    SLA_HIP(hipMemsetAsync(match, 0, sizeof(unsigned long long), s));
    SLA_HIP(hipMemsetAsync(maxlen, 0, sizeof(int), s));
    // the candidate: the middle row's farthest offset
    int64_t mid[2] = {0, 0};
    int32_t last = 0;
    if (h.rp64) {
        SLA_HIP(hipMemcpyAsync(mid, (const int64_t *)h.row_ptr + n / 2, 16, hipMemcpyDeviceToHost, s));
    } else {
        int32_t m32[2];
        SLA_HIP(hipMemcpyAsync(m32, (const int32_t *)h.row_ptr + n / 2, 8, hipMemcpyDeviceToHost, s));
        SLA_HIP(hipStreamSynchronize(s));
        mid[0] = m32[0];
        mid[1] = m32[1];
    }
    SLA_HIP(hipStreamSynchronize(s));
    if (mid[1] <= mid[0]) return;
    SLA_HIP(hipMemcpyAsync(&last, h.col + mid[1] - 1, 4, hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    const int64_t band = (int64_t)last - n / 2;
    if (band < 2) return;
    if (h.rp64)
        hipLaunchKernelGGL(k_band_count<int64_t>, dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const int64_t *)h.row_ptr, (const int32_t *)h.col, n, band, match, maxlen);
    else
        hipLaunchKernelGGL(k_band_count<int32_t>, dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const int32_t *)h.row_ptr, (const int32_t *)h.col, n, band, match, maxlen);
    SLA_HIP(hipGetLastError());
    unsigned long long hm = 0;
    int hl = 0;
    SLA_HIP(hipMemcpyAsync(&hm, match, sizeof(hm), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipMemcpyAsync(&hl, maxlen, sizeof(hl), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    if ((double)hm < 0.9 * (double)n || hl < 1 || hl > kLongRow || band < 4096 || n < 8 * band)
        return;
    // wavefronts per XCD of the SpMV (its grid is the resident count when the
    // tiles outnumber it, as they do here)
    const int64_t W = tile_spmv_waves_per_xcd(h, h.spmv_ring);
    // tiles the ring form of the SpMV takes: at most 63 rows and 253 entries
    const int64_t max_rows = h.spmv_ring ? std::min<int64_t>(63, 253 / hl)
                                         : std::min<int64_t>(64, kTileCap / hl);
    int64_t best_p = 0;
    double best_err = 1e300;
    for (int64_t P = 1; P <= 16; ++P) {
        if (W % P) continue;
        const int64_t L = W / P;
        const double rows = (double)band / (double)L;
        if (rows < 36.0 || std::ceil(rows) > (double)max_rows) continue;
        const double err = std::fabs(rows - 45.0);
        if (err < best_err) {
            best_err = err;
            best_p = P;
        }
    }
    if (best_p == 0) return;
    h.band_n = band;
    h.band_p = (int32_t)best_p;
    h.band_l = W / best_p;
}

void build_tiles(Handle &h, hipStream_t s, const int64_t *seg_rows, int32_t nseg) {
    const int64_t n = h.n;
    if (nseg == 0) choose_band(h, s);
    else h.band_n = h.band_l = h.band_p = 0;
    Scratch sc(s);
    int64_t *flag = sc.get<int64_t>(n);
    int64_t *excl = sc.get<int64_t>(n);
    if (h.rp64)
        hipLaunchKernelGGL(k_tile_flags<int64_t>, dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const int64_t *)h.row_ptr, n, h.band_n, h.band_l, flag);
    else
        hipLaunchKernelGGL(k_tile_flags<int32_t>, dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const int32_t *)h.row_ptr, n, h.band_n, h.band_l, flag);
    SLA_HIP(hipGetLastError());
    exclusive_scan_i64(flag, excl, n, s);
    const int64_t nt = read_i64(excl + (n - 1), s) + read_i64(flag + (n - 1), s);
    int32_t *tstart = sc.get<int32_t>(nt + 1);
    int64_t *tk0 = sc.get<int64_t>(nt + 1);
    hipLaunchKernelGGL(k_tile_fill, dim3(grid_for(n)), dim3(kBlock), 0, s, (const int64_t *)flag,
                       (const int64_t *)excl, n, tstart);
    SLA_HIP(hipGetLastError());
    const int32_t nn = (int32_t)n;
    SLA_HIP(hipMemcpyAsync(tstart + nt, &nn, 4, hipMemcpyHostToDevice, s));
    if (h.rp64)
        hipLaunchKernelGGL(k_tile_k0<int64_t>, dim3(grid_for(nt + 1)), dim3(kBlock), 0, s,
                           (const int64_t *)h.row_ptr, (const int32_t *)tstart, nt, tk0);
    else
        hipLaunchKernelGGL(k_tile_k0<int32_t>, dim3(grid_for(nt + 1)), dim3(kBlock), 0, s,
                           (const int32_t *)h.row_ptr, (const int32_t *)tstart, nt, tk0);
    SLA_HIP(hipGetLastError());
    // split on the host: a one-row tile longer than kLongRow goes to the long-row list
    std::vector<int32_t> hs((size_t)nt + 1);
    std::vector<int64_t> hk((size_t)nt + 1);
    SLA_HIP(hipMemcpyAsync(hs.data(), tstart, (size_t)(nt + 1) * 4, hipMemcpyDeviceToHost, s));
    SLA_HIP(hipMemcpyAsync(hk.data(), tk0, (size_t)(nt + 1) * 8, hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    // row_ptr at the member boundaries (segmented handles)
    std::vector<int64_t> bk((size_t)(nseg > 0 ? nseg + 1 : 0));
    if (nseg > 0) {
        int64_t *drows = sc.get<int64_t>(nseg + 1);
        int64_t *dk = sc.get<int64_t>(nseg + 1);
        SLA_HIP(hipMemcpyAsync(drows, seg_rows, 8 * (size_t)(nseg + 1), hipMemcpyHostToDevice, s));
        const unsigned gg = (unsigned)((nseg + 1 + kBlock - 1) / kBlock);
        if (h.rp64)
            hipLaunchKernelGGL(k_gather_rp<int64_t>, dim3(gg), dim3(kBlock), 0, s,
                               (const int64_t *)h.row_ptr, drows, (int64_t)nseg + 1, dk);
        else
            hipLaunchKernelGGL(k_gather_rp<int32_t>, dim3(gg), dim3(kBlock), 0, s,
                               (const int32_t *)h.row_ptr, drows, (int64_t)nseg + 1, dk);
        SLA_HIP(hipGetLastError());
        SLA_HIP(hipMemcpyAsync(bk.data(), dk, 8 * (size_t)(nseg + 1), hipMemcpyDeviceToHost, s));
    }
    SLA_HIP(hipStreamSynchronize(s));
    std::vector<TileDesc> shorts;
    std::vector<int32_t> longs;
    shorts.reserve((size_t)nt);
    int64_t rpos = 0;
    auto add = [&](const TileDesc &e) {
        TileDesc d = e;
        if (d.re - d.rs == 1 && d.k1 - d.k0 > kLongRow) {
            longs.push_back(d.rs);
        } else {
            d.rpos = rpos;
            rpos += d.re - d.rs + 1;
            shorts.push_back(d);
        }
    };
    int32_t nb = 1;  // next member boundary to look at
    for (int64_t t = 0; t < nt; ++t) {
        TileDesc d{hs[t], hs[t + 1], hk[t], hk[t + 1], 0, 0, 0};
        // a tile that spans member boundaries becomes one piece per member
        while (nb < nseg && seg_rows[nb] <= d.rs) ++nb;
        while (nb < nseg && seg_rows[nb] < d.re) {
            const int32_t b = (int32_t)seg_rows[nb];
            add(TileDesc{d.rs, b, d.k0, bk[(size_t)nb], 0, 0, 0});
            d.rs = b;
            d.k0 = bk[(size_t)nb];
            ++nb;
        }
        add(d);
    }
    h.ntiles = (int64_t)shorts.size();
    h.nlong = (int64_t)longs.size();
    if (nseg > 0) {
        // each member's first tile and first long row (both lists in row order)
        std::vector<int64_t> t0((size_t)nseg + 1), l0((size_t)nseg + 1);
        size_t it = 0, il = 0;
        for (int32_t q = 0; q <= nseg; ++q) {
            const int64_t r = seg_rows[q];
            while (it < shorts.size() && shorts[it].rs < r) ++it;
            while (il < longs.size() && longs[il] < r) ++il;
            t0[(size_t)q] = (int64_t)it;
            l0[(size_t)q] = (int64_t)il;
        }
        h.seg_tile0 = (int64_t *)dalloc(h, 8 * ((size_t)nseg + 1));
        h.seg_long0 = (int64_t *)dalloc(h, 8 * ((size_t)nseg + 1));
        // (+4: the SpMV reads the flags as 32-bit words)
        h.tile_live = (uint8_t *)dalloc(h, shorts.size() + 4);
        h.tile_dot = (double *)dalloc(h, sizeof(double) * (shorts.size() + 1));
        SLA_HIP(hipMemcpyAsync(h.seg_tile0, t0.data(), 8 * ((size_t)nseg + 1), hipMemcpyHostToDevice,
                               s));
        SLA_HIP(hipMemcpyAsync(h.seg_long0, l0.data(), 8 * ((size_t)nseg + 1), hipMemcpyHostToDevice,
                               s));
        SLA_HIP(hipMemsetAsync(h.tile_live, 1, shorts.size() + 1, s));
        SLA_HIP(hipStreamSynchronize(s));
    }
    h.tiles = (TileDesc *)dalloc(h, sizeof(TileDesc) * (shorts.size() + 1));
    h.long_rows = (int32_t *)dalloc(h, sizeof(int32_t) * (longs.size() + 1));
    h.long_dot = (double *)dalloc(h, sizeof(double) * 2 * (longs.size() + 1));  // two dots
    if (!shorts.empty())
        SLA_HIP(hipMemcpyAsync(h.tiles, shorts.data(), sizeof(TileDesc) * shorts.size(),
                               hipMemcpyHostToDevice, s));
    if (!longs.empty())
        SLA_HIP(hipMemcpyAsync(h.long_rows, longs.data(), sizeof(int32_t) * longs.size(),
                               hipMemcpyHostToDevice, s));
    // 16-bit index forms for the single-system SpMV
    h.col16 = (uint16_t *)dalloc(h, sizeof(uint16_t) * (size_t)(h.nnz + kEntryPad));
    h.roff16 = (uint16_t *)dalloc(h, sizeof(uint16_t) * (size_t)(rpos + kEntryPad));
    SLA_HIP(hipMemsetAsync(h.col16, 0, sizeof(uint16_t) * (size_t)(h.nnz + kEntryPad), s));
    SLA_HIP(hipMemsetAsync(h.roff16, 0, sizeof(uint16_t) * (size_t)(rpos + kEntryPad), s));
    h.all_narrow = false;
    if (h.ntiles > 0) {
        int *wide = sc.get<int>(1);
        SLA_HIP(hipMemsetAsync(wide, 0, sizeof(int), s));
        const unsigned g = (unsigned)((h.ntiles + kWaves - 1) / kWaves);
        if (h.rp64)
            hipLaunchKernelGGL(k_tile_compress<int64_t>, dim3(g), dim3(kBlock), 0, s, h.tiles,
                               h.ntiles, (const int64_t *)h.row_ptr, (const int32_t *)h.col,
                               h.col16, h.roff16, wide);
        else
            hipLaunchKernelGGL(k_tile_compress<int32_t>, dim3(g), dim3(kBlock), 0, s, h.tiles,
                               h.ntiles, (const int32_t *)h.row_ptr, (const int32_t *)h.col,
                               h.col16, h.roff16, wide);
        SLA_HIP(hipGetLastError());
        h.wide_tiles = read_flag(wide, s);
        h.all_narrow = h.wide_tiles == 0;
    }
    // the ring form of the SpMV: every tile's entries from k0 rounded down to
    // a multiple of 4 fit one 4-entry group per lane, its row offsets one per lane
    h.ring_tiles = h.all_narrow;
    for (const TileDesc &d : shorts)
        if (d.k1 - (d.k0 & ~(int64_t)3) > 4 * 64 || d.re - d.rs > 63) {
            h.ring_tiles = false;
            break;
        }
    SLA_HIP(hipStreamSynchronize(s));
    if (nseg == 0) build_dia(h, s);
}

// ------------------------------------------------------------------ Jacobi

void compute_dinv(Handle &h, hipStream_t s) {
    Scratch sc(s);
    int *bad = sc.get<int>(1);
    SLA_HIP(hipMemsetAsync(bad, 0, sizeof(int), s));
    const unsigned g = grid_for(h.n * h.B);
    auto go = [&](auto ttag, auto rtag) {
        using T = decltype(ttag);
        using RP = decltype(rtag);
        hipLaunchKernelGGL((k_dinv<T, RP>), dim3(g), dim3(kBlock), 0, s, (const RP *)h.row_ptr,
                           (const int32_t *)h.col, (const T *)h.vals, h.n, h.B, (T *)h.dinv, bad);
    };
    if (h.vt == SLA_F64) {
        if (h.rp64) go(double(), int64_t());
        else go(double(), int32_t());
    } else {
        if (h.rp64) go(float(), int64_t());
        else go(float(), int32_t());
    }
    SLA_HIP(hipGetLastError());
    const int flags = read_flag(bad, s);
    h.diag_ok = flags == 0;
    h.diag_nonzero = (flags & kDiagUnusable) == 0;
}

// ---- a single system held by diagonals
struct DiaOffs {
    int32_t o[kDiaMax];
    int32_t m;
};

// flag = 1 if an entry's offset j - i is not one of the m candidates
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_dia_check(const RP *__restrict__ row_ptr,
                                                      const int32_t *__restrict__ col, int64_t n,
                                                      DiaOffs d, int *__restrict__ flag) {
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        for (int64_t k = row_ptr[i]; k < (int64_t)row_ptr[i + 1]; ++k) {
            const int64_t o = (int64_t)col[k] - i;
            bool hit = false;
            for (int q = 0; q < d.m; ++q) hit |= o == (int64_t)d.o[q];
            bad |= hit ? 0 : 1;
        }
    if (bad) atomicOr(flag, 1);
}

// map[k] = q n + i for entry k = (i, i + o_q)
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_dia_map(const RP *__restrict__ row_ptr,
                                                    const int32_t *__restrict__ col, int64_t n,
                                                    DiaOffs d, int32_t *__restrict__ map) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        for (int64_t k = row_ptr[i]; k < (int64_t)row_ptr[i + 1]; ++k) {
            const int64_t o = (int64_t)col[k] - i;
            int q = 0;
            while (q < d.m - 1 && (int64_t)d.o[q] != o) ++q;
            map[k] = (int32_t)dia_slot(q, i, d.m);
        }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_dia_scatter(const T *__restrict__ vals,
                                                        const int32_t *__restrict__ map,
                                                        int64_t nnz, T *__restrict__ out) {
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz;
         k += (int64_t)gridDim.x * kBlock)
        out[map[k]] = vals[k];
}

// key = length << 40 | (2^40 - 1 - row), maximised: the first longest row
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_longest_row(const RP *__restrict__ row_ptr, int64_t n,
                                                        unsigned long long *__restrict__ key) {
    unsigned long long best = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const unsigned long long len = (unsigned long long)(row_ptr[i + 1] - row_ptr[i]);
        const unsigned long long k = (len << 40) | ((1ull << 40) - 1 - (unsigned long long)i);
        best = k > best ? k : best;
    }
    if (best) atomicMax(key, best);
}

// A single system whose entries lie on 5 or 7 distinct offsets j - i (the
// 2D and 3D stencils), with m n at most a quarter above nnz, is also held by
// diagonals: the candidates are the offsets of a longest row, checked
// against every entry on the device; offsets ascending, so a row's
// diagonals run in its column order.
void build_dia(Handle &h, hipStream_t s) {
    h.dia_m = 0;
    const int64_t n = h.n;
    if (h.B != 1 || h.nseg > 0 || n < 2 || h.nnz < 1) return;
    // the candidate row: the first of the longest rows (found on the device)
    Scratch sc0(s);
    unsigned long long *key = sc0.get<unsigned long long>(1);
    SLA_HIP(hipMemsetAsync(key, 0, sizeof(unsigned long long), s));
    if (h.rp64)
        hipLaunchKernelGGL(k_longest_row<int64_t>, dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const int64_t *)h.row_ptr, n, key);
    else
        hipLaunchKernelGGL(k_longest_row<int32_t>, dim3(grid_for(n)), dim3(kBlock), 0, s,
                           (const int32_t *)h.row_ptr, n, key);
    SLA_HIP(hipGetLastError());
    unsigned long long hkey = 0;
    SLA_HIP(hipMemcpyAsync(&hkey, key, sizeof(hkey), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    const int64_t crow = (int64_t)((1ull << 40) - 1 - (hkey & ((1ull << 40) - 1)));
    int64_t mid[2] = {0, 0};
    if (h.rp64) {
        SLA_HIP(hipMemcpyAsync(mid, (const int64_t *)h.row_ptr + crow, 16, hipMemcpyDeviceToHost, s));
    } else {
        int32_t m32[2] = {0, 0};
        SLA_HIP(hipMemcpyAsync(m32, (const int32_t *)h.row_ptr + crow, 8, hipMemcpyDeviceToHost, s));
        SLA_HIP(hipStreamSynchronize(s));
        mid[0] = m32[0];
        mid[1] = m32[1];
    }
    SLA_HIP(hipStreamSynchronize(s));
    const int64_t m = mid[1] - mid[0];
    if (m != 5 && m != 7) return;
    if ((double)m * (double)n > 1.25 * (double)h.nnz || dia_slots(n, (int)m) >= (int64_t)INT32_MAX) return;
    int32_t cols[kDiaMax];
    SLA_HIP(hipMemcpyAsync(cols, h.col + mid[0], sizeof(int32_t) * (size_t)m, hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    DiaOffs d{};
    d.m = (int32_t)m;
    for (int q = 0; q < m; ++q) d.o[q] = (int32_t)(cols[q] - crow);   // ascending (sorted row)
    Scratch sc(s);
    int *flag = sc.get<int>(1);
    SLA_HIP(hipMemsetAsync(flag, 0, sizeof(int), s));
    const unsigned g = grid_for(n);
    if (h.rp64)
        hipLaunchKernelGGL(k_dia_check<int64_t>, dim3(g), dim3(kBlock), 0, s,
                           (const int64_t *)h.row_ptr, (const int32_t *)h.col, n, d, flag);
    else
        hipLaunchKernelGGL(k_dia_check<int32_t>, dim3(g), dim3(kBlock), 0, s,
                           (const int32_t *)h.row_ptr, (const int32_t *)h.col, n, d, flag);
    SLA_HIP(hipGetLastError());
    if (read_flag(flag, s) != 0) return;
    h.dia_off = (int32_t *)dalloc(h, sizeof(int32_t) * kDiaMax);
    h.dia_map = (int32_t *)dalloc(h, sizeof(int32_t) * (size_t)h.nnz);
    h.dia_val = dalloc(h, (size_t)dia_slots(n, (int)m) * h.vbytes);
    SLA_HIP(hipMemcpyAsync(h.dia_off, d.o, sizeof(int32_t) * kDiaMax, hipMemcpyHostToDevice, s));
    SLA_HIP(hipMemsetAsync(h.dia_val, 0, (size_t)dia_slots(n, (int)m) * h.vbytes, s));
    if (h.rp64)
        hipLaunchKernelGGL(k_dia_map<int64_t>, dim3(g), dim3(kBlock), 0, s,
                           (const int64_t *)h.row_ptr, (const int32_t *)h.col, n, d, h.dia_map);
    else
        hipLaunchKernelGGL(k_dia_map<int32_t>, dim3(g), dim3(kBlock), 0, s,
                           (const int32_t *)h.row_ptr, (const int32_t *)h.col, n, d, h.dia_map);
    SLA_HIP(hipGetLastError());
    h.dia_m = (int32_t)m;
    dia_scatter(h, s);
    SLA_HIP(hipStreamSynchronize(s));
}

void dia_scatter(Handle &h, hipStream_t s) {
    if (h.dia_m == 0 || h.nnz == 0) return;
    const unsigned g = grid_for(h.nnz);
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_dia_scatter<double>, dim3(g), dim3(kBlock), 0, s,
                           (const double *)h.vals, (const int32_t *)h.dia_map, h.nnz,
                           (double *)h.dia_val);
    else
        hipLaunchKernelGGL(k_dia_scatter<float>, dim3(g), dim3(kBlock), 0, s,
                           (const float *)h.vals, (const int32_t *)h.dia_map, h.nnz,
                           (float *)h.dia_val);
    SLA_HIP(hipGetLastError());
}

bool check_symmetric(Handle &h, hipStream_t s) {
    Scratch sc(s);
    int *flag = sc.get<int>(1);
    SLA_HIP(hipMemsetAsync(flag, 0, sizeof(int), s));
    const unsigned g = grid_for(h.n);
    auto go = [&](auto ttag, auto rtag) {
        using T = decltype(ttag);
        using RP = decltype(rtag);
        hipLaunchKernelGGL((k_symmetric<T, RP>), dim3(g), dim3(kBlock), 0, s,
                           (const RP *)h.row_ptr, (const int32_t *)h.col, (const T *)h.vals, h.n,
                           h.B, flag);
    };
    if (h.vt == SLA_F64) {
        if (h.rp64) go(double(), int64_t());
        else go(double(), int32_t());
    } else {
        if (h.rp64) go(float(), int64_t());
        else go(float(), int32_t());
    }
    SLA_HIP(hipGetLastError());
    return read_flag(flag, s) == 0;
}

void gather_to_input(Handle &h, const void *in, void *out, hipStream_t s) {
    if (h.nnz_in == 0) return;
    if (!h.slot) {
        SLA_HIP(hipMemcpyAsync(out, in, (size_t)h.nnz * h.B * h.vbytes, hipMemcpyDeviceToDevice, s));
        return;
    }
    const unsigned g = grid_for(h.nnz_in * h.B);
    if (h.vt == SLA_F64)
        hipLaunchKernelGGL(k_gather<double>, dim3(g), dim3(kBlock), 0, s, (const double *)in,
                           (const int64_t *)h.slot, h.nnz, h.nnz_in, h.B, (double *)out);
    else
        hipLaunchKernelGGL(k_gather<float>, dim3(g), dim3(kBlock), 0, s, (const float *)in,
                           (const int64_t *)h.slot, h.nnz, h.nnz_in, h.B, (float *)out);
    SLA_HIP(hipGetLastError());
}

void values_to_batch_major(Handle &h, void *out, hipStream_t s) {
    if (h.nnz == 0) return;
    if (h.B == 1)
        SLA_HIP(hipMemcpyAsync(out, h.vals, (size_t)h.nnz * h.vbytes, hipMemcpyDeviceToDevice, s));
    else
        transpose(h.vals, out, h.nnz, h.B, h.vbytes, s);
}

}  // namespace sla

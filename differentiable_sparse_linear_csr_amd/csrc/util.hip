// Integer scan, stable LSD radix sort of (key, index) pairs, and tiled
// transposes — the building blocks of CSR assembly. All are deterministic.
#include "common.h"

namespace sla {

namespace {

constexpr int kScanItems = 8;
constexpr int kScanTile = kBlock * kScanItems;  // 2048

// Inclusive scan across the block of one value per thread; returns the
// exclusive prefix and writes the block total to *total.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *lds_w, int64_t *total) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int64_t inc = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    if (lane == 63) lds_w[w] = inc;
    __syncthreads();
    int64_t wpre = 0;
    for (int k = 0; k < w; ++k) wpre += lds_w[k];
    *total = lds_w[0] + lds_w[1] + lds_w[2] + lds_w[3];
    __syncthreads();
    return wpre + inc - v;
}

__global__ __launch_bounds__(kBlock) void k_scan_sums(const int64_t *__restrict__ in, int64_t m,
                                                      int64_t *__restrict__ sums) {
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int64_t s = 0;
    for (int j = 0; j < kScanItems; ++j) {
        const int64_t e = base + (int64_t)j * kBlock + threadIdx.x;
        if (e < m) s += in[e];
    }
    // integer block sum via the shuffle tree (exact)
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ int64_t ws[kWaves];
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sums[blockIdx.x] = ws[0] + ws[1] + ws[2] + ws[3];
}

// exclusive scan of one tile plus the tile's offset (in == out allowed: a
// block reads its whole tile before writing it)
__global__ __launch_bounds__(kBlock) void k_scan_tile(const int64_t *in, int64_t m,
                                                      const int64_t *offs, int64_t *out) {
    __shared__ int64_t tile[kScanTile];
    __shared__ int64_t lds_w[kWaves];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    for (int j = 0; j < kScanItems; ++j) {
        const int64_t e = base + (int64_t)j * kBlock + threadIdx.x;
        tile[j * kBlock + threadIdx.x] = e < m ? in[e] : 0;
    }
    __syncthreads();
    // each thread owns kScanItems consecutive items
    int64_t loc[kScanItems];
    int64_t s = 0;
    for (int j = 0; j < kScanItems; ++j) {
        loc[j] = tile[threadIdx.x * kScanItems + j];
        s += loc[j];
    }
    int64_t total;
    int64_t pre = block_exclusive_scan(s, lds_w, &total);
    pre += offs ? offs[blockIdx.x] : 0;
    for (int j = 0; j < kScanItems; ++j) {
        tile[threadIdx.x * kScanItems + j] = pre;
        pre += loc[j];
    }
    __syncthreads();
    for (int j = 0; j < kScanItems; ++j) {
        const int64_t e = base + (int64_t)j * kBlock + threadIdx.x;
        if (e < m) out[e] = tile[j * kBlock + threadIdx.x];
    }
}

// ------------------------------------------------------------------ radix sort
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortItems = 16;
constexpr int kSortTile = kBlock * kSortItems;  // 4096 keys per block

__global__ __launch_bounds__(kBlock) void k_radix_hist(const uint64_t *__restrict__ keys, int64_t m,
                                                       int shift, int64_t nblk,
                                                       int64_t *__restrict__ hist) {
    __shared__ int32_t cnt[kRadix];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    for (int j = 0; j < kSortItems; ++j) {
        const int64_t e = base + (int64_t)j * kBlock + threadIdx.x;
        if (e < m) atomicAdd(&cnt[(keys[e] >> shift) & (kRadix - 1)], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter: keys are visited in tile order (round j, then wave, then
// lane); equal digits keep that order. Ranks inside a wave come from ballot
// matching of the 8 digit bits.
__global__ __launch_bounds__(kBlock) void k_radix_scatter(
    const uint64_t *__restrict__ kin, const int64_t *__restrict__ vin, int64_t m, int shift,
    int64_t nblk, const int64_t *__restrict__ offs, uint64_t *__restrict__ kout,
    int64_t *__restrict__ vout) {
    __shared__ int64_t base[kRadix];
    __shared__ int32_t wcnt[kWaves][kRadix];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    base[t] = offs[(int64_t)t * nblk + blockIdx.x];
    for (int k = 0; k < kWaves; ++k) wcnt[k][t] = 0;
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    const int64_t tile0 = (int64_t)blockIdx.x * kSortTile;
    for (int j = 0; j < kSortItems; ++j) {
        const int64_t e = tile0 + (int64_t)j * kBlock + t;
        const bool valid = e < m;
        const uint64_t key = valid ? kin[e] : 0ull;
        const int64_t val = valid ? vin[e] : 0;
        const int d = (int)((key >> shift) & (kRadix - 1));
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < kRadixBits; ++bit) {
            const bool on = (d >> bit) & 1;
            const uint64_t bb = __ballot(valid && on);
            peers &= on ? bb : ~bb;
        }
        const int lrank = __popcll(peers & lt_mask);
        if (valid && lrank == 0) wcnt[w][d] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int64_t pos = base[d] + lrank;
            for (int k = 0; k < w; ++k) pos += wcnt[k][d];
            kout[pos] = key;
            vout[pos] = val;
        }
        __syncthreads();
        base[t] += (int64_t)wcnt[0][t] + wcnt[1][t] + wcnt[2][t] + wcnt[3][t];
        for (int k = 0; k < kWaves; ++k) wcnt[k][t] = 0;
        __syncthreads();
    }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_transpose(const T *__restrict__ in, T *__restrict__ out,
                                                      int64_t rows, int64_t cols, int64_t ntc) {
    // 64x64 tile through LDS; out[c][r] = in[r][c]; flat grid over (row tile, col tile)
    __shared__ T tile[64][65];
    const int64_t bt = blockIdx.x;
    const int64_t r0 = (bt / ntc) * 64, c0 = (bt % ntc) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int k = ty; k < 64; k += kWaves) {
        const int64_t r = r0 + k, c = c0 + tx;
        if (r < rows && c < cols) tile[k][tx] = in[r * cols + c];
    }
    __syncthreads();
    for (int k = ty; k < 64; k += kWaves) {
        const int64_t c = c0 + k, r = r0 + tx;
        if (r < rows && c < cols) out[c * rows + r] = tile[tx][k];
    }
}

__global__ __launch_bounds__(kBlock) void k_iota(int64_t *__restrict__ out, int64_t m) {
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < m;
         e += (int64_t)gridDim.x * kBlock)
        out[e] = e;
}

}  // namespace

void iota_i64(int64_t *out, int64_t m, hipStream_t s) {
    if (m <= 0) return;
    int64_t g = (m + kBlock - 1) / kBlock;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(k_iota, dim3((unsigned)g), dim3(kBlock), 0, s, out, m);
    SLA_HIP(hipGetLastError());
}

void exclusive_scan_i64(const int64_t *in, int64_t *out, int64_t m, hipStream_t s) {
    if (m <= 0) return;
    const int64_t nblk = (m + kScanTile - 1) / kScanTile;
    if (nblk == 1) {
        hipLaunchKernelGGL(k_scan_tile, dim3(1), dim3(kBlock), 0, s, in, m, nullptr, out);
        SLA_HIP(hipGetLastError());
        return;
    }
    int64_t *sums = nullptr;
    SLA_HIP(hipMallocAsync((void **)&sums, (size_t)nblk * sizeof(int64_t) * 2, s));
    int64_t *offs = sums + nblk;
    hipLaunchKernelGGL(k_scan_sums, dim3((unsigned)nblk), dim3(kBlock), 0, s, in, m, sums);
    SLA_HIP(hipGetLastError());
    exclusive_scan_i64(sums, offs, nblk, s);
    hipLaunchKernelGGL(k_scan_tile, dim3((unsigned)nblk), dim3(kBlock), 0, s, in, m,
                       (const int64_t *)offs, out);
    SLA_HIP(hipGetLastError());
    SLA_HIP(hipFreeAsync(sums, s));
}

void radix_sort_pairs(uint64_t *keys, int64_t *vals, int64_t m, int key_bits, hipStream_t s) {
    if (m <= 1 || key_bits <= 0) return;
    const int64_t nblk = (m + kSortTile - 1) / kSortTile;
    uint64_t *k2 = nullptr;
    int64_t *v2 = nullptr, *hist = nullptr;
    SLA_HIP(hipMallocAsync((void **)&k2, (size_t)m * sizeof(uint64_t), s));
    SLA_HIP(hipMallocAsync((void **)&v2, (size_t)m * sizeof(int64_t), s));
    SLA_HIP(hipMallocAsync((void **)&hist, (size_t)nblk * kRadix * sizeof(int64_t), s));
    uint64_t *ka = keys, *kb = k2;
    int64_t *va = vals, *vb = v2;
    const int passes = (key_bits + kRadixBits - 1) / kRadixBits;
    for (int pidx = 0; pidx < passes; ++pidx) {
        const int shift = pidx * kRadixBits;
        hipLaunchKernelGGL(k_radix_hist, dim3((unsigned)nblk), dim3(kBlock), 0, s,
                           (const uint64_t *)ka, m, shift, nblk, hist);
        SLA_HIP(hipGetLastError());
        exclusive_scan_i64(hist, hist, nblk * kRadix, s);
        hipLaunchKernelGGL(k_radix_scatter, dim3((unsigned)nblk), dim3(kBlock), 0, s,
                           (const uint64_t *)ka, (const int64_t *)va, m, shift, nblk,
                           (const int64_t *)hist, kb, vb);
        SLA_HIP(hipGetLastError());
        std::swap(ka, kb);
        std::swap(va, vb);
    }
    if (ka != keys) {
        SLA_HIP(hipMemcpyAsync(keys, ka, (size_t)m * sizeof(uint64_t), hipMemcpyDeviceToDevice, s));
        SLA_HIP(hipMemcpyAsync(vals, va, (size_t)m * sizeof(int64_t), hipMemcpyDeviceToDevice, s));
    }
    SLA_HIP(hipFreeAsync(k2, s));
    SLA_HIP(hipFreeAsync(v2, s));
    SLA_HIP(hipFreeAsync(hist, s));
}

void transpose(const void *in, void *out, int64_t rows, int64_t cols, int vbytes, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return;
    const int64_t ntc = (cols + 63) / 64, ntr = (rows + 63) / 64;
    const dim3 grid((unsigned)(ntc * ntr));
    if (vbytes == 8)
        hipLaunchKernelGGL(k_transpose<double>, grid, dim3(kBlock), 0, s, (const double *)in,
                           (double *)out, rows, cols, ntc);
    else if (vbytes == 4)
        hipLaunchKernelGGL(k_transpose<float>, grid, dim3(kBlock), 0, s, (const float *)in,
                           (float *)out, rows, cols, ntc);
    else
        fail(SLA_ERR_INVALID_ARG, "transpose: element size");
    SLA_HIP(hipGetLastError());
}

}  // namespace sla

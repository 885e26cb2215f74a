/*
 * The C ABI used from plain C: a 2D five-point Poisson matrix (N x N
 * interior nodes, Dirichlet) given as CSR with int32 indices in device
 * memory the caller owns, then create, PCG solve, matvec, adjoint backward,
 * BiCGStab on a non-symmetric variant, and one refused call.
 *
 * Usage: abi_solve N out.bin  -- writes the PCG solution x (N*N doubles) to
 * out.bin and prints one line of results; exit status 0 when every check
 * holds.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sla.h"

#define CHECK_HIP(e)                                                          \
    do {                                                                      \
        hipError_t err_ = (e);                                                \
        if (err_ != hipSuccess) {                                             \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)err_, __FILE__, __LINE__); \
            return 2;                                                         \
        }                                                                     \
    } while (0)
#define CHECK_SLA(e)                                                          \
    do {                                                                      \
        sla_status st_ = (e);                                                 \
        if (st_ != SLA_OK) {                                                  \
            fprintf(stderr, "sla error %d (%s) at line %d\n", (int)st_, sla_last_error(), __LINE__); \
            return 3;                                                         \
        }                                                                     \
    } while (0)

static double norm(const double *v, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += v[i] * v[i];
    return sqrt(s);
}

int main(int argc, char **argv) {
    if (argc < 3) {
        fprintf(stderr, "usage: %s N out.bin\n", argv[0]);
        return 1;
    }
    const int N = atoi(argv[1]);
    const int64_t n = (int64_t)N * N;
    /* CSR of the unit five-point Laplacian, columns increasing in each row;
       conv adds a first-order upwind term in x (non-symmetric) */
    int32_t *rp = malloc(sizeof(int32_t) * (n + 1));
    int32_t *col = malloc(sizeof(int32_t) * 5 * n);
    double *val = malloc(sizeof(double) * 5 * n), *conv = malloc(sizeof(double) * 5 * n);
    double *b = malloc(sizeof(double) * n), *x = malloc(sizeof(double) * n);
    double *y = malloc(sizeof(double) * n);
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t yy = i / N, xx = i % N;
        rp[i] = (int32_t)k;
        const int64_t nb[5] = {i - N, i - 1, i, i + 1, i + N};
        const int ok[5] = {yy > 0, xx > 0, 1, xx < N - 1, yy < N - 1};
        for (int j = 0; j < 5; ++j) {
            if (!ok[j]) continue;
            col[k] = (int32_t)nb[j];
            val[k] = j == 2 ? 4.0 : -1.0;
            conv[k] = j == 2 ? 5.0 : (j == 1 ? -2.0 : -1.0);
            ++k;
        }
        b[i] = sin(0.1 * (double)i) + 0.5;
    }
    rp[n] = (int32_t)k;
    const int64_t nnz = k;

    void *d_rp, *d_col, *d_val, *d_conv, *d_b, *d_x, *d_y, *d_gb, *d_gv;
    CHECK_HIP(hipMalloc(&d_rp, sizeof(int32_t) * (n + 1)));
    CHECK_HIP(hipMalloc(&d_col, sizeof(int32_t) * nnz));
    CHECK_HIP(hipMalloc(&d_val, sizeof(double) * nnz));
    CHECK_HIP(hipMalloc(&d_conv, sizeof(double) * nnz));
    CHECK_HIP(hipMalloc(&d_b, sizeof(double) * n));
    CHECK_HIP(hipMalloc(&d_x, sizeof(double) * n));
    CHECK_HIP(hipMalloc(&d_y, sizeof(double) * n));
    CHECK_HIP(hipMalloc(&d_gb, sizeof(double) * n));
    CHECK_HIP(hipMalloc(&d_gv, sizeof(double) * nnz));
    CHECK_HIP(hipMemcpy(d_rp, rp, sizeof(int32_t) * (n + 1), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_col, col, sizeof(int32_t) * nnz, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_val, val, sizeof(double) * nnz, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_conv, conv, sizeof(double) * nnz, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_b, b, sizeof(double) * n, hipMemcpyHostToDevice));

    sla_csr A = NULL, C = NULL;
    CHECK_SLA(sla_csr_create(&A, SLA_INPUT_CSR, n, nnz, 1, SLA_I32, d_rp, SLA_I32, d_col, SLA_F64,
                             d_val, SLA_FLAG_CHECK_SYMMETRIC, NULL));
    sla_info info, ainfo, binfo;
    CHECK_SLA(sla_pcg_solve(A, d_b, d_x, 1e-10, 5000, &info, NULL));
    int32_t path = 0;
    uint32_t fallbacks = 0;
    CHECK_SLA(sla_csr_get_last_path(A, &path, &fallbacks));
    CHECK_SLA(sla_spmv(A, d_x, d_y, NULL));
    CHECK_HIP(hipMemcpy(x, d_x, sizeof(double) * n, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(y, d_y, sizeof(double) * n, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < n; ++i) y[i] -= b[i];
    const double true_res = norm(y, n) / norm(b, n);
    /* adjoint of L = sum(x): grad_x = 1 */
    for (int64_t i = 0; i < n; ++i) y[i] = 1.0;
    CHECK_HIP(hipMemcpy(d_y, y, sizeof(double) * n, hipMemcpyHostToDevice));
    CHECK_SLA(sla_adjoint_backward(A, d_x, d_y, d_gb, d_gv, 1e-10, 5000, &ainfo, NULL));
    /* BiCGStab on the non-symmetric matrix */
    CHECK_SLA(sla_csr_create(&C, SLA_INPUT_CSR, n, nnz, 1, SLA_I32, d_rp, SLA_I32, d_col, SLA_F64,
                             d_conv, 0, NULL));
    CHECK_SLA(sla_bicgstab_solve(C, d_b, d_y, 1e-10, 5000, &binfo, NULL));
    /* a refused call: null right-hand side */
    const sla_status bad = sla_pcg_solve(A, NULL, d_x, 1e-10, 10, &info, NULL);
    const int bad_ok = bad == SLA_ERR_INVALID_ARG && strlen(sla_last_error()) > 0;

    FILE *f = fopen(argv[2], "wb");
    if (!f || fwrite(x, sizeof(double), (size_t)n, f) != (size_t)n) return 4;
    fclose(f);
    printf("iterations=%d status=%d rel_residual=%.3e true_residual=%.3e adjoint_iterations=%d "
           "adjoint_status=%d bicgstab_iterations=%d bicgstab_status=%d refused=%d path=%d "
           "fallbacks=%u version=%s\n",
           info.iterations, info.status, info.rel_residual, true_res, ainfo.iterations,
           ainfo.status, binfo.iterations, binfo.status, bad_ok, (int)path, (unsigned)fallbacks,
           sla_version());
    sla_csr_destroy(A);
    sla_csr_destroy(C);
    hipFree(d_rp); hipFree(d_col); hipFree(d_val); hipFree(d_conv); hipFree(d_b);
    hipFree(d_x); hipFree(d_y); hipFree(d_gb); hipFree(d_gv);
    free(rp); free(col); free(val); free(conv); free(b); free(x); free(y);
    const int pass = info.status == SLA_CONVERGED && true_res <= 1e-9 &&
                     ainfo.status == SLA_CONVERGED && binfo.status == SLA_CONVERGED && bad_ok;
    return pass ? 0 : 5;
}

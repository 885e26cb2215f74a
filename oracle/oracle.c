/*
 * CPU oracle for the sparse solve path — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test-suite, the package's smoke check and the benchmark's CPU
 * baseline leg may load this library. The product path never calls it and
 * shares no code, header, table or helper with it.
 *
 * Plain, slow, obviously correct C: natural loop order, sequential sums, no
 * blocking and no fused steps beyond what the definitions below state. Build
 * with -ffp-contract=off so a*b+c is never fused. OpenMP is used only on loops
 * whose iterations are independent (matrix rows, vector entries, batch
 * members); every reduction is a sequential loop, so results do not depend on
 * the thread count.
 *
 * Sources (torch-sla: "Differentiable Sparse Linear Algebra with Adjoint
 * Solvers and Sparse Tensor Parallelism for PyTorch", arXiv 2601.13994):
 *  - SparseTensor holds one matrix or a batch sharing one pattern (tensor-types
 *    passage of the API section);
 *  - the pytorch-native backend solves SPD systems by CG with Jacobi
 *    preconditioning (backend list; Table 3 and Table 4 text);
 *  - backward solves A^T lambda = dL/dx and assembles matrix gradients
 *    -lambda_i x_j on the stored entries (adjoint paragraph of the distributed
 *    section, referring to the adjoint derivation of Section 3.2);
 *  - the same backend also solves general systems by BiCGStab (backend list),
 *    which the distributed section says follows the CG template.
 * The pages print no PCG recurrence; the textbook preconditioned CG
 * (Hestenes-Stiefel with M = diag(A), x0 = 0) is used, and for BiCGStab van
 * der Vorst's preconditioned recurrence. Readings of the places
 * where the pages are silent are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_INVALID_ARG 1
#define ORC_ERR_INDEX_RANGE 2
#define ORC_ERR_INVALID_CSR 3
#define ORC_ERR_BAD_DIAGONAL 5
#define ORC_ERR_OOM 6

/* loops over fewer rows than this run on one thread (thread start-up would
 * dominate; results do not depend on it) */
#define ORC_MIN_PARALLEL 65536

#define ORC_CONVERGED 0
#define ORC_MAXIT 1
#define ORC_BREAKDOWN 2

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads for the calling thread's later parallel loops (timing only:
 * results do not depend on it) */
void orc_set_num_threads(int k) {
#ifdef _OPENMP
    if (k > 0) omp_set_num_threads(k);
#else
    (void)k;
#endif
}

/* ------------------------------------------------------------------ assembly
 * COO -> CSR. Reading (pages silent on format and duplicates): entries are
 * ordered by (row, col) with a stable sort, so equal positions keep their
 * input order; equal positions are merged by summing left to right in the
 * value type; slot[e] is the CSR position input entry e was merged into. A
 * batch of value sets shares the permutation.
 */
static int key_less(const int64_t *rows, const int64_t *cols, int64_t a, int64_t b) {
    return rows[a] < rows[b] || (rows[a] == rows[b] && cols[a] < cols[b]);
}

/* bottom-up stable merge sort of perm[0..m) by (rows, cols) */
static int stable_sort_perm(int64_t m, const int64_t *rows, const int64_t *cols, int64_t *perm) {
    int64_t *tmp = (int64_t *)malloc((size_t)(m > 0 ? m : 1) * sizeof(int64_t));
    if (!tmp) return ORC_ERR_OOM;
    int64_t *src = perm, *dst = tmp;
    for (int64_t width = 1; width < m; width *= 2) {
        for (int64_t lo = 0; lo < m; lo += 2 * width) {
            int64_t mid = lo + width < m ? lo + width : m;
            int64_t hi = lo + 2 * width < m ? lo + 2 * width : m;
            int64_t i = lo, j = mid, o = lo;
            while (i < mid && j < hi) {
                /* take from the right run only if strictly smaller: stable */
                if (key_less(rows, cols, src[j], src[i])) dst[o++] = src[j++];
                else dst[o++] = src[i++];
            }
            while (i < mid) dst[o++] = src[i++];
            while (j < hi) dst[o++] = src[j++];
        }
        int64_t *t = src; src = dst; dst = t;
    }
    if (src != perm) memcpy(perm, src, (size_t)m * sizeof(int64_t));
    free(tmp);
    return ORC_OK;
}

/* vals/csr_vals: [batch][nnz_in] with row stride nnz_in (only the first
 * *nnz_out columns of csr_vals are written). vbytes is 4 (float) or 8 (double). */
int orc_coo_to_csr(int64_t n, int64_t nnz_in, int32_t batch, const int64_t *rows,
                   const int64_t *cols, int32_t vbytes, const void *vals, int64_t *row_ptr,
                   int64_t *col_idx, void *csr_vals, int64_t *slot, int64_t *nnz_out) {
    if (n < 1 || nnz_in < 0 || batch < 1 || (vbytes != 4 && vbytes != 8)) return ORC_ERR_INVALID_ARG;
    for (int64_t e = 0; e < nnz_in; ++e)
        if (rows[e] < 0 || rows[e] >= n || cols[e] < 0 || cols[e] >= n) return ORC_ERR_INDEX_RANGE;

    int64_t *perm = (int64_t *)malloc((size_t)(nnz_in > 0 ? nnz_in : 1) * sizeof(int64_t));
    if (!perm) return ORC_ERR_OOM;
    for (int64_t e = 0; e < nnz_in; ++e) perm[e] = e;
    int st = stable_sort_perm(nnz_in, rows, cols, perm);
    if (st != ORC_OK) { free(perm); return st; }

    /* unique positions in sorted order */
    int64_t u = -1;
    for (int64_t t = 0; t < nnz_in; ++t) {
        int64_t e = perm[t];
        if (t == 0 || rows[e] != rows[perm[t - 1]] || cols[e] != cols[perm[t - 1]]) {
            ++u;
            col_idx[u] = cols[e];
        }
        slot[e] = u;
    }
    int64_t nnz = u + 1;
    *nnz_out = nnz;

    /* merge duplicates: first value, then left-to-right additions in sorted (= input) order */
    for (int32_t s = 0; s < batch; ++s) {
        if (vbytes == 8) {
            const double *v = (const double *)vals + (int64_t)s * nnz_in;
            double *o = (double *)csr_vals + (int64_t)s * nnz_in;
            for (int64_t t = 0; t < nnz_in; ++t) {
                int64_t e = perm[t];
                if (t == 0 || slot[e] != slot[perm[t - 1]]) o[slot[e]] = v[e];
                else o[slot[e]] = o[slot[e]] + v[e];
            }
        } else {
            const float *v = (const float *)vals + (int64_t)s * nnz_in;
            float *o = (float *)csr_vals + (int64_t)s * nnz_in;
            for (int64_t t = 0; t < nnz_in; ++t) {
                int64_t e = perm[t];
                if (t == 0 || slot[e] != slot[perm[t - 1]]) o[slot[e]] = v[e];
                else o[slot[e]] = o[slot[e]] + v[e];
            }
        }
    }

    /* row pointer: count unique entries per row, then running sum */
    for (int64_t i = 0; i <= n; ++i) row_ptr[i] = 0;
    {
        int64_t prev = -1;
        for (int64_t t = 0; t < nnz_in; ++t) {
            int64_t e = perm[t];
            if (slot[e] != prev) { row_ptr[rows[e] + 1] += 1; prev = slot[e]; }
        }
    }
    for (int64_t i = 0; i < n; ++i) row_ptr[i + 1] += row_ptr[i];
    free(perm);
    return ORC_OK;
}

/* Validate CSR input that is adopted as is: row_ptr[0] = 0, non-decreasing,
 * row_ptr[n] = nnz, columns in range and strictly increasing inside a row. */
int orc_check_csr(int64_t n, int64_t nnz, const int64_t *row_ptr, const int64_t *col) {
    if (n < 1 || nnz < 0) return ORC_ERR_INVALID_ARG;
    if (row_ptr[0] != 0 || row_ptr[n] != nnz) return ORC_ERR_INVALID_CSR;
    for (int64_t i = 0; i < n; ++i)
        if (row_ptr[i + 1] < row_ptr[i]) return ORC_ERR_INVALID_CSR;
    for (int64_t k = 0; k < nnz; ++k)
        if (col[k] < 0 || col[k] >= n) return ORC_ERR_INDEX_RANGE;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = row_ptr[i] + 1; k < row_ptr[i + 1]; ++k)
            if (col[k] <= col[k - 1]) return ORC_ERR_INVALID_CSR;
    return ORC_OK;
}

/* Explicit transpose (counting sort by column, stable in row order). */
static int transpose_f64(int64_t n, const int64_t *row_ptr, const int64_t *col, const double *val,
                         int64_t *t_ptr, int64_t *t_col, double *t_val) {
    int64_t nnz = row_ptr[n];
    for (int64_t j = 0; j <= n; ++j) t_ptr[j] = 0;
    for (int64_t k = 0; k < nnz; ++k) t_ptr[col[k] + 1] += 1;
    for (int64_t j = 0; j < n; ++j) t_ptr[j + 1] += t_ptr[j];
    int64_t *fill = (int64_t *)malloc((size_t)(n + 1) * sizeof(int64_t));
    if (!fill) return ORC_ERR_OOM;
    memcpy(fill, t_ptr, (size_t)(n + 1) * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            int64_t d = fill[col[k]]++;
            t_col[d] = i;
            t_val[d] = val[k];
        }
    free(fill);
    return ORC_OK;
}

static int transpose_f32(int64_t n, const int64_t *row_ptr, const int64_t *col, const float *val,
                         int64_t *t_ptr, int64_t *t_col, float *t_val) {
    int64_t nnz = row_ptr[n];
    for (int64_t j = 0; j <= n; ++j) t_ptr[j] = 0;
    for (int64_t k = 0; k < nnz; ++k) t_ptr[col[k] + 1] += 1;
    for (int64_t j = 0; j < n; ++j) t_ptr[j + 1] += t_ptr[j];
    int64_t *fill = (int64_t *)malloc((size_t)(n + 1) * sizeof(int64_t));
    if (!fill) return ORC_ERR_OOM;
    memcpy(fill, t_ptr, (size_t)(n + 1) * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            int64_t d = fill[col[k]]++;
            t_col[d] = i;
            t_val[d] = val[k];
        }
    free(fill);
    return ORC_OK;
}

/* 1 if A equals its transpose bit for bit (same pattern, identical values). */
int orc_is_symmetric_f64(int64_t n, const int64_t *row_ptr, const int64_t *col, const double *val) {
    int64_t nnz = row_ptr[n];
    int64_t *tp = (int64_t *)malloc((size_t)(n + 1) * sizeof(int64_t));
    int64_t *tc = (int64_t *)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
    double *tv = (double *)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(double));
    int res = -1;
    if (tp && tc && tv && transpose_f64(n, row_ptr, col, val, tp, tc, tv) == ORC_OK) {
        res = 1;
        for (int64_t i = 0; i <= n && res; ++i) if (tp[i] != row_ptr[i]) res = 0;
        for (int64_t k = 0; k < nnz && res; ++k)
            if (tc[k] != col[k] || memcmp(&tv[k], &val[k], sizeof(double)) != 0) res = 0;
    }
    free(tp); free(tc); free(tv);
    return res;
}

/* ------------------------------------------------------------------ SpMV
 * y = A x (the .matvec of SparseTensor). fp64: y_i = sum over the row's
 * entries in storage order of val*x[col], accumulated sequentially from 0.
 * fp32 storage: products and sums in fp64, one rounding to fp32 on store
 * (reading: the pages fix no precision for the fp32 case). */
void orc_spmv_f64(int64_t n, const int64_t *row_ptr, const int64_t *col, const double *val,
                  const double *x, double *y) {
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) s = s + val[k] * x[col[k]];
        y[i] = s;
    }
}

void orc_spmv_f32(int64_t n, const int64_t *row_ptr, const int64_t *col, const float *val,
                  const float *x, float *y) {
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            s = s + (double)val[k] * (double)x[col[k]];
        y[i] = (float)s;
    }
}

/* ------------------------------------------------------------------ SpMV backward
 * torch-sla counts matvec among the operations that carry gradients (the
 * tensor-types passage; Table 1's operation list). For y = A x and an upstream
 * gradient g = dL/dy the definitions are
 *   dL/dx_j    = sum over stored entries (i, j) of a_ij g_i   (A^T g)
 *   dL/da_ij   = g_i x_j                                      (stored entries)
 * A^T g is accumulated while walking A row by row, so for each j the terms
 * arrive in increasing i; fp32 storage keeps the sums in fp64 and rounds
 * once per stored value. */
void orc_spmv_backward_f64(int64_t n, const int64_t *row_ptr, const int64_t *col,
                           const double *val, const double *x, const double *g, double *grad_x,
                           double *grad_vals) {
    for (int64_t j = 0; j < n; ++j) grad_x[j] = 0.0;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            grad_x[col[k]] = grad_x[col[k]] + val[k] * g[i];
            grad_vals[k] = g[i] * x[col[k]];
        }
}

int orc_spmv_backward_f32(int64_t n, const int64_t *row_ptr, const int64_t *col, const float *val,
                          const float *x, const float *g, float *grad_x, float *grad_vals) {
    double *acc = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    if (!acc) return ORC_ERR_OOM;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) {
            acc[col[k]] = acc[col[k]] + (double)val[k] * (double)g[i];
            grad_vals[k] = (float)((double)g[i] * (double)x[col[k]]);
        }
    for (int64_t j = 0; j < n; ++j) grad_x[j] = (float)acc[j];
    free(acc);
    return ORC_OK;
}

/* ------------------------------------------------------------------ Jacobi
 * M = diag(A): d_i is the stored entry (i, i); it must exist, be finite and
 * positive (the matrix is SPD). dinv_i = 1/d_i; the preconditioner is applied
 * as a multiplication by dinv (reading). fp32: 1/d in fp64, rounded once. */
int orc_jacobi_f64(int64_t n, const int64_t *row_ptr, const int64_t *col, const double *val,
                   double *dinv) {
    for (int64_t i = 0; i < n; ++i) {
        int found = 0;
        double d = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            if (col[k] == i) { d = val[k]; found = 1; }
        if (!found || !(d > 0.0) || !isfinite(d)) return ORC_ERR_BAD_DIAGONAL;
        dinv[i] = 1.0 / d;
    }
    return ORC_OK;
}

int orc_jacobi_f32(int64_t n, const int64_t *row_ptr, const int64_t *col, const float *val,
                   float *dinv) {
    for (int64_t i = 0; i < n; ++i) {
        int found = 0;
        float d = 0.0f;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            if (col[k] == i) { d = val[k]; found = 1; }
        if (!found || !(d > 0.0f) || !isfinite(d)) return ORC_ERR_BAD_DIAGONAL;
        dinv[i] = (float)(1.0 / (double)d);
    }
    return ORC_OK;
}

static double dot_f64(int64_t n, const double *a, const double *b) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s = s + a[i] * b[i];
    return s;
}

/* ------------------------------------------------------------------ PCG
 * Jacobi-preconditioned CG for SPD A, x0 = 0:
 *   r = b, z = M^-1 r, p = z, rho = r.z
 *   each iteration k = 1..maxit:
 *     q = A p; sigma = p.q        (breakdown if sigma is not > 0 or not finite)
 *     alpha = rho / sigma; x += alpha p; r -= alpha q
 *     stop (converged) when ||r||_2 <= tol ||b||_2, r the updated residual
 *     z = M^-1 r; rho' = r.z; beta = rho'/rho; p = z + beta p
 * Readings: the pages name the two reductions <r,r> and <p,Ap> of each CG
 * step; with Jacobi the r.z product is formed next to r.r. b = 0 returns x = 0
 * after 0 iterations. rel_res is ||r||/||b|| of the last updated residual.
 * outcome: ORC_CONVERGED / ORC_MAXIT / ORC_BREAKDOWN. */
int orc_pcg_f64(int64_t n, const int64_t *row_ptr, const int64_t *col, const double *val,
                const double *b, double tol, int32_t maxit, double *x, int32_t *iters,
                double *rel_res, int32_t *outcome) {
    if (n < 1 || maxit < 0) return ORC_ERR_INVALID_ARG;
    double *dinv = (double *)malloc((size_t)n * sizeof(double));
    double *r = (double *)malloc((size_t)n * sizeof(double));
    double *p = (double *)malloc((size_t)n * sizeof(double));
    double *q = (double *)malloc((size_t)n * sizeof(double));
    double *z = (double *)malloc((size_t)n * sizeof(double));
    if (!dinv || !r || !p || !q || !z) {
        free(dinv); free(r); free(p); free(q); free(z);
        return ORC_ERR_OOM;
    }
    int st = orc_jacobi_f64(n, row_ptr, col, val, dinv);
    if (st != ORC_OK) { free(dinv); free(r); free(p); free(q); free(z); return st; }

    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; }
    double bb = dot_f64(n, b, b);
    *iters = 0; *rel_res = 0.0; *outcome = ORC_CONVERGED;
    if (bb == 0.0) goto done;
    for (int64_t i = 0; i < n; ++i) { z[i] = dinv[i] * r[i]; p[i] = z[i]; }
    double rho = dot_f64(n, r, z);
    double rr = bb;
    *outcome = ORC_MAXIT;
    *iters = maxit;
    for (int32_t k = 1; k <= maxit; ++k) {
        orc_spmv_f64(n, row_ptr, col, val, p, q);
        double sigma = dot_f64(n, p, q);
        if (!(sigma > 0.0) || !isfinite(sigma)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        double alpha = rho / sigma;
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) { x[i] = x[i] + alpha * p[i]; r[i] = r[i] - alpha * q[i]; }
        rr = dot_f64(n, r, r);
        if (sqrt(rr) <= tol * sqrt(bb)) { *outcome = ORC_CONVERGED; *iters = k; break; }
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) z[i] = dinv[i] * r[i];
        double rho_new = dot_f64(n, r, z);
        double beta = rho_new / rho;
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) p[i] = z[i] + beta * p[i];
        rho = rho_new;
    }
    *rel_res = sqrt(rr / bb);
done:
    free(dinv); free(r); free(p); free(q); free(z);
    return ORC_OK;
}

/* fp32 storage, fp64 arithmetic: every stored vector (x, r, p, q) and dinv is
 * float; each elementwise result is formed in double and rounded once on
 * store; dot products accumulate in double over the stored float values; z is
 * never stored (formed in double from the stored dinv and r). */
int orc_pcg_f32(int64_t n, const int64_t *row_ptr, const int64_t *col, const float *val,
                const float *b, double tol, int32_t maxit, float *x, int32_t *iters,
                double *rel_res, int32_t *outcome) {
    if (n < 1 || maxit < 0) return ORC_ERR_INVALID_ARG;
    float *dinv = (float *)malloc((size_t)n * sizeof(float));
    float *r = (float *)malloc((size_t)n * sizeof(float));
    float *p = (float *)malloc((size_t)n * sizeof(float));
    float *q = (float *)malloc((size_t)n * sizeof(float));
    if (!dinv || !r || !p || !q) { free(dinv); free(r); free(p); free(q); return ORC_ERR_OOM; }
    int st = orc_jacobi_f32(n, row_ptr, col, val, dinv);
    if (st != ORC_OK) { free(dinv); free(r); free(p); free(q); return st; }

    double bb = 0.0;
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0f; r[i] = b[i]; bb = bb + (double)b[i] * (double)b[i]; }
    *iters = 0; *rel_res = 0.0; *outcome = ORC_CONVERGED;
    if (bb == 0.0) goto done32;
    double rho = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double z = (double)dinv[i] * (double)r[i];
        p[i] = (float)z;
        rho = rho + (double)r[i] * z;
    }
    double rr = bb;
    *outcome = ORC_MAXIT;
    *iters = maxit;
    for (int32_t k = 1; k <= maxit; ++k) {
        orc_spmv_f32(n, row_ptr, col, val, p, q);
        double sigma = 0.0;
        for (int64_t i = 0; i < n; ++i) sigma = sigma + (double)p[i] * (double)q[i];
        if (!(sigma > 0.0) || !isfinite(sigma)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        double alpha = rho / sigma;
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) {
            x[i] = (float)((double)x[i] + alpha * (double)p[i]);
            r[i] = (float)((double)r[i] - alpha * (double)q[i]);
        }
        rr = 0.0;
        for (int64_t i = 0; i < n; ++i) rr = rr + (double)r[i] * (double)r[i];
        if (sqrt(rr) <= tol * sqrt(bb)) { *outcome = ORC_CONVERGED; *iters = k; break; }
        double rho_new = 0.0;
        for (int64_t i = 0; i < n; ++i) rho_new = rho_new + (double)r[i] * ((double)dinv[i] * (double)r[i]);
        double beta = rho_new / rho;
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i)
            p[i] = (float)((double)dinv[i] * (double)r[i] + beta * (double)p[i]);
        rho = rho_new;
    }
    *rel_res = sqrt(rr / bb);
done32:
    free(dinv); free(r); free(p); free(q);
    return ORC_OK;
}

/* Batch sharing one pattern: B independent solves, system s using value set s
 * (vals [B][nnz]) and right-hand side s (b, x: [B][n]); each system stops on
 * its own test (reading: per-system stopping, so slice s equals the single
 * solve of (A_s, b_s)). vbytes selects fp64 or fp32 storage. */
int orc_pcg_batched(int64_t n, int32_t batch, const int64_t *row_ptr, const int64_t *col,
                    int32_t vbytes, const void *vals, const void *b, double tol, int32_t maxit,
                    void *x, int32_t *iters, double *rel_res, int32_t *outcome) {
    if (batch < 1 || (vbytes != 4 && vbytes != 8)) return ORC_ERR_INVALID_ARG;
    int64_t nnz = row_ptr[n];
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) if (batch > 1)
    for (int32_t s = 0; s < batch; ++s) {
        int st;
        if (vbytes == 8)
            st = orc_pcg_f64(n, row_ptr, col, (const double *)vals + (int64_t)s * nnz,
                             (const double *)b + (int64_t)s * n, tol, maxit,
                             (double *)x + (int64_t)s * n, &iters[s], &rel_res[s], &outcome[s]);
        else
            st = orc_pcg_f32(n, row_ptr, col, (const float *)vals + (int64_t)s * nnz,
                             (const float *)b + (int64_t)s * n, tol, maxit,
                             (float *)x + (int64_t)s * n, &iters[s], &rel_res[s], &outcome[s]);
        if (st != ORC_OK) {
#pragma omp critical
            err = st;
        }
    }
    return err;
}

/* ------------------------------------------------------------------ adjoint
 * Backward of x = A^{-1} b for upstream g = dL/dx: solve A^T lambda = g (same
 * PCG, same tol and maxit, x0 = 0 — reading: the pages fix no adjoint
 * tolerance), then dL/db = lambda and, for every stored entry k = (i, j),
 * dL/dval[k] = -lambda_i x_j. A^T is formed explicitly so the solve is the
 * definition written out; for the SPD matrices the path targets it equals A.
 * fp32 storage: lambda is float (fp32 PCG), grad = float(-(double)l*(double)x). */
int orc_adjoint(int64_t n, int32_t batch, const int64_t *row_ptr, const int64_t *col,
                int32_t vbytes, const void *vals, const void *x, const void *g, double tol,
                int32_t maxit, void *lambda, void *grad_vals, int32_t *iters, double *rel_res,
                int32_t *outcome) {
    if (n < 1 || batch < 1 || (vbytes != 4 && vbytes != 8)) return ORC_ERR_INVALID_ARG;
    int64_t nnz = row_ptr[n];
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1) if (batch > 1)
    for (int32_t s = 0; s < batch; ++s) {
        int st = ORC_OK;
        int64_t *tp = (int64_t *)malloc((size_t)(n + 1) * sizeof(int64_t));
        int64_t *tc = (int64_t *)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
        void *tv = malloc((size_t)(nnz > 0 ? nnz : 1) * (size_t)vbytes);
        if (!tp || !tc || !tv) st = ORC_ERR_OOM;
        else if (vbytes == 8) {
            const double *v = (const double *)vals + (int64_t)s * nnz;
            const double *xs = (const double *)x + (int64_t)s * n;
            double *ls = (double *)lambda + (int64_t)s * n;
            double *gr = (double *)grad_vals + (int64_t)s * nnz;
            st = transpose_f64(n, row_ptr, col, v, tp, tc, (double *)tv);
            if (st == ORC_OK)
                st = orc_pcg_f64(n, tp, tc, (const double *)tv, (const double *)g + (int64_t)s * n,
                                 tol, maxit, ls, &iters[s], &rel_res[s], &outcome[s]);
            if (st == ORC_OK)
                for (int64_t i = 0; i < n; ++i)
                    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) gr[k] = -ls[i] * xs[col[k]];
        } else {
            const float *v = (const float *)vals + (int64_t)s * nnz;
            const float *xs = (const float *)x + (int64_t)s * n;
            float *ls = (float *)lambda + (int64_t)s * n;
            float *gr = (float *)grad_vals + (int64_t)s * nnz;
            st = transpose_f32(n, row_ptr, col, v, tp, tc, (float *)tv);
            if (st == ORC_OK)
                st = orc_pcg_f32(n, tp, tc, (const float *)tv, (const float *)g + (int64_t)s * n,
                                 tol, maxit, ls, &iters[s], &rel_res[s], &outcome[s]);
            if (st == ORC_OK)
                for (int64_t i = 0; i < n; ++i)
                    for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
                        gr[k] = (float)(-(double)ls[i] * (double)xs[col[k]]);
        }
        free(tp); free(tc); free(tv);
        if (st != ORC_OK) {
#pragma omp critical
            err = st;
        }
    }
    return err;
}

/* ------------------------------------------------------------------ BiCGStab
 * torch-sla's pytorch-native backend also offers BiCGStab for general
 * (non-symmetric) systems (backend list of the API section; the distributed
 * section notes that BiCGStab follows the CG template with more inner
 * products). The pages print no recurrence; the one used is van der Vorst's
 * preconditioned BiCGStab (SIAM J. Sci. Stat. Comput. 13, 1992; the
 * "Templates" book's preconditioned form), with the Jacobi preconditioner
 * M = diag(A) applied on the right, x0 = 0 and shadow residual r^ = b:
 *   r = b, rho = r^.r
 *   each iteration k = 1..maxit:
 *     p = r                         (k = 1)
 *     p = r + beta (p - omega v)    (k > 1)
 *     p^ = M^-1 p; v = A p^; sigma = r^.v       breakdown: sigma = 0
 *     alpha = rho / sigma; s = r - alpha v
 *     ||s|| <= tol ||b||: x += alpha p^, r = s, converged (half step)
 *     s^ = M^-1 s; t = A s^; omega = t.s / t.t  breakdown: t.t = 0 or omega = 0
 *     x += alpha p^ + omega s^; r = s - omega t
 *     ||r|| <= tol ||b||: converged; k = maxit: budget spent
 *     rho' = r^.r                               breakdown: rho' = 0
 *     beta = (rho'/rho)(alpha/omega); rho = rho'
 * Readings (the pages fix none of these): breakdown is an exact zero or a
 * non-finite value of the quantity named; a breakdown at sigma (or a
 * non-finite ||s||) leaves x and r as they were; one at omega keeps the half
 * step (x += alpha p^, r = s), which is a valid iterate; iterations count the
 * loop passes started, including the one that stopped. b = 0 returns x = 0
 * after 0 iterations. rel_res is ||r||/||b|| of the last residual formed (s
 * after a half step). Jacobi here needs a present, non-zero, finite diagonal
 * of either sign. x += alpha p^ + omega s^ is formed as (x + alpha p^) +
 * omega s^. */
static int jacobi_nonzero_f64(int64_t n, const int64_t *row_ptr, const int64_t *col,
                              const double *val, double *dinv) {
    for (int64_t i = 0; i < n; ++i) {
        int found = 0;
        double d = 0.0;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            if (col[k] == i) { d = val[k]; found = 1; }
        if (!found || d == 0.0 || !isfinite(d)) return ORC_ERR_BAD_DIAGONAL;
        dinv[i] = 1.0 / d;
    }
    return ORC_OK;
}

static int jacobi_nonzero_f32(int64_t n, const int64_t *row_ptr, const int64_t *col,
                              const float *val, float *dinv) {
    for (int64_t i = 0; i < n; ++i) {
        int found = 0;
        float d = 0.0f;
        for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
            if (col[k] == i) { d = val[k]; found = 1; }
        if (!found || d == 0.0f || !isfinite(d)) return ORC_ERR_BAD_DIAGONAL;
        dinv[i] = (float)(1.0 / (double)d);
    }
    return ORC_OK;
}

int orc_bicgstab_f64(int64_t n, const int64_t *row_ptr, const int64_t *col, const double *val,
                     const double *b, double tol, int32_t maxit, double *x, int32_t *iters,
                     double *rel_res, int32_t *outcome) {
    if (n < 1 || maxit < 0) return ORC_ERR_INVALID_ARG;
    double *w[9];
    int st = ORC_OK;
    for (int j = 0; j < 9; ++j) {
        w[j] = (double *)malloc((size_t)n * sizeof(double));
        if (!w[j]) st = ORC_ERR_OOM;
    }
    double *dinv = w[0], *r = w[1], *rh = w[2], *p = w[3], *ph = w[4], *v = w[5], *s = w[6],
           *sh = w[7], *t = w[8];
    if (st == ORC_OK) st = jacobi_nonzero_f64(n, row_ptr, col, val, dinv);
    if (st != ORC_OK) {
        for (int j = 0; j < 9; ++j) free(w[j]);
        return st;
    }
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0; r[i] = b[i]; rh[i] = b[i]; }
    double bb = dot_f64(n, b, b);
    double rr = bb, rho = bb, alpha = 0.0, omega = 0.0, beta = 0.0;
    *iters = 0; *rel_res = 0.0; *outcome = ORC_CONVERGED;
    if (bb == 0.0) goto done;
    *outcome = ORC_MAXIT;
    *iters = maxit;
    for (int32_t k = 1; k <= maxit; ++k) {
        if (k == 1)
            for (int64_t i = 0; i < n; ++i) p[i] = r[i];
        else
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
            for (int64_t i = 0; i < n; ++i) p[i] = r[i] + beta * (p[i] - omega * v[i]);
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) ph[i] = dinv[i] * p[i];
        orc_spmv_f64(n, row_ptr, col, val, ph, v);
        double sigma = dot_f64(n, rh, v);
        if (sigma == 0.0 || !isfinite(sigma)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        alpha = rho / sigma;
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) s[i] = r[i] - alpha * v[i];
        double ss = dot_f64(n, s, s);
        if (!isfinite(ss)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        if (sqrt(ss) <= tol * sqrt(bb)) {
            for (int64_t i = 0; i < n; ++i) { x[i] = x[i] + alpha * ph[i]; r[i] = s[i]; }
            rr = ss;
            *outcome = ORC_CONVERGED; *iters = k;
            break;
        }
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) sh[i] = dinv[i] * s[i];
        orc_spmv_f64(n, row_ptr, col, val, sh, t);
        double tt = dot_f64(n, t, t), ts = dot_f64(n, t, s);
        omega = tt == 0.0 ? 0.0 : ts / tt;
        if (tt == 0.0 || !isfinite(tt) || !isfinite(omega) || omega == 0.0) {
            for (int64_t i = 0; i < n; ++i) { x[i] = x[i] + alpha * ph[i]; r[i] = s[i]; }
            rr = ss;
            *outcome = ORC_BREAKDOWN; *iters = k;
            break;
        }
#pragma omp parallel for schedule(static) if (n >= ORC_MIN_PARALLEL)
        for (int64_t i = 0; i < n; ++i) {
            x[i] = (x[i] + alpha * ph[i]) + omega * sh[i];
            r[i] = s[i] - omega * t[i];
        }
        rr = dot_f64(n, r, r);
        if (sqrt(rr) <= tol * sqrt(bb)) { *outcome = ORC_CONVERGED; *iters = k; break; }
        if (!isfinite(rr)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        if (k == maxit) break;
        double rho_new = dot_f64(n, rh, r);
        if (rho_new == 0.0 || !isfinite(rho_new)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        beta = (rho_new / rho) * (alpha / omega);
        rho = rho_new;
    }
    *rel_res = sqrt(rr / bb);
done:
    for (int j = 0; j < 9; ++j) free(w[j]);
    return ORC_OK;
}

/* fp32 storage, fp64 arithmetic (as for PCG): every stored vector (x, r, p,
 * p^, v, s, s^, t) and dinv is float, each element formed in double from the
 * stored floats and rounded once on store; inner products accumulate in
 * double over the stored floats; r^ is b itself. */
static double dot_f32(int64_t n, const float *a, const float *b) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s = s + (double)a[i] * (double)b[i];
    return s;
}

int orc_bicgstab_f32(int64_t n, const int64_t *row_ptr, const int64_t *col, const float *val,
                     const float *b, double tol, int32_t maxit, float *x, int32_t *iters,
                     double *rel_res, int32_t *outcome) {
    if (n < 1 || maxit < 0) return ORC_ERR_INVALID_ARG;
    float *w[8];
    int st = ORC_OK;
    for (int j = 0; j < 8; ++j) {
        w[j] = (float *)malloc((size_t)n * sizeof(float));
        if (!w[j]) st = ORC_ERR_OOM;
    }
    float *dinv = w[0], *r = w[1], *p = w[2], *ph = w[3], *v = w[4], *s = w[5], *sh = w[6],
          *t = w[7];
    const float *rh = b;
    if (st == ORC_OK) st = jacobi_nonzero_f32(n, row_ptr, col, val, dinv);
    if (st != ORC_OK) {
        for (int j = 0; j < 8; ++j) free(w[j]);
        return st;
    }
    for (int64_t i = 0; i < n; ++i) { x[i] = 0.0f; r[i] = b[i]; }
    double bb = dot_f32(n, b, b);
    double rr = bb, rho = bb, alpha = 0.0, omega = 0.0, beta = 0.0;
    *iters = 0; *rel_res = 0.0; *outcome = ORC_CONVERGED;
    if (bb == 0.0) goto done32;
    *outcome = ORC_MAXIT;
    *iters = maxit;
    for (int32_t k = 1; k <= maxit; ++k) {
        if (k == 1)
            for (int64_t i = 0; i < n; ++i) p[i] = r[i];
        else
            for (int64_t i = 0; i < n; ++i)
                p[i] = (float)((double)r[i] + beta * ((double)p[i] - omega * (double)v[i]));
        for (int64_t i = 0; i < n; ++i) ph[i] = (float)((double)dinv[i] * (double)p[i]);
        orc_spmv_f32(n, row_ptr, col, val, ph, v);
        double sigma = dot_f32(n, rh, v);
        if (sigma == 0.0 || !isfinite(sigma)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        alpha = rho / sigma;
        for (int64_t i = 0; i < n; ++i) s[i] = (float)((double)r[i] - alpha * (double)v[i]);
        double ss = dot_f32(n, s, s);
        if (!isfinite(ss)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        if (sqrt(ss) <= tol * sqrt(bb)) {
            for (int64_t i = 0; i < n; ++i) {
                x[i] = (float)((double)x[i] + alpha * (double)ph[i]);
                r[i] = s[i];
            }
            rr = ss;
            *outcome = ORC_CONVERGED; *iters = k;
            break;
        }
        for (int64_t i = 0; i < n; ++i) sh[i] = (float)((double)dinv[i] * (double)s[i]);
        orc_spmv_f32(n, row_ptr, col, val, sh, t);
        double tt = dot_f32(n, t, t), ts = dot_f32(n, t, s);
        omega = tt == 0.0 ? 0.0 : ts / tt;
        if (tt == 0.0 || !isfinite(tt) || !isfinite(omega) || omega == 0.0) {
            for (int64_t i = 0; i < n; ++i) {
                x[i] = (float)((double)x[i] + alpha * (double)ph[i]);
                r[i] = s[i];
            }
            rr = ss;
            *outcome = ORC_BREAKDOWN; *iters = k;
            break;
        }
        for (int64_t i = 0; i < n; ++i) {
            x[i] = (float)(((double)x[i] + alpha * (double)ph[i]) + omega * (double)sh[i]);
            r[i] = (float)((double)s[i] - omega * (double)t[i]);
        }
        rr = dot_f32(n, r, r);
        if (sqrt(rr) <= tol * sqrt(bb)) { *outcome = ORC_CONVERGED; *iters = k; break; }
        if (!isfinite(rr)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        if (k == maxit) break;
        double rho_new = dot_f32(n, rh, r);
        if (rho_new == 0.0 || !isfinite(rho_new)) { *outcome = ORC_BREAKDOWN; *iters = k; break; }
        beta = (rho_new / rho) * (alpha / omega);
        rho = rho_new;
    }
    *rel_res = sqrt(rr / bb);
done32:
    for (int j = 0; j < 8; ++j) free(w[j]);
    return ORC_OK;
}

/* Backward of x = A^{-1} b solved by BiCGStab, for upstream g = dL/dx: the
 * same adjoint as for PCG (solve A^T lambda = g, then dL/db = lambda and
 * dL/dval[k] = -lambda_i x_j for stored entry k = (i, j)), with the adjoint
 * system solved by the BiCGStab above on the explicitly formed A^T (same tol
 * and maxit). One system (the solver takes one). */
int orc_bicgstab_adjoint(int64_t n, const int64_t *row_ptr, const int64_t *col, int32_t vbytes,
                         const void *vals, const void *x, const void *g, double tol,
                         int32_t maxit, void *lambda, void *grad_vals, int32_t *iters,
                         double *rel_res, int32_t *outcome) {
    if (n < 1 || (vbytes != 4 && vbytes != 8)) return ORC_ERR_INVALID_ARG;
    int64_t nnz = row_ptr[n];
    int st = ORC_OK;
    int64_t *tp = (int64_t *)malloc((size_t)(n + 1) * sizeof(int64_t));
    int64_t *tc = (int64_t *)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
    void *tv = malloc((size_t)(nnz > 0 ? nnz : 1) * (size_t)vbytes);
    if (!tp || !tc || !tv) st = ORC_ERR_OOM;
    else if (vbytes == 8) {
        const double *xs = (const double *)x;
        double *ls = (double *)lambda, *gr = (double *)grad_vals;
        st = transpose_f64(n, row_ptr, col, (const double *)vals, tp, tc, (double *)tv);
        if (st == ORC_OK)
            st = orc_bicgstab_f64(n, tp, tc, (const double *)tv, (const double *)g, tol, maxit, ls,
                                  iters, rel_res, outcome);
        if (st == ORC_OK)
            for (int64_t i = 0; i < n; ++i)
                for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k) gr[k] = -ls[i] * xs[col[k]];
    } else {
        const float *xs = (const float *)x;
        float *ls = (float *)lambda, *gr = (float *)grad_vals;
        st = transpose_f32(n, row_ptr, col, (const float *)vals, tp, tc, (float *)tv);
        if (st == ORC_OK)
            st = orc_bicgstab_f32(n, tp, tc, (const float *)tv, (const float *)g, tol, maxit, ls,
                                  iters, rel_res, outcome);
        if (st == ORC_OK)
            for (int64_t i = 0; i < n; ++i)
                for (int64_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
                    gr[k] = (float)(-(double)ls[i] * (double)xs[col[k]]);
    }
    free(tp); free(tc); free(tv);
    return st;
}

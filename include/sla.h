/*
 * sla.h — C ABI of the MI355X sparse solve library: CSR assembly, SpMV,
 * Jacobi-preconditioned CG and its adjoint backward, for one matrix or a
 * batch of matrices sharing one sparsity pattern.
 *
 * What the calls compute follows torch-sla ("Differentiable Sparse Linear
 * Algebra with Adjoint Solvers and Sparse Tensor Parallelism for PyTorch",
 * arXiv 2601.13994):
 *  - a SparseTensor holds one matrix or a batch sharing one pattern, and
 *    exposes .matvec and .solve (tensor-types passage of its API section);
 *  - the pytorch-native backend solves SPD systems by CG with Jacobi
 *    preconditioning, all tensors staying on the device (backend list; the
 *    distributed-CG paragraph; Table 3 and Table 4 text);
 *  - the solve is wrapped as one autograd node whose backward solves
 *    A^T lambda = dL/dx and forms the matrix gradient -lambda_i x_j on the
 *    stored entries (autograd-wrapping paragraph; adjoint paragraph of the
 *    distributed section, result of its Section 3.2; Figure 2 discussion).
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless marked (host). Device arrays are
 *    contiguous. Batched vectors are batch-major: [batch][n]; batched values
 *    are [batch][nnz].
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is ordered on it. Calls on one handle must not overlap (the handle owns
 *    one solve workspace).
 *  - Ownership: the library copies what it keeps; the caller keeps ownership
 *    of every argument pointer, and nothing is retained after a call returns.
 *    A handle owns its device memory, allocated at create; solves allocate
 *    nothing on the device.
 *  - Errors: every call returns an sla_status and never aborts or throws;
 *    sla_last_error() gives a message for the calling thread's last failure.
 *    Solver outcomes are reported per system in sla_info, not as errors.
 *  - Limits: 1 <= n < 2^31, 1 <= batch <= 256, nnz < 2^62.
 */
#ifndef SLA_H
#define SLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sla_csr_s *sla_csr; /* opaque handle */

typedef enum {
    SLA_OK = 0,
    SLA_ERR_INVALID_ARG = 1,   /* null pointer, bad enum, size out of range */
    SLA_ERR_INDEX_RANGE = 2,   /* a row or column index outside [0, n) */
    SLA_ERR_INVALID_CSR = 3,   /* CSR input: row_ptr not 0..nnz non-decreasing, or columns
                                  not strictly increasing inside a row */
    SLA_ERR_NOT_SYMMETRIC = 4, /* SLA_FLAG_CHECK_SYMMETRIC given and A != A^T bit for bit */
    SLA_ERR_BAD_DIAGONAL = 5,  /* solve on a matrix with a diagonal entry Jacobi cannot
                                  use: missing, non-finite, or <= 0 for PCG (d_i > 0),
                                  = 0 for BiCGStab (d_i != 0) */
    SLA_ERR_OOM = 6,           /* device or pinned-host allocation failed */
    SLA_ERR_HIP = 7            /* a HIP runtime call failed */
} sla_status;

typedef enum { SLA_F32 = 0, SLA_F64 = 1 } sla_dtype;
typedef enum { SLA_I32 = 0, SLA_I64 = 1 } sla_itype;
typedef enum { SLA_INPUT_COO = 0, SLA_INPUT_CSR = 1 } sla_format;

enum {
    SLA_FLAG_CHECK_SYMMETRIC = 1u, /* reject A != A^T (bitwise) at create and set_values */
    SLA_FLAG_REORDER = 2u,         /* always solve on P A P^T, P a reverse Cuthill-McKee
                                      permutation of the pattern (see sla_csr_create) */
    SLA_FLAG_NO_REORDER = 4u       /* never reorder */
};

/* per-system outcome of a solve */
typedef enum { SLA_CONVERGED = 0, SLA_MAXIT = 1, SLA_BREAKDOWN = 2 } sla_outcome;

typedef struct {
    int32_t iterations;   /* iterations performed (the one that met the test counts) */
    int32_t status;       /* sla_outcome */
    double rel_residual;  /* ||r_k||_2 / ||b||_2 of the recursively updated residual;
                             0 when b = 0 */
} sla_info;

/* options for sla_csr_set_option */
enum {
    SLA_OPT_CHECK_INTERVAL = 1, /* iterations per host poll of the convergence flag (>= 1,
                                   default 16); results do not depend on it */
    SLA_OPT_USE_GRAPH = 2,      /* 1 (default): replay the polled iteration block as a
                                   hipGraph; 0: launch kernels one by one */
    SLA_OPT_PROFILE = 3,        /* 1: time every kernel launch of later calls with hipEvents
                                   (implies eager launches); 0 (default): off */
    SLA_OPT_RESIDENT = 4,       /* PCG solve as one cooperative kernel that keeps x, r, p
                                   and dinv on chip (same recurrence, same outcomes); a
                                   batch runs as one independent group of workgroups per
                                   system: 0 never; 1 (default) and 2 whenever
                                   applicable (the faster path wherever it applies, as
                                   measured; 2 is kept as the explicit form). Applicable: not
                                   segmented, no row longer than 128 entries, n <= 8192
                                   rows per CU of each system's share of the CUs (a
                                   multiple of 8 CUs per system, at most 256), cooperative launch
                                   available. A cooperative launch refused at solve time
                                   (not all workgroups can run at once, or another process
                                   holds the device's cooperative-launch resource) falls
                                   back to the per-step kernels; so does a solve whose
                                   bounded grid-wide wait gave up (see SLA_OPT_SPIN_LIMIT).
                                   sla_csr_get_last_path tells which path ran. */
    SLA_OPT_FUSED_UPDATE = 5,   /* 1 (default): a single system, or a batch, whose update
                                   fits one pass of the resident workgroups runs the update
                                   and the direction as one kernel (r, p, dinv stay in
                                   registers while beta is formed and broadcast); 0: two
                                   kernels. Same arithmetic either way. If the broadcast
                                   wait of the fused kernel gives up (its workgroups do not
                                   all run at once: the GPU is shared), the solve is run
                                   again with two kernels and the handle keeps to them
                                   (this option set to 0) until it is set to 1 again. */
    SLA_OPT_COOPERATIVE = 6,    /* 1 (default): the single-kernel solve is started with
                                   hipLaunchCooperativeKernel, which guarantees that all its
                                   workgroups (one per CU at most) run at once; 0: an
                                   ordinary launch of the same grid, for tools that cannot
                                   follow cooperative launches. Without the guarantee a
                                   workgroup that does not start (the GPU shared with other
                                   work) makes the others' bounded waits expire: the solve
                                   then runs again on the per-step kernels (same result;
                                   reported by sla_csr_get_last_path), never hangs. */
    SLA_OPT_SPIN_LIMIT = 7,     /* polls a bounded grid-wide wait (single-kernel solve,
                                   fused update) makes before it gives up; default 2^22
                                   (about a second), 0 .. 2^32 - 1. A wait that gives up
                                   never changes a result: the solve is run again from the
                                   start on kernels without such waits. 0 makes every wait
                                   that is not already satisfied give up at once, which
                                   exercises that path. */
    SLA_OPT_SPMV_RING = 8,      /* 1 (default): the per-step SpMV of a single system whose
                                   row tiles are all small (at most 63 rows and 253 entries,
                                   columns within 65535 of the tile's smallest) keeps four
                                   tiles' entries and two tiles' gathers in flight per
                                   wavefront; 0: one tile ahead. Same tiles, same sums, bitwise
                                   equal results. The value gradient of such a handle
                                   (sla_spmv_backward, the adjoints) follows the same
                                   setting: four tiles ahead, or one tile per wavefront;
                                   bitwise equal too. */
    SLA_OPT_FOLD_DIRECTION = 9, /* 1 (default): a per-step PCG solve with fp64 values, of a
                                   single system on such tiles (no row longer than 128
                                   entries) or of a batch whose B / (16 / value bytes) is a
                                   power of two, that is too large for the fused update
                                   (SLA_OPT_FUSED_UPDATE), forms p = z + beta p inside the
                                   SpMV, where it reads p, and applies x += alpha p there one
                                   iteration later; the update then reads r, q, dinv and
                                   writes r and z = dinv r. Two kernels and two vector
                                   passes fewer per iteration; the same recurrence, z
                                   rounded once more in fp64. 0: three kernels. fp32
                                   values never fold (z would add an fp32 rounding). */
    SLA_OPT_RESIDENT_DIA = 11,  /* 1 (default): the single-kernel solve of one system whose
                                   entries lie on 5 or 7 diagonals (offsets j - i), with
                                   at most a quarter more diagonal slots than entries (the
                                   2D and 3D stencils), holds the matrix by diagonals: the
                                   SpMV phase reads values[d][i] and p[i + offset_d], no
                                   column indices, each row summed over its diagonals in
                                   column order; 0: the row tiles. The diagonals are a second
                                   copy of the values, made at create and at every
                                   sla_csr_set_values. */
    SLA_OPT_SPMV_DIA = 12,      /* 1 (default): the per-step SpMV of such a system (the one
                                   sla_spmv, the per-step PCG solve and its folded form and
                                   BiCGStab run) reads the diagonals too: one row
                                   per lane, every load of a wavefront 512 contiguous
                                   bytes, each row summed over its diagonals in column
                                   order; 0: the row tiles. */
    SLA_OPT_RESIDENT_WALK = 10  /* the single-kernel solve's SpMV phase: 2 (default) picks by
                                   matrix size, 0 and 1 force a form. 0: each wavefront sums
                                   a contiguous run of its workgroup's tiles; 1: the
                                   workgroup's tiles interleaved over its wavefronts (w, w + 8,
                                   ...), so that a CU reads one stretch of the matrix at a
                                   time. Automatic: interleaved when the values and column
                                   indices exceed the 256 MB Infinity Cache (the matrix then
                                   streams from HBM), else contiguous. Same tiles, same sums,
                                   bitwise equal results. */
};

/* How the last sla_pcg_solve / sla_adjoint_backward / BiCGStab call on a
 * handle ran (sla_csr_get_last_path). */
enum {
    SLA_PATH_NONE = 0,          /* no solve yet */
    SLA_PATH_SINGLE_KERNEL = 1, /* the whole solve in one cooperative kernel */
    SLA_PATH_PER_STEP = 2       /* kernels per step, k steps per polled hipGraph */
};
/* why the preferred path was not the one that produced the result (bits) */
enum {
    SLA_FALLBACK_COOPERATIVE_REFUSED = 1u, /* the single-kernel solve applied, but its
                                              cooperative launch was refused */
    SLA_FALLBACK_WAIT_TIMED_OUT = 2u       /* a bounded grid-wide wait gave up and the solve
                                              was run again without that kernel */
};

/* kernel kinds reported by sla_profile_get */
enum {
    SLA_KERNEL_SPMV_DOT = 0,  /* q = A p fused with the per-block p.q partials and alpha */
    SLA_KERNEL_UPDATE = 1,    /* x += alpha p, r -= alpha q, r.z and r.r partials, beta, test
                                 (and p = z + beta p when fused, see SLA_OPT_FUSED_UPDATE) */
    SLA_KERNEL_DIRECTION = 2, /* p = z + beta p */
    SLA_KERNEL_INIT = 3,      /* r = b, x = 0, p = z, b.b and r.z */
    SLA_KERNEL_SPMV = 4,      /* plain y = A x */
    SLA_KERNEL_GRAD = 5,      /* grad_vals[k] = -lambda[row k] x[col k] */
    SLA_KERNEL_CG_RESIDENT = 6, /* a whole solve (every system of a batch) in one cooperative
                                   kernel */
    SLA_KERNEL_COUNT = 7
};

/*
 * Build a handle from COO triples or CSR arrays (SparseTensor construction).
 *  fmt = SLA_INPUT_COO: rows_or_row_ptr and cols are [nnz_in] index arrays of
 *    itypes row_itype / col_itype. Entries are ordered by (row, col) with a
 *    stable sort, and entries at one position are summed left to right in
 *    input order, in the value type. The resulting CSR is bit-identical for
 *    any thread/launch configuration.
 *  fmt = SLA_INPUT_CSR: rows_or_row_ptr is row_ptr [n+1] (row_itype), cols is
 *    [nnz_in] with columns strictly increasing inside each row; it is
 *    validated and adopted as is.
 *  values: [batch][nnz_in] of vtype, in input order.
 *  flags: SLA_FLAG_CHECK_SYMMETRIC rejects matrices that are not bitwise
 *    symmetric (for every value set).
 *  Reordering for locality: the solver may run on P A P^T with P a reverse
 *    Cuthill-McKee permutation of the pattern (computed on the host at
 *    create), which turns scattered gathers into nearby ones. Jacobi-PCG is
 *    invariant under symmetric permutation in exact arithmetic (diag(P A P^T)
 *    = P diag(A) P^T), so only the summation order inside each row changes.
 *    Every argument and result of every call stays in the caller's order and
 *    the caller's CSR (sla_csr_get returns A's arrays). Default: reorder when
 *    more than half of the SpMV tiles gather from a column range of 2^16 or
 *    more, n >= 2^16 and nnz < 2^28; SLA_FLAG_REORDER forces it (n > 1),
 *    SLA_FLAG_NO_REORDER disables it. A reordered handle holds a second copy
 *    of the matrix and its solver workspace.
 * Synchronizes `stream` before returning (validation results are read back).
 * On failure *out is set to NULL.
 */
sla_status sla_csr_create(sla_csr *out, sla_format fmt, int64_t n, int64_t nnz_in, int32_t batch,
                          sla_itype row_itype, const void *rows_or_row_ptr,
                          sla_itype col_itype, const void *cols,
                          sla_dtype vtype, const void *values, uint32_t flags, void *stream);

/*
 * A list of independent systems with distinct patterns solved together
 * (torch-sla's SparseTensorList: matrices of different patterns batched, the
 * tensor-types passage), held as one block-diagonal matrix. The caller passes
 * that matrix exactly as to sla_csr_create (batch 1; indices already offset
 * so that system q owns rows and columns [seg_rows[q], seg_rows[q+1])) and
 * seg_rows: host [nseg+1], seg_rows[0] = 0, strictly increasing,
 * seg_rows[nseg] = n. An entry outside its row's diagonal block gives
 * SLA_ERR_INDEX_RANGE. sla_spmv multiplies the whole block-diagonal matrix;
 * sla_pcg_solve and sla_adjoint_backward run every system's own Jacobi-PCG
 * (its own step sizes, stopping test and iteration count, as if solved alone)
 * and fill info[0..nseg). SLA_FLAG_REORDER is rejected (segments are never
 * reordered); the single-kernel solve and the fused update do not apply.
 */
sla_status sla_csr_create_segmented(sla_csr *out, sla_format fmt, int64_t n, int64_t nnz_in,
                                    sla_itype row_itype, const void *rows_or_row_ptr,
                                    sla_itype col_itype, const void *cols, sla_dtype vtype,
                                    const void *values, int32_t nseg, const int64_t *seg_rows,
                                    uint32_t flags, void *stream);

/* Segments of a handle (host outputs): *nseg = 0 for an unsegmented handle;
 * seg_rows (host [nseg+1], may be NULL) receives the row boundaries. */
sla_status sla_csr_get_segments(sla_csr h, int32_t *nseg, int64_t *seg_rows);

/* Replace the values (same pattern, same input order and count as at create):
 * values [batch][nnz_in] of the handle's vtype. Duplicate positions are merged
 * exactly as at create. Synchronizes `stream`. */
sla_status sla_csr_set_values(sla_csr h, const void *values, void *stream);

/* Shapes and the handle's index arrays (host outputs; any may be NULL).
 * row_ptr has itype *row_itype (SLA_I32 when nnz < 2^31 for COO input, else
 * the input's), col_idx is int32 [nnz]. slot (int64 [nnz_in]) maps input entry
 * e to the CSR position it was merged into; it is NULL when that map is the
 * identity (sorted, duplicate-free input). The pointers stay valid until
 * destroy and must not be written. */
sla_status sla_csr_get(sla_csr h, int64_t *n, int64_t *nnz, int64_t *nnz_in, int32_t *batch,
                       int32_t *vtype, int32_t *row_itype, const void **row_ptr,
                       const void **col_idx, const int64_t **slot);

/* Copy the pattern into caller buffers (any may be NULL): row_ptr_out [n+1]
 * of the handle's row itype, col_idx_out int32 [nnz], slot_out int64 [nnz_in]
 * (written as 0..nnz_in-1 when the map is the identity). Asynchronous. */
sla_status sla_csr_get_pattern(sla_csr h, void *row_ptr_out, void *col_idx_out, int64_t *slot_out,
                               void *stream);

/* Copy the CSR values out as [batch][nnz] (CSR order) of the handle's vtype. */
sla_status sla_csr_get_values(sla_csr h, void *values_out, void *stream);

/* Gather a CSR-ordered array [batch][nnz] to input order [batch][nnz_in]:
 * out[b][e] = in[b][slot[e]] (duplicates each receive their merged entry's value). */
sla_status sla_csr_gather_to_input(sla_csr h, const void *csr_order, void *input_order,
                                   void *stream);

/* Set one option (SLA_OPT_*) on the handle. It also applies to the kernels
 * the handle runs on its behalf: the reordered solver handle and the A^T
 * built for sla_spmv_backward / sla_bicgstab_adjoint (profiling aside: A^T's
 * launches are not profiled). Unknown keys and out-of-range values return
 * SLA_ERR_INVALID_ARG. */
sla_status sla_csr_set_option(sla_csr h, int32_t key, int64_t value);

/* Sparse matrix-vector product y = A x for every batch member (.matvec).
 * x, y: [batch][n] of the handle's vtype; must not alias. fp32 handles form
 * products and sums in fp64 and round once. Asynchronous. */
sla_status sla_spmv(sla_csr h, const void *x, void *y, void *stream);

/* Backward of y = A x (.matvec under autograd; torch-sla counts matvec among
 * the operations that carry gradients, tensor-types passage and Table 1) for
 * an upstream gradient grad_y = dL/dy:
 *   grad_x = A^T grad_y                          [batch][n], or NULL
 *   grad_vals[b][k] = grad_y[b][row k] x[b][col k]   [batch][nnz], CSR order, or NULL
 * x, grad_y: [batch][n]. grad_x must not alias x or grad_y. fp32 handles form
 * products and sums in fp64. Asynchronous. A handle created with
 * SLA_FLAG_CHECK_SYMMETRIC uses A itself for A^T; otherwise the first call
 * builds a handle of A^T on the device (a stable radix sort of the entries by
 * column; allocates, once per handle) and later calls only refresh its values
 * after sla_csr_set_values.
 * grad_vals reaches input order through sla_csr_gather_to_input. */
sla_status sla_spmv_backward(sla_csr h, const void *x, const void *grad_y, void *grad_x,
                             void *grad_vals, void *stream);

/*
 * Jacobi-preconditioned CG from x0 = 0 for every batch member (.solve):
 *   r = b, z = D^-1 r, p = z; per iteration q = A p, alpha = r.z / p.q,
 *   x += alpha p, r -= alpha q, stop when ||r|| <= tol ||b||, else
 *   beta = r'.z' / r.z, p = z' + beta p.
 * Each system stops on its own test; p.q <= 0 or non-finite ends it with
 * SLA_BREAKDOWN (A not SPD). b, x: [batch][n]; info: host [batch] ([nseg] for a
 * segmented handle).
 * maxit >= 0, tol >= 0 (tol = 0 runs exactly maxit iterations).
 * Returns SLA_ERR_BAD_DIAGONAL if some d_i is missing, <= 0 or not finite.
 * fp32 handles store vectors in fp32 and compute in fp64.
 * Blocks the host until the solve has finished (info is filled).
 */
sla_status sla_pcg_solve(sla_csr h, const void *b, void *x, double tol, int32_t maxit,
                         sla_info *info, void *stream);

/*
 * Adjoint backward of x = A^{-1} b for upstream grad_x = dL/dx: solves
 * A lambda = grad_x with the same PCG (A symmetric, so A^T = A), then
 *   grad_b = lambda                                  ([batch][n], or NULL)
 *   grad_vals[b][k] = -lambda[b][row(k)] * x[b][col(k)] ([batch][nnz] in CSR
 *                                                        order, or NULL)
 * x is the forward solution [batch][n]. info (host [batch]) reports the
 * adjoint solve. Blocks the host until done.
 */
sla_status sla_adjoint_backward(sla_csr h, const void *x, const void *grad_x, void *grad_b,
                                void *grad_vals, double tol, int32_t maxit, sla_info *info,
                                void *stream);

/*
 * Jacobi-PCG for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): one
 * fp64 system given directly as CSR arrays, no handle, no allocation. The
 * recurrence, stopping test and outcomes are those of sla_pcg_solve (the
 * same results up to rounding order: iteration counts within 2).
 *  n: 1 <= n <= SLA_NOALLOC_MAX_ROWS (2^21), else SLA_ERR_INVALID_ARG;
 *  0 <= nnz < 2^31. row_ptr int32 [n+1] (0 .. nnz, non-decreasing), col_idx
 *  int32 [nnz] (in [0, n), strictly increasing inside a row), values fp64
 *  [nnz]: checked on the device first (SLA_ERR_INVALID_CSR,
 *  SLA_ERR_INDEX_RANGE; SLA_ERR_BAD_DIAGONAL unless every diagonal entry is
 *  present, positive and finite). b, x: fp64 [n]; x receives the solution
 *  and must not alias b. info: host [1].
 *  Workspace: a fixed array of this library in device memory, 64 MiB for
 *  four vectors of 2^21 doubles plus 58 KiB for the reductions' partials and
 *  counters and the solve's scalars, which every GPU the library runs on
 *  holds until the process ends. Every call on one GPU uses that
 *  GPU's array: calls that overlap on one GPU (other host threads, other
 *  streams) race and give wrong results. Work is ordered on `stream`; the
 *  call blocks the host until the solve has finished (it reads the running
 *  flag every 16 iterations). The product is the general one-lane-per-row
 *  SpMV, slower than a handle's tiled one.
 */
#define SLA_NOALLOC_MAX_ROWS (1 << 21)
sla_status sla_pcg_solve_noalloc(int64_t n, int64_t nnz, const int32_t *row_ptr,
                                 const int32_t *col_idx, const double *values, const double *b,
                                 double *x, double tol, int32_t maxit, sla_info *info,
                                 void *stream);

/*
 * Jacobi-preconditioned BiCGStab from x0 = 0 for a general (non-symmetric)
 * system. torch-sla lists BiCGStab beside CG in its pytorch-native backend
 * (backend list of the API section; the distributed section: the CG template
 * with more inner products). The recurrence is van der Vorst's preconditioned
 * BiCGStab with D = diag(A) and shadow residual r^ = b:
 *   p = r (first) or r + beta (p - omega v); p^ = D^-1 p; v = A p^;
 *   alpha = r^.r / r^.v; s = r - alpha v; if ||s|| <= tol ||b||: x += alpha p^,
 *   converged; s^ = D^-1 s; t = A s^; omega = t.s / t.t;
 *   x += alpha p^ + omega s^; r = s - omega t; stop when ||r|| <= tol ||b||;
 *   beta = (r^.r' / r^.r)(alpha / omega).
 * SLA_BREAKDOWN when r^.v, t.t, omega or the new r^.r is exactly 0 or not
 * finite: at r^.v, x keeps its value; at omega, x takes the half step x +
 * alpha p^. Iterations count the steps started (a half step counts as one).
 * One system per handle: batch 1 and not segmented (else
 * SLA_ERR_INVALID_ARG). b, x: [n] device vectors; info: host [1].
 * maxit >= 0, tol >= 0. Returns SLA_ERR_BAD_DIAGONAL if some d_i is missing,
 * zero or not finite (negative entries are fine). fp32 handles store vectors
 * in fp32 and compute in fp64. Blocks the host until the solve has finished.
 * Profiling (SLA_OPT_PROFILE) books the two SpMVs under SLA_KERNEL_SPMV_DOT,
 * the half-step and update kernels under SLA_KERNEL_UPDATE and the p, p^
 * kernel under SLA_KERNEL_DIRECTION.
 */
sla_status sla_bicgstab_solve(sla_csr h, const void *b, void *x, double tol, int32_t maxit,
                              sla_info *info, void *stream);

/*
 * Adjoint backward of x = A^{-1} b solved by BiCGStab, for upstream grad_x =
 * dL/dx (the adjoint of the distributed section, with the adjoint system
 * A^T lambda = dL/dx solved by the same BiCGStab): then
 *   grad_b = lambda                              ([n], or NULL)
 *   grad_vals[k] = -lambda[row(k)] * x[col(k)]    ([nnz] in CSR order, or NULL)
 * A^T is the handle itself when it was created with SLA_FLAG_CHECK_SYMMETRIC;
 * otherwise the first call builds a handle of A^T on the device (values
 * gathered, and refreshed after set_values), as sla_spmv_backward does. x is the forward solution [n]; grad_b must not
 * alias x or grad_x. info (host [1]) reports the adjoint solve. Same
 * restrictions and errors as sla_bicgstab_solve. Blocks the host until done.
 */
sla_status sla_bicgstab_adjoint(sla_csr h, const void *x, const void *grad_x, void *grad_b,
                                void *grad_vals, double tol, int32_t maxit, sla_info *info,
                                void *stream);

/* How the solver holds the matrix (host outputs; any may be NULL): reordered
 * = 1 when it runs on P A P^T; narrow_columns = 1 when every SpMV tile reads
 * 16-bit column offsets, 2 when in addition every tile is small enough for
 * the four-tile pipeline of SLA_OPT_SPMV_RING; tiles and long_rows count the
 * SpMV's short-row tiles and its rows longer than 128 entries. */
sla_status sla_csr_get_layout(sla_csr h, int32_t *reordered, int32_t *narrow_columns,
                              int64_t *tiles, int64_t *long_rows);

/* How the last solve on the handle ran (host outputs; either may be NULL):
 * *path an SLA_PATH_* value, *fallbacks a mask of SLA_FALLBACK_* bits (0
 * when the preferred path ran). Results do not depend on the path. */
sla_status sla_csr_get_last_path(sla_csr h, int32_t *path, uint32_t *fallbacks);

/* Diagonals the solver holds the matrix by (host outputs; either may be
 * NULL; for a reordered handle, of P A P^T): *ndiag = their number for the
 * single-kernel solve once a solve has built its plan and
 * SLA_OPT_RESIDENT_DIA applies, else 0 (row tiles, or no single-kernel solve
 * yet); *per_step = their number where the per-step SpMV reads them
 * (SLA_OPT_SPMV_DIA), else 0. */
sla_status sla_csr_get_diagonals(sla_csr h, int32_t *ndiag, int32_t *per_step);

/* Accumulated kernel timings of calls made while SLA_OPT_PROFILE was on
 * (host outputs): number of launches and total milliseconds per kind. */
sla_status sla_profile_get(sla_csr h, int32_t kind, int64_t *launches, double *total_ms);
sla_status sla_profile_reset(sla_csr h);

/* Device bytes owned by the handle (matrix, index maps, solve workspace). */
sla_status sla_csr_memory(sla_csr h, int64_t *bytes);

void sla_csr_destroy(sla_csr h);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *sla_last_error(void);

/* Library version string. */
const char *sla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */

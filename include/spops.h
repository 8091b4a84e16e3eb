/*
 * spops.h -- C ABI of libspops, unstructured CSR sparse-dense products on
 * AMD Instinct MI355X (gfx950).
 *
 * Operations (all defined on the spops README, IST-DASLab):
 *   spops_spmm            section "Sparse Matrix Multiplication (SpMM)"
 *   spops_sddmm           section "Sampled Dense-Dense Matrix Multiplication (SDDMM)"
 *   spops_csr_add         section "Sparse Addition"
 *   spops_csr_transpose   section "CSR Transpose" (also as a permutation of
 *                         the values: spops_csr_transpose_permutation and
 *                         spops_permute_values)
 *   spops_sort_rows_by_nnz  the row_idx list of section "Usage"
 * and, built on spops_spmm, a conjugate-gradient solver (spops_cg; the
 * torchsparsegradutils README, section "Built-in Iterative Solvers"), and a
 * masked Adam step for trained value vectors (spops_masked_adam; the
 * SparseAdam page of tensorplay.optim), and rows with 2-bit delta-coded
 * columns with their SpMV (spops_delta_*; the UST news page, sections
 * "Formatos menos comuns" and "Performance").
 *
 * Sparse layout (section "Usage"): an m x n matrix with nnz stored entries is
 *   values[nnz]        the stored values (f32, f16 or bf16);
 *   row_offsets[m+1]   int32; row r owns positions [row_offsets[r], row_offsets[r+1]);
 *   col_idx[nnz]       column of each stored value; int16 when n <= 32767, else int32;
 *   row_idx[m]         a permutation of 0..m-1 ordering the rows by entry count.
 * Section "Important Notes" of the same page asks for contiguous inputs,
 * int32 row offsets and int16 for the other index lists; int32 is accepted
 * wherever 16 bits cannot address the extent (n or m above 32767).
 *
 * Conventions shared by every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller (e.g. a
 *     torch tensor's storage).  Dense matrices are row-major with an explicit
 *     leading dimension (elements between consecutive rows) and unit stride
 *     inside a row.  Element pointers must be aligned to their element size.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the default stream).  Execute calls never allocate device memory and
 *     never synchronize; plan-creation calls do both and say so, and the
 *     solver spops_cg synchronizes at its convergence checks.
 *   - Validation reads host-side metadata only (sizes, types, pointers).  On
 *     any error status nothing is launched and no output is written.
 *     Device-resident index data is not validated: indices outside their
 *     range never cause out-of-bounds accesses (kernels skip or clamp them)
 *     but the results for such entries are unspecified.
 *   - Duplicate (row, column) entries inside a row are a precondition
 *     violation for spmm/sddmm/csr_add (results unspecified).
 *   - Floating-point accumulation is in fp32.  Results are deterministic: the
 *     same call on the same inputs gives bitwise-identical outputs.
 *   - Asynchronous device errors surface at the caller's next synchronization.
 *   - Every function is reentrant.  Two calls whose outputs overlap race.
 */
#ifndef SPOPS_H
#define SPOPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPOPS_ABI_VERSION 1

typedef enum spops_status {
  SPOPS_OK = 0,
  SPOPS_ERR_NULL = 1,          /* a required pointer is NULL */
  SPOPS_ERR_SHAPE = 2,         /* negative, inconsistent or too large sizes / leading dims */
  SPOPS_ERR_DTYPE = 3,         /* unknown dtype or unsupported combination */
  SPOPS_ERR_INDEX_WIDTH = 4,   /* int16 index list whose extent exceeds 32767 */
  SPOPS_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than the size query returned */
  SPOPS_ERR_UNSUPPORTED = 6,   /* valid request this build does not implement */
  SPOPS_ERR_PLAN = 7,          /* plan built for a different mask */
  SPOPS_ERR_HIP = 8,           /* a HIP runtime call or kernel launch failed */
  SPOPS_ERR_ARGUMENT = 9,      /* a scalar argument (tolerance, rate, ...) out of its range */
  SPOPS_ERR_INDEX_ORDER = 10,  /* columns not strictly ascending inside a row, or out of range */
  SPOPS_ERR_INVALID_INDEX = 11 /* spops_validate_csr found invalid index data */
} spops_status;

typedef enum spops_dtype { SPOPS_F32 = 0, SPOPS_F16 = 1, SPOPS_BF16 = 2 } spops_dtype;
typedef enum spops_itype { SPOPS_I16 = 0, SPOPS_I32 = 1 } spops_itype;

/* The two SDDMM kernels of section "Sampled Dense-Dense Matrix Multiplication
 * (SDDMM)": the general one (named after sputnik on the page) and the
 * structure-aware one, which is the default there. */
typedef enum spops_sddmm_backend {
  SPOPS_SDDMM_STRUCTURE_AWARE = 0,
  SPOPS_SDDMM_GENERAL = 1
} spops_sddmm_backend;

/* A CSR matrix (layout above).  `values` may be NULL where only the pattern
 * is used (an SDDMM output mask, a pattern-only transpose).  `row_idx` may be
 * NULL where an entry point says so; when given it must be a permutation of
 * 0..rows-1 (any order is correct; most-entries-first balances the work). */
typedef struct spops_csr {
  int64_t rows, cols, nnz;
  spops_dtype val_type;          /* ignored when values == NULL */
  spops_itype col_type;          /* SPOPS_I16 requires cols <= 32767 */
  spops_itype row_idx_type;      /* SPOPS_I16 requires rows <= 32767 */
  const void* values;            /* [nnz] */
  const int32_t* row_offsets;    /* [rows+1]: [0] = 0, nondecreasing, [rows] = nnz */
  const void* row_idx;           /* [rows] */
  const void* col_idx;           /* [nnz]; need not be sorted within a row */
} spops_csr;

/* ABI version (SPOPS_ABI_VERSION) and a static description of a status. */
int spops_abi_version(void);
const char* spops_status_string(spops_status status);

/* Process-wide switches, read by every later call (0 = the default for all).
 * They select alternative code paths for tests and tuning; results are the
 * same definition whatever they hold.
 *   SPOPS_OPT_SPMM_POINTER_LOADS    nonzero: SpMM reads its operands through
 *       plain pointers (the path otherwise taken for operands of 2 GiB and
 *       more).
 *   SPOPS_OPT_TRANSPOSE_FORCE_SCAN  nonzero: csr_transpose scans its count
 *       table even for inputs whose scatter could derive its own offsets.
 *   SPOPS_OPT_TRANSPOSE_WIDE_RECORDS  nonzero: csr_transpose's first pass
 *       writes 16-byte records even where 8-byte ones fit.
 *   SPOPS_OPT_SDDMM_BUCKETS  1..8: column buckets of the structure-aware
 *       remainder in plans built afterwards (0: chosen per mask).
 *   SPOPS_OPT_SDDMM_SPLITS   1..16: K splits of the structure-aware dense
 *       tiles (0: chosen per plan and K); changes spops_sddmm_workspace_size.
 *   SPOPS_OPT_SDDMM_REST_SPLIT  1..8 or 16: pieces of K for the structure-aware
 *       remainder (1: no split; 0: chosen from the size of BT); changes
 *       spops_sddmm_workspace_size.
 * spops_set_option returns SPOPS_ERR_UNSUPPORTED for an unknown option and
 * SPOPS_ERR_ARGUMENT for a negative value.  Calls running concurrently with
 * a change may see either value. */
typedef enum spops_option {
  SPOPS_OPT_SPMM_POINTER_LOADS = 0,
  SPOPS_OPT_TRANSPOSE_FORCE_SCAN = 1,
  SPOPS_OPT_TRANSPOSE_WIDE_RECORDS = 2,
  SPOPS_OPT_SDDMM_BUCKETS = 3,
  SPOPS_OPT_SDDMM_SPLITS = 4,
  SPOPS_OPT_SDDMM_REST_SPLIT = 5
} spops_option;
spops_status spops_set_option(spops_option option, int64_t value);
spops_status spops_get_option(spops_option option, int64_t* value);

/* ------------------------------------------------------------------ SpMM --
 * Section "Sparse Matrix Multiplication (SpMM)": C = A * B.
 *   A:  rows x cols CSR with values; row_idx required.
 *   B:  cols x N dense, element type b_type == A->val_type, leading dim ldb >= N.
 *   C:  rows x N dense, written (not accumulated), leading dim ldc >= N;
 *       c_type is SPOPS_F32 or b_type (then the fp32 sum is rounded to
 *       nearest-even once).  Rows of A without entries give zero rows.
 *   C[r][j] = sum over the entries (r, c, v) of A of v * B[c][j].
 *   plan (nullable): a schedule from spops_spmm_plan_create for A.  Without
 *   one no row is split, which is correct but slow for rows with thousands
 *   of entries.  With one, `workspace` must hold
 *   spops_spmm_workspace_size(plan, N) bytes (may be 0, then NULL is fine). */
typedef struct spops_spmm_plan spops_spmm_plan;

spops_status spops_spmm(const spops_csr* A, const void* B, spops_dtype b_type, int64_t N,
                        int64_t ldb, void* C, spops_dtype c_type, int64_t ldc,
                        const spops_spmm_plan* plan, void* workspace, size_t workspace_bytes,
                        void* hip_stream);

/* Builds the row-splitting schedule for A's pattern (row_offsets, row_idx):
 * rows longer than one chunk are split into fixed chunks whose fp32 partial
 * rows are summed in chunk order, so results stay deterministic.  Allocates
 * device memory and synchronizes `hip_stream`.  The plan stays valid while
 * A's row_offsets and row_idx contents are unchanged; it serves any B, N and
 * dtype. */
spops_status spops_spmm_plan_create(const spops_csr* A, void* hip_stream,
                                    spops_spmm_plan** plan);
spops_status spops_spmm_plan_destroy(spops_spmm_plan* plan);
/* Bytes of workspace spops_spmm needs with this plan for N columns. */
spops_status spops_spmm_workspace_size(const spops_spmm_plan* plan, int64_t N, size_t* bytes);
/* Plan summary: chunks = workgroups the plan gives to long rows (every row
 * of more than 128 entries, or of more than 64 when the row lengths are
 * skewed -- longest row above twice the mean plus 32 -- and at most 1/32 of
 * the rows have 65 to 128 entries), each covering up to a chunk length of
 * entries: the longest row rounded up to a power of two, at most 4096, when
 * that still gives at least 128 chunks, else 512; split_rows = long rows of
 * more than one chunk (their partial rows are added afterwards in chunk
 * order); max_row_nnz = longest row. */
spops_status spops_spmm_plan_info(const spops_spmm_plan* plan, int64_t* split_rows,
                                  int64_t* chunks, int64_t* max_row_nnz);

/* ----------------------------------------------------------------- SDDMM --
 * Section "Sampled Dense-Dense Matrix Multiplication (SDDMM)":
 *   out[p] = sum_k A[r][k] * BT[c][k]  for every stored position p = (r, c)
 *   of `mask` (values and row_idx not used), in the mask's CSR order.
 *   A:  mask->rows x K dense, leading dim lda >= K.
 *   BT: mask->cols x K dense (B transposed), leading dim ldbt >= K.
 *   A and BT share in_type; out_type is SPOPS_F32 or in_type.
 *   backend SPOPS_SDDMM_GENERAL: one kernel for any pattern; `plan` ignored.
 *   backend SPOPS_SDDMM_STRUCTURE_AWARE: runs the rows and columns where the
 *   mask's entries cluster as dense tiles on the matrix cores and the rest
 *   with the general kernel.  The partition comes from `plan` (see
 *   spops_sddmm_plan_create); with plan == NULL it is built inside the call,
 *   on the stream, in the caller's workspace, with the default density
 *   threshold (slower than reusing a plan, but it neither allocates nor
 *   synchronizes, so it can be captured in a HIP graph).  The dense tiles
 *   need 16-bit inputs, K a multiple of 8, lda and ldbt multiples of 8,
 *   16-byte aligned A and BT, and rows x leading dimension x 2 bytes under
 *   2 GiB for each of A and BT; other calls run the general kernel (with a
 *   plan that found no tiles, over the plan's column buckets).
 *   workspace: spops_sddmm_workspace_size bytes (NULL when that is 0),
 *   256-byte aligned; its contents on entry do not matter.  Too small:
 *   SPOPS_ERR_WORKSPACE.  Both backends compute the same values up to fp32
 *   summation order. */
typedef struct spops_sddmm_plan spops_sddmm_plan;

spops_status spops_sddmm(const spops_csr* mask, const void* A, int64_t K, int64_t lda,
                         const void* BT, int64_t ldbt, spops_dtype in_type, void* out_values,
                         spops_dtype out_type, spops_sddmm_backend backend,
                         const spops_sddmm_plan* plan, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/* Workspace of spops_sddmm for this mask, K, input type, backend and plan:
 *   general backend, or inputs the dense tiles cannot take: 0;
 *   structure-aware with a plan: fp32 partial sums when the plan splits K
 *     across workgroups (S splits x entries in tiles x 4 bytes; 0 without
 *     a split);
 *   structure-aware without a plan: the plan built inside the call (a few
 *     int32 arrays of the mask's sizes and entry count). */
spops_status spops_sddmm_workspace_size(const spops_csr* mask, int64_t K, spops_dtype in_type,
                                        spops_sddmm_backend backend,
                                        const spops_sddmm_plan* plan, size_t* bytes);

/* Finds the clustered rows/columns of the mask and partitions its entries.
 * A row is dense when its entry count is at least tau * cols; a column is
 * dense when, over the remaining rows, its count is at least tau * rows.
 * tau <= 0 selects the default: tau = 0.02, and a dense row or column also
 * holds at least 128 entries (one tile's width), so that small or uniform
 * masks stay on the general kernel.  tau > 1 disables the dense tiles (all
 * entries go to the general kernel).  Allocates, synchronizes.  Valid while
 * the mask's row_offsets / col_idx contents are unchanged. */
spops_status spops_sddmm_plan_create(const spops_csr* mask, double tau, void* hip_stream,
                                     spops_sddmm_plan** plan);
spops_status spops_sddmm_plan_destroy(spops_sddmm_plan* plan);
/* Plan summary: dense rows, dense columns, entries covered by dense tiles,
 * entries left to the general kernel, number of dense tiles. */
spops_status spops_sddmm_plan_info(const spops_sddmm_plan* plan, int64_t* dense_rows,
                                   int64_t* dense_cols, int64_t* tiled_nnz,
                                   int64_t* rest_nnz, int64_t* tiles);

/* ------------------------------------------------------------ validation --
 * Checks a CSR's device-resident index data against the layout of section
 * "Usage" (the operations themselves do not: they only avoid out-of-bounds
 * accesses, and the results for invalid data are unspecified):
 *   SPOPS_INVALID_OFFSETS    row_offsets[0] != 0, row_offsets[rows] != nnz,
 *                            or a decreasing pair;
 *   SPOPS_INVALID_COLUMN     a column index outside [0, cols);
 *   SPOPS_INVALID_ROW_IDX    row_idx (checked when A->row_idx is not NULL)
 *                            is not a permutation of 0..rows-1;
 *   SPOPS_INVALID_DUPLICATE  a (row, column) pair stored twice (checked when
 *                            check_duplicates is nonzero and offsets and
 *                            columns are valid).
 * Values are not read.  Every device read stays inside the lengths the
 * descriptor gives.  Returns SPOPS_OK for valid data, SPOPS_ERR_INVALID_INDEX
 * when any check fails, with the failed checks OR-ed into *findings
 * (nullable).  workspace: spops_validate_csr_workspace_size bytes, 256-byte
 * aligned, contents on entry irrelevant.  Synchronizes hip_stream. */
typedef enum spops_invalid_flags {
  SPOPS_INVALID_OFFSETS = 1,
  SPOPS_INVALID_COLUMN = 2,
  SPOPS_INVALID_ROW_IDX = 4,
  SPOPS_INVALID_DUPLICATE = 8
} spops_invalid_flags;
spops_status spops_validate_csr_workspace_size(int64_t rows, int64_t cols, int64_t nnz,
                                               size_t* bytes);
spops_status spops_validate_csr(const spops_csr* A, int check_duplicates, void* workspace,
                                size_t workspace_bytes, uint32_t* findings, void* hip_stream);

/* --------------------------------------------------------------- csr_add --
 * Section "Sparse Addition", in place on the dense operand:
 *   W[r][c] = round(W[r][c] + v)  for every entry (r, c, v) of A;
 * every other element of W keeps its bits.  w_type == A->val_type; the sum
 * is formed in fp32 and rounded once to w_type (nearest-even), which equals
 * the correctly rounded sum for f32, f16 and bf16.  W is A->rows x A->cols
 * with leading dim ldw >= A->cols.  row_idx is not used (may be NULL). */
spops_status spops_csr_add(const spops_csr* A, void* W, spops_dtype w_type, int64_t ldw,
                           void* hip_stream);

/* --------------------------------------------------------- csr_transpose --
 * Section "CSR Transpose": A^T (cols x rows) as a CSR, i.e. the CSC of A.
 *   out_row_offsets[cols+1], out_col_idx[nnz] (type out_col_type; SPOPS_I16
 *   requires rows <= 32767), out_values[nnz] (same dtype as A; ignored when
 *   A->values is NULL).  Entries of each output row appear in ascending
 *   source-row order (a stable sort by column), so the result is unique and
 *   independent of the order of columns inside A's rows.  Index outputs are
 *   exact; values are moved bit for bit.  row_idx is not used.
 *   The workspace (size from spops_csr_transpose_workspace_size) is scratch
 *   for the radix passes; its contents on entry do not matter. */
spops_status spops_csr_transpose_workspace_size(int64_t rows, int64_t cols, int64_t nnz,
                                                size_t* bytes);
spops_status spops_csr_transpose(const spops_csr* A, void* out_values, int32_t* out_row_offsets,
                                 void* out_col_idx, spops_itype out_col_type, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);

/* The permutation spops_csr_transpose applies to the values (section "CSR
 * Transpose"), for a pattern whose values change while its positions do not
 * (the transposed product in a sparse layer's backward pass):
 *   out_src[j] = index among A's stored entries of A^T's stored entry j;
 * out_row_offsets and out_col_idx are written as by spops_csr_transpose.
 * A->values is not used.  Then A^T's values for any values of A are one
 * spops_permute_values call.  workspace:
 * spops_csr_transpose_permutation_workspace_size bytes, 256-byte aligned. */
spops_status spops_csr_transpose_permutation_workspace_size(int64_t rows, int64_t cols,
                                                            int64_t nnz, size_t* bytes);
spops_status spops_csr_transpose_permutation(const spops_csr* A, int32_t* out_src,
                                             int32_t* out_row_offsets, void* out_col_idx,
                                             spops_itype out_col_type, void* workspace,
                                             size_t workspace_bytes, void* hip_stream);

/* out[j] = in[src[j]] for 0 <= j < n, elements of `type` moved bit for bit
 * (with src from spops_csr_transpose_permutation: A^T's values from A's).
 * in has n_in elements; an src[j] outside [0, n_in) writes zero bits.
 * in and out must not overlap. */
spops_status spops_permute_values(const void* in, int64_t n_in, spops_dtype type,
                                  const int32_t* src, int64_t n, void* out, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * transpose with its scratch in a fixed array inside the library instead of
 * a workspace argument.  Inputs and outputs as for spops_csr_transpose.
 * Allocates nothing and calls no allocating routine; the array (32 MiB, its
 * size from spops_csr_transpose_noalloc_limit) exists once per GPU and is
 * held until the process ends.  Inputs whose transpose needs more scratch
 * than that (spops_csr_transpose_workspace_size) are rejected with
 * SPOPS_ERR_WORKSPACE before anything is launched.  Every call on one GPU
 * uses that GPU's array: calls that overlap in time on the same GPU (other
 * streams, other threads) race and give undefined results; calls in order
 * on one stream are safe.  The array's contents on entry do not matter. */
spops_status spops_csr_transpose_noalloc(const spops_csr* A, void* out_values,
                                         int32_t* out_row_offsets, void* out_col_idx,
                                         spops_itype out_col_type, void* hip_stream);
spops_status spops_csr_transpose_noalloc_limit(size_t* bytes);

/* ------------------------------------------------------------ row order --
 * The row_idx list of section "Usage": rows sorted by entry count, most
 * entries first, equal counts in ascending row order (the page leaves
 * direction and ties open; this is the reading taken).  `cols` bounds every
 * row's count (counts are clamped to it).  row_idx_type SPOPS_I16 requires
 * rows <= 32767. */
spops_status spops_sort_rows_by_nnz_workspace_size(int64_t rows, int64_t cols, size_t* bytes);
spops_status spops_sort_rows_by_nnz(const int32_t* row_offsets, int64_t rows, int64_t cols,
                                    void* row_idx, spops_itype row_idx_type, void* workspace,
                                    size_t workspace_bytes, void* hip_stream);

/* --------------------------------------------------- conjugate gradients --
 * Solves A x = b for a symmetric positive definite A with conjugate
 * gradients.  The torchsparsegradutils README lists a CG solver among its
 * built-in iterative solvers ("Built-in Iterative Solvers") and calls a
 * sparse solve with it and a tolerance ("Generic solve"); the page gives no
 * steps, so the method is that of Hestenes and Stiefel (1952):
 *   r = b - A x, p = r; per iteration q = A p (the SpMM above with N = 1),
 *   alpha = r.r / p.q, x += alpha p, r -= alpha q,
 *   beta = r'.r' / r.r, p = r' + beta p.
 *   A:  rows x rows CSR, f32 values, row_idx required (as for spops_spmm).
 *   b:  [rows] f32.  x: [rows] f32, the initial guess on entry, the solution
 *       on exit.  Vectors are f32; dot products and the scalar steps are
 *       float64, summed in a fixed order (deterministic).
 *   Stops after the first iteration whose recursive residual has
 *   r.r <= rtol^2 * b.b, or after max_iter iterations, or (without writing
 *   x) when p.q is not positive (A is not positive definite).
 *   check_every (>= 1): iterations enqueued between two convergence checks;
 *   each check reads the solver state back and synchronizes hip_stream, so
 *   this call BLOCKS until it returns.  Iterations enqueued past convergence
 *   leave x unchanged.
 *   plan (nullable): spops_spmm_plan_create's plan for A.
 *   iters_out, rel_resid_out (nullable): iterations done and sqrt(r.r / b.b)
 *   (0 when b = 0).
 *   workspace: spops_cg_workspace_size bytes (vectors r, p, q, partial sums,
 *   solver state, the SpMM's workspace); contents on entry do not matter.
 *   rtol < 0 or NaN, max_iter < 0, check_every < 1 give SPOPS_ERR_ARGUMENT;
 *   rows != cols SPOPS_ERR_SHAPE; values other than f32 SPOPS_ERR_DTYPE. */
spops_status spops_cg_workspace_size(const spops_csr* A, const spops_spmm_plan* plan,
                                     size_t* bytes);
spops_status spops_cg(const spops_csr* A, const void* b, void* x, double rtol, int64_t max_iter,
                      int64_t check_every, const spops_spmm_plan* plan, void* workspace,
                      size_t workspace_bytes, int64_t* iters_out, double* rel_resid_out,
                      void* hip_stream);

/* ----------------------------------------------------------- masked Adam --
 * One step of the masked Adam of the SparseAdam page (tensorplay.optim):
 * only the positions where the gradient is materialized update their
 * moments and their value; a materialized zero still counts.  The step is
 * Adam's (Kingma and Ba, 2015, in the efficient form of their Section 2):
 *   m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
 *   value -= alpha_t m / (sqrt(v) + eps),
 *   alpha_t = lr sqrt(1 - beta2^step) / (1 - beta1^step),
 * with g negated when `maximize` is nonzero.
 *   values:   [nnz] trained values (val_type f32, f16 or bf16), updated in
 *             place (fp32 arithmetic, rounded once to val_type).
 *   exp_avg, exp_avg_sq: [nnz] f32 moments, updated in place (zeros before
 *             the first step).
 *   grad:     [ngrad] gradient in val_type.  positions == NULL: every value
 *             has a gradient entry (ngrad must equal nnz).  Otherwise
 *             positions[ngrad] (int32) names the value of each entry; they
 *             must be distinct (a coalesced sparse gradient; duplicates race)
 *             and those outside [0, nnz) are skipped.
 *   step:     the step number t >= 1 (the caller counts steps).
 *   lr >= 0, 0 <= beta1 < 1, 0 <= beta2 < 1, eps >= 0, all finite, else
 *   SPOPS_ERR_ARGUMENT (step < 1 too). */
spops_status spops_masked_adam(void* values, spops_dtype val_type, int64_t nnz, const void* grad,
                               const int32_t* positions, int64_t ngrad, float* exp_avg,
                               float* exp_avg_sq, int64_t step, double lr, double beta1,
                               double beta2, double eps, int maximize, void* hip_stream);

/* ------------------------------------------------------ delta-coded rows --
 * The 2-bit delta-compressed row format of the UST news page (section
 * "Formatos menos comuns": rows dense, column coordinates stored as 2-bit
 * differences; section "Performance": its MACKO SpMV for low sparsity, with
 * padding that stops at the end of each row).  Layout:
 *   enc_offsets[rows+1] (int32): row r owns encoded entries
 *     [enc_offsets[r], enc_offsets[r+1]);  E = enc_offsets[rows].
 *   codes[ceil(E/16)] (uint32): entry e has the 2-bit code in bits
 *     2(e mod 16)..2(e mod 16)+1 of codes[e/16]; its column is the previous
 *     entry's column + code + 1, starting from -1 at each row.
 *   enc_values[16 ceil(E/16)]: the values (val_type); entries that bridge a
 *     gap above 4 columns are zero-valued padding entries (code 3, four
 *     columns each); the tail after E is zero.  Nothing is padded after a
 *     row's last stored entry.
 * Building it takes two calls: spops_delta_size writes enc_offsets and
 * returns E (it synchronizes); the caller allocates codes and enc_values;
 * spops_delta_encode fills them.  The CSR's columns must be strictly
 * ascending inside each row and in [0, cols) (SPOPS_ERR_INDEX_ORDER from
 * spops_delta_size otherwise). */
spops_status spops_delta_size_workspace(int64_t rows, size_t* bytes);
spops_status spops_delta_size(const spops_csr* A, int32_t* enc_offsets, int64_t* enc_entries,
                              void* workspace, size_t workspace_bytes, void* hip_stream);
/* Fills codes and enc_values (A->values required, same dtype) for the
 * enc_offsets / E that spops_delta_size returned for A. */
spops_status spops_delta_encode(const spops_csr* A, const int32_t* enc_offsets,
                                int64_t enc_entries, uint32_t* codes, void* enc_values,
                                void* hip_stream);
/* y = A x for A in the delta format (rows x cols):
 *   x: [cols] in val_type;  y: [rows], y_type SPOPS_F32 or val_type (one
 *   rounding of the fp32 sum).  fp32 accumulation; deterministic. */
spops_status spops_delta_spmv(int64_t rows, int64_t cols, const int32_t* enc_offsets,
                              int64_t enc_entries, const uint32_t* codes, const void* enc_values,
                              spops_dtype val_type, const void* x, void* y, spops_dtype y_type,
                              void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPOPS_H */

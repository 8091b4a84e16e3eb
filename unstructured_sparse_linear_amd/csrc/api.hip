// api.hip -- the extern "C" entry points declared in include/spops.h.
// Host-side validation of metadata only, then kernel launches on the
// caller's stream.  See the header for the meaning of every argument.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <new>

#include "kernels.h"
#include "spops.h"

using namespace spops;

struct spops_spmm_plan {
  SpmmSchedule sch;
  int64_t rows, nnz;
  const void* ro;
  const void* row_idx;
};

struct spops_sddmm_plan {
  SddmmPlanDev dev;
};

namespace spops {
namespace {
std::atomic<int64_t> g_options[kOptCount];
}  // namespace
int64_t option(int o) {
  return (o >= 0 && o < kOptCount) ? g_options[o].load(std::memory_order_relaxed) : 0;
}
}  // namespace spops

namespace {

// Default density threshold.  A row (column) is dense at 2% of the
// columns (remaining rows), but never below one tile's width of entries:
// on small matrices 2% is close to the mean row length, and such rows would
// fill the 128-wide tiles far less than the general kernel's gathers.
constexpr double kDefaultTau = 0.02;
constexpr int64_t kDefaultMinDense = spops::kSddmmTN;

bool dtype_ok(int d) { return d == SPOPS_F32 || d == SPOPS_F16 || d == SPOPS_BF16; }
bool itype_ok(int t) { return t == SPOPS_I16 || t == SPOPS_I32; }
int elem_bytes(int d) { return d == SPOPS_F32 ? 4 : 2; }

// Structural metadata of a CSR.  Values / row_idx are checked only when the
// operation uses them.
spops_status check_csr(const spops_csr* A, bool need_values, bool need_row_idx) {
  if (!A) return SPOPS_ERR_NULL;
  if (A->rows < 0 || A->cols < 0 || A->nnz < 0) return SPOPS_ERR_SHAPE;
  if (A->rows > INT32_MAX - 1 || A->cols > INT32_MAX - 1 || A->nnz > INT32_MAX)
    return SPOPS_ERR_SHAPE;
  if (A->nnz > 0 && (A->rows == 0 || A->cols == 0)) return SPOPS_ERR_SHAPE;
  if (!itype_ok(A->col_type)) return SPOPS_ERR_DTYPE;
  if (A->col_type == SPOPS_I16 && A->cols > 32767) return SPOPS_ERR_INDEX_WIDTH;
  if (!A->row_offsets) return SPOPS_ERR_NULL;
  if (A->nnz > 0 && !A->col_idx) return SPOPS_ERR_NULL;
  if (need_values) {
    if (!dtype_ok(A->val_type)) return SPOPS_ERR_DTYPE;
    if (A->nnz > 0 && !A->values) return SPOPS_ERR_NULL;
  }
  if (need_row_idx) {
    if (!itype_ok(A->row_idx_type)) return SPOPS_ERR_DTYPE;
    if (A->row_idx_type == SPOPS_I16 && A->rows > 32767) return SPOPS_ERR_INDEX_WIDTH;
    if (A->rows > 0 && !A->row_idx) return SPOPS_ERR_NULL;
  }
  return SPOPS_OK;
}

spops_status from_hip(hipError_t e) { return e == hipSuccess ? SPOPS_OK : SPOPS_ERR_HIP; }

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Launch arguments of C = A * B for validated inputs.
SpmmArgs spmm_args(const spops_csr* A, const void* B, spops_dtype b_type, int64_t N, int64_t ldb,
                   void* C, spops_dtype c_type, int64_t ldc, const spops_spmm_plan* plan,
                   void* workspace) {
  SpmmArgs a{};
  a.m = A->rows;
  a.k = A->cols;
  a.nnz = A->nnz;
  a.N = N;
  a.ldb = ldb;
  a.ldc = ldc;
  a.ro = A->row_offsets;
  a.col = A->col_idx;
  a.col_i32 = A->col_type == SPOPS_I32;
  a.val = A->values;
  a.row_idx = A->row_idx;
  a.ri_i32 = A->row_idx_type == SPOPS_I32;
  a.B = B;
  a.C = C;
  a.dtype = b_type;
  a.out_dtype = c_type;
  if (plan) {
    a.natural = plan->sch.natural;
    a.max_row = plan->sch.max_row;
  }
  if (plan && plan->sch.flat.U > 0 && plan->sch.blk_row) {
    a.blk_row = plan->sch.blk_row;
    a.flat_E = plan->sch.flat.E;
    a.flat_T = plan->sch.flat.T;
    a.flat_U = plan->sch.flat.U;
  }
  if (plan && plan->sch.P > 0) {
    a.P = plan->sch.P;
    a.S = plan->sch.S;
    a.T = plan->sch.T;
    a.CLs = 0;
    while ((1 << a.CLs) < plan->sch.CL) ++a.CLs;
    a.item_pos = plan->sch.item_pos;
    a.item_chunk = plan->sch.item_chunk;
    a.split_pos = plan->sch.split_pos;
    a.split_start = plan->sch.split_start;
    a.split_end = plan->sch.split_end;
    a.partial = (float*)workspace;
  }
  return a;
}

}  // namespace

extern "C" {

int spops_abi_version(void) { return SPOPS_ABI_VERSION; }

spops_status spops_set_option(spops_option opt, int64_t value) {
  if ((int)opt < 0 || (int)opt >= kOptCount) return SPOPS_ERR_UNSUPPORTED;
  if (value < 0) return SPOPS_ERR_ARGUMENT;
  g_options[(int)opt].store(value, std::memory_order_relaxed);
  return SPOPS_OK;
}

spops_status spops_get_option(spops_option opt, int64_t* value) {
  if (!value) return SPOPS_ERR_NULL;
  if ((int)opt < 0 || (int)opt >= kOptCount) return SPOPS_ERR_UNSUPPORTED;
  *value = g_options[(int)opt].load(std::memory_order_relaxed);
  return SPOPS_OK;
}

const char* spops_status_string(spops_status s) {
  switch (s) {
    case SPOPS_OK: return "ok";
    case SPOPS_ERR_NULL: return "a required pointer is NULL";
    case SPOPS_ERR_SHAPE: return "invalid or inconsistent sizes or leading dimensions";
    case SPOPS_ERR_DTYPE: return "unknown dtype or unsupported dtype combination";
    case SPOPS_ERR_INDEX_WIDTH: return "int16 index list cannot address this extent";
    case SPOPS_ERR_WORKSPACE: return "workspace missing or too small";
    case SPOPS_ERR_UNSUPPORTED: return "unsupported request";
    case SPOPS_ERR_PLAN: return "plan was built for a different matrix";
    case SPOPS_ERR_HIP: return "HIP runtime error";
    case SPOPS_ERR_ARGUMENT: return "scalar argument out of range";
    case SPOPS_ERR_INDEX_ORDER: return "columns not strictly ascending in a row, or out of range";
    case SPOPS_ERR_INVALID_INDEX: return "the CSR index data is invalid (see the validator's findings)";
  }
  return "unknown status";
}

// ---------------------------------------------------------------- SpMM ---

spops_status spops_spmm_plan_create(const spops_csr* A, void* hip_stream,
                                    spops_spmm_plan** plan) {
  if (!plan) return SPOPS_ERR_NULL;
  *plan = nullptr;
  spops_status st = check_csr(A, false, true);
  if (st != SPOPS_OK) return st;
  spops_spmm_plan* p = new (std::nothrow) spops_spmm_plan();
  if (!p) return SPOPS_ERR_HIP;
  p->rows = A->rows;
  p->nnz = A->nnz;
  p->ro = A->row_offsets;
  p->row_idx = A->row_idx;
  hipError_t e = build_spmm_schedule(A->row_offsets, A->row_idx, A->row_idx_type == SPOPS_I32,
                                     A->rows, A->nnz, kSpmmSplitLen, &p->sch,
                                     as_stream(hip_stream));
  if (e != hipSuccess) {
    delete p;
    return SPOPS_ERR_HIP;
  }
  *plan = p;
  return SPOPS_OK;
}

spops_status spops_spmm_plan_destroy(spops_spmm_plan* plan) {
  if (!plan) return SPOPS_OK;
  free_spmm_schedule(&plan->sch);
  delete plan;
  return SPOPS_OK;
}

spops_status spops_spmm_workspace_size(const spops_spmm_plan* plan, int64_t N, size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  if (N < 0) return SPOPS_ERR_SHAPE;
  *bytes = (plan && plan->sch.S > 0) ? align256((size_t)plan->sch.P * (size_t)N * 4) : 0;
  return SPOPS_OK;
}

spops_status spops_spmm_plan_info(const spops_spmm_plan* plan, int64_t* split_rows,
                                  int64_t* chunks, int64_t* max_row_nnz) {
  if (!plan) return SPOPS_ERR_NULL;
  if (split_rows) *split_rows = plan->sch.S;
  if (chunks) *chunks = plan->sch.P;
  if (max_row_nnz) *max_row_nnz = plan->sch.max_row;
  return SPOPS_OK;
}

spops_status spops_spmm(const spops_csr* A, const void* B, spops_dtype b_type, int64_t N,
                        int64_t ldb, void* C, spops_dtype c_type, int64_t ldc,
                        const spops_spmm_plan* plan, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
  spops_status st = check_csr(A, true, true);
  if (st != SPOPS_OK) return st;
  if (!dtype_ok(b_type) || !dtype_ok(c_type)) return SPOPS_ERR_DTYPE;
  if (b_type != A->val_type) return SPOPS_ERR_DTYPE;
  if (c_type != SPOPS_F32 && c_type != b_type) return SPOPS_ERR_DTYPE;
  if (N < 0 || ldb < (N > 0 ? N : 1) || ldc < (N > 0 ? N : 1)) return SPOPS_ERR_SHAPE;
  if (N == 0 || A->rows == 0) return SPOPS_OK;
  if (!C) return SPOPS_ERR_NULL;
  if (A->nnz > 0 && !B) return SPOPS_ERR_NULL;
  if (plan) {
    if (plan->rows != A->rows || plan->nnz != A->nnz || plan->ro != A->row_offsets ||
        plan->row_idx != A->row_idx)
      return SPOPS_ERR_PLAN;
    size_t need = 0;
    spops_spmm_workspace_size(plan, N, &need);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SPOPS_ERR_WORKSPACE;
  }
  const SpmmArgs a = spmm_args(A, B, b_type, N, ldb, C, c_type, ldc, plan, workspace);
  return from_hip(launch_spmm(a, as_stream(hip_stream)));
}

// --------------------------------------------------------------- SDDMM ---

static void free_sddmm_plan_mem(SddmmPlanDev* p) {
  if (p->mem) (void)hipFree(p->mem);  // teardown: nothing to report
  *p = SddmmPlanDev{};
}

spops_status spops_sddmm_plan_create(const spops_csr* mask, double tau, void* hip_stream,
                                     spops_sddmm_plan** plan) {
  if (!plan) return SPOPS_ERR_NULL;
  *plan = nullptr;
  spops_status st = check_csr(mask, false, false);
  if (st != SPOPS_OK) return st;
  int64_t min_dense = 1;
  if (!(tau > 0.0) || isnan(tau)) {
    tau = kDefaultTau;
    min_dense = kDefaultMinDense;
  }
  spops_sddmm_plan* p = new (std::nothrow) spops_sddmm_plan();
  if (!p) return SPOPS_ERR_HIP;
  hipStream_t s = as_stream(hip_stream);
  const int64_t m = mask->rows, n = mask->cols, nnz = mask->nnz;
  void* mem = nullptr;
  void* scratch = nullptr;
  hipError_t e = hipMalloc(&mem, sddmm_plan_bytes(m, n, nnz));
  if (e == hipSuccess) e = hipMalloc(&scratch, sddmm_plan_scratch_bytes(m, n, nnz));
  if (e == hipSuccess)
    e = enqueue_sddmm_plan(m, n, nnz, mask->row_offsets, mask->col_idx,
                           mask->col_type == SPOPS_I32, tau, min_dense, mem, scratch, &p->dev,
                           s);
  if (e == hipSuccess) e = fetch_sddmm_plan_counts(&p->dev, s);  // synchronizes s
  else if (scratch) (void)hipStreamSynchronize(s);  // e already holds the failure
  if (scratch) (void)hipFree(scratch);
  p->dev.mem = mem;
  if (e != hipSuccess) {
    free_sddmm_plan_mem(&p->dev);
    delete p;
    return SPOPS_ERR_HIP;
  }
  *plan = p;
  return SPOPS_OK;
}

spops_status spops_sddmm_plan_destroy(spops_sddmm_plan* plan) {
  if (!plan) return SPOPS_OK;
  free_sddmm_plan_mem(&plan->dev);
  delete plan;
  return SPOPS_OK;
}

spops_status spops_sddmm_plan_info(const spops_sddmm_plan* plan, int64_t* dense_rows,
                                   int64_t* dense_cols, int64_t* tiled_nnz, int64_t* rest_nnz,
                                   int64_t* tiles) {
  if (!plan) return SPOPS_ERR_NULL;
  const SddmmPlanScalars& h = plan->dev.h;
  if (dense_rows) *dense_rows = h.H;
  if (dense_cols) *dense_cols = h.Hc;
  if (tiled_nnz) *tiled_nnz = h.tiled;
  if (rest_nnz) *rest_nnz = h.rest;
  if (tiles) *tiles = h.tiles;
  return SPOPS_OK;
}

// The dense tiles need 16-bit inputs, K a multiple of 8 and 16-byte rows
// (MFMA operands are 8 consecutive K elements).
static bool sddmm_tiles_possible(spops_dtype in_type, int64_t K) {
  return in_type != SPOPS_F32 && K > 0 && K % 8 == 0;
}
// The tile kernel reads A and BT through buffer resources with 32-bit
// offsets: each operand's extent (rows x leading dimension) must stay under
// 2 GiB; larger operands take the entry-list path.
static bool sddmm_tiles_ok(spops_dtype in_type, int64_t m, int64_t n, int64_t K, int64_t lda,
                           int64_t ldbt, const void* A, const void* BT) {
  return sddmm_tiles_possible(in_type, K) && lda % 8 == 0 && ldbt % 8 == 0 &&
         ((uintptr_t)A % 16 == 0) && ((uintptr_t)BT % 16 == 0) &&
         m * lda * 2 < ((int64_t)1 << 31) && n * ldbt * 2 < ((int64_t)1 << 31);
}

// The entry-list kernel reads 16-byte vectors along K.
static bool sddmm_list_ok(spops_dtype in_type, int64_t K, int64_t lda, int64_t ldbt,
                          const void* A, const void* BT) {
  const int64_t v = in_type == SPOPS_F32 ? 4 : 8;
  return K > 0 && K % v == 0 && lda % v == 0 && ldbt % v == 0 && ((uintptr_t)A % 16 == 0) &&
         ((uintptr_t)BT % 16 == 0);
}

// Workspace of a structure-aware call without a plan: the plan built inside
// the call (its arrays, then its temporaries).
static size_t sddmm_inline_plan_bytes(const spops_csr* mask) {
  return align256(sddmm_plan_bytes(mask->rows, mask->cols, mask->nnz)) +
         sddmm_plan_scratch_bytes(mask->rows, mask->cols, mask->nnz);
}

// Pieces of K for the plan's remainder (1: none).  Splitting K over the
// XCDs (piece b on XCD b) lets each L2 hold its slice of BT, so the
// remainder's BT rows, each gathered by several entries, come from L2; it
// pays when BT exceeds what the eight L2s hold together (16 pieces, two
// per XCD, measured best on the 45 MB BT of the cross-clustered mask).  The option
// kOptSddmmRestSplit sets the count (1 turns the split off).
static int sddmm_rest_pieces(const SddmmPlanDev& P, int64_t K, spops_dtype in_type) {
  if (!P.host_ok || P.h.rest <= 0 || in_type == SPOPS_F32) return 1;
  const int64_t opt = option(kOptSddmmRestSplit);
  int pieces = opt > 0 ? (int)(opt < 16 ? opt : 16)
                       : (P.n * K * 2 > ((int64_t)32 << 20) ? 16 : 1);
  if (pieces > 8) pieces = 16;
  while (pieces > 1 && K % (8 * pieces) != 0) pieces /= 2;
  return pieces;
}

static size_t sddmm_plan_ws_bytes(const SddmmPlanDev& P, int64_t K, spops_dtype in_type,
                                  size_t* rest_off) {
  const size_t tiles = align256(sddmm_split_bytes(P, sddmm_tile_schedule(P, K)));
  const int pieces = sddmm_rest_pieces(P, K, in_type);
  *rest_off = tiles;
  return tiles + (pieces > 1 ? align256((size_t)pieces * (size_t)P.h.rest * 4) : 0);
}

spops_status spops_sddmm_workspace_size(const spops_csr* mask, int64_t K, spops_dtype in_type,
                                        spops_sddmm_backend backend,
                                        const spops_sddmm_plan* plan, size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  *bytes = 0;
  spops_status st = check_csr(mask, false, false);
  if (st != SPOPS_OK) return st;
  if (!dtype_ok(in_type)) return SPOPS_ERR_DTYPE;
  if (backend != SPOPS_SDDMM_STRUCTURE_AWARE && backend != SPOPS_SDDMM_GENERAL)
    return SPOPS_ERR_UNSUPPORTED;
  if (K < 0) return SPOPS_ERR_SHAPE;
  if (backend != SPOPS_SDDMM_STRUCTURE_AWARE || !sddmm_tiles_possible(in_type, K) ||
      mask->nnz == 0)
    return SPOPS_OK;
  size_t rest_off = 0;
  if (plan)
    *bytes = sddmm_plan_ws_bytes(plan->dev, K, in_type, &rest_off);
  else
    *bytes = sddmm_inline_plan_bytes(mask);
  return SPOPS_OK;
}

spops_status spops_sddmm(const spops_csr* mask, const void* A, int64_t K, int64_t lda,
                         const void* BT, int64_t ldbt, spops_dtype in_type, void* out_values,
                         spops_dtype out_type, spops_sddmm_backend backend,
                         const spops_sddmm_plan* plan, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  spops_status st = check_csr(mask, false, false);
  if (st != SPOPS_OK) return st;
  if (!dtype_ok(in_type) || !dtype_ok(out_type)) return SPOPS_ERR_DTYPE;
  if (out_type != SPOPS_F32 && out_type != in_type) return SPOPS_ERR_DTYPE;
  if (backend != SPOPS_SDDMM_STRUCTURE_AWARE && backend != SPOPS_SDDMM_GENERAL)
    return SPOPS_ERR_UNSUPPORTED;
  if (K < 0 || lda < (K > 0 ? K : 1) || ldbt < (K > 0 ? K : 1)) return SPOPS_ERR_SHAPE;
  if (mask->nnz == 0) return SPOPS_OK;
  if (!out_values) return SPOPS_ERR_NULL;
  if (K > 0 && (!A || !BT)) return SPOPS_ERR_NULL;
  if (plan && backend == SPOPS_SDDMM_STRUCTURE_AWARE &&
      (plan->dev.m != mask->rows || plan->dev.n != mask->cols || plan->dev.nnz != mask->nnz ||
       plan->dev.mask_ro != mask->row_offsets || plan->dev.mask_col != mask->col_idx))
    return SPOPS_ERR_PLAN;
  hipStream_t s = as_stream(hip_stream);

  const bool tiles_ok = sddmm_tiles_ok(in_type, mask->rows, mask->cols, K, lda, ldbt, A, BT);
  const bool list_ok = sddmm_list_ok(in_type, K, lda, ldbt, A, BT);
  SddmmListArgs r{};
  r.m = mask->rows;
  r.n = mask->cols;
  r.K = K;
  r.lda = lda;
  r.ldbt = ldbt;
  r.col = mask->col_idx;
  r.col_i32 = mask->col_type == SPOPS_I32;
  r.A = A;
  r.BT = BT;
  r.out = out_values;
  r.dtype = in_type;
  r.out_dtype = out_type;
  // the whole mask in CSR order: the entry-list kernel, or the scalar kernel
  // when K or the operands do not allow 16-byte vectors
  auto general = [&]() {
    if (list_ok) {
      r.ro = mask->row_offsets;
      r.nb = 1;
      r.bstart[0] = 0;
      r.bstart[1] = mask->nnz;
      return from_hip(launch_sddmm_list(r, s));
    }
    SddmmArgs g{};
    g.m = mask->rows;
    g.n = mask->cols;
    g.K = K;
    g.lda = lda;
    g.ldbt = ldbt;
    g.ro = mask->row_offsets;
    g.count = mask->nnz;
    g.col = mask->col_idx;
    g.col_i32 = mask->col_type == SPOPS_I32;
    g.A = A;
    g.BT = BT;
    g.out = out_values;
    g.dtype = in_type;
    g.out_dtype = out_type;
    return from_hip(launch_sddmm_general(g, s));
  };
  // the plan's remainder through the entry-list kernel, bucket by bucket,
  // or with K cut into pieces (partial sums in `part`, then their sum)
  auto remainder = [&](const SddmmPlanDev& P, int pieces, float* part) {
    r.pos = P.ent_pos;
    r.rows = P.ent_rc;
    r.cols = P.ent_col;
    if (P.host_ok) {
      if (P.h.rest == 0) return hipSuccess;
      if (pieces > 1) {
        // every piece covers the whole remainder: in row order, so that a
        // row's A slice is loaded once per piece
        r.pos = P.row_pos;
        r.rows = P.row_rc;
        r.cols = P.row_col;
        r.nb = pieces;
        r.ksplit = pieces;
        r.kpiece = K / pieces;
        r.part = part;
        r.bstart[0] = 0;
        r.bstart[1] = P.h.rest;
        hipError_t e = launch_sddmm_list(r, s);
        if (e != hipSuccess) return e;
        return launch_sddmm_piece_sum(part, pieces, P.h.rest, P.row_pos, 0, out_values, out_type,
                                      s);
      }
      r.nb = P.h.nb;
      for (int b = 0; b <= P.h.nb; ++b) r.bstart[b] = P.bucket_start[b];
    } else {
      r.nb = P.nb_max;
      r.bstart_dev = P.key_start + P.rest_key;
      r.max_bucket = mask->nnz;
    }
    return launch_sddmm_list(r, s);
  };
  if (backend == SPOPS_SDDMM_GENERAL) return general();
  if (!tiles_ok) {
    // 32-bit or unaligned inputs: the plan's remainder still runs where the
    // plan found no tiles (its remainder is then the whole mask)
    if (plan && plan->dev.host_ok && plan->dev.h.tiles == 0 && list_ok)
      return from_hip(remainder(plan->dev, 1, nullptr));
    return general();
  }
  if (!plan) {
    // plan built here, in the caller's workspace, on the stream: no
    // allocation, no synchronization
    const size_t need = sddmm_inline_plan_bytes(mask);
    if (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256 != 0)
      return SPOPS_ERR_WORKSPACE;
    SddmmPlanDev P;
    char* ws = (char*)workspace;
    hipError_t e = enqueue_sddmm_plan(
        mask->rows, mask->cols, mask->nnz, mask->row_offsets, mask->col_idx,
        mask->col_type == SPOPS_I32, kDefaultTau, kDefaultMinDense, ws,
        ws + align256(sddmm_plan_bytes(mask->rows, mask->cols, mask->nnz)), &P, s);
    if (e == hipSuccess)
      e = launch_sddmm_tiles(P, K, A, lda, BT, ldbt, in_type, out_values, out_type,
                             sddmm_tile_schedule(P, K), nullptr, s);
    if (e == hipSuccess) e = remainder(P, 1, nullptr);
    return from_hip(e);
  }
  const SddmmPlanDev& P = plan->dev;
  const SddmmTileSched sched = sddmm_tile_schedule(P, K);
  size_t rest_off = 0;
  const size_t need = sddmm_plan_ws_bytes(P, K, in_type, &rest_off);
  if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 16 != 0))
    return SPOPS_ERR_WORKSPACE;
  hipError_t e = launch_sddmm_tiles(P, K, A, lda, BT, ldbt, in_type, out_values, out_type,
                                    sched, (float*)workspace, s);
  if (e == hipSuccess)
    e = remainder(P, sddmm_rest_pieces(P, K, in_type), (float*)((char*)workspace + rest_off));
  return from_hip(e);
}

// ------------------------------------------------------------- csr_add ---

spops_status spops_csr_add(const spops_csr* A, void* W, spops_dtype w_type, int64_t ldw,
                           void* hip_stream) {
  spops_status st = check_csr(A, true, false);
  if (st != SPOPS_OK) return st;
  if (!dtype_ok(w_type)) return SPOPS_ERR_DTYPE;
  if (w_type != A->val_type) return SPOPS_ERR_DTYPE;
  if (ldw < (A->cols > 0 ? A->cols : 1)) return SPOPS_ERR_SHAPE;
  if (A->nnz == 0) return SPOPS_OK;
  if (!W) return SPOPS_ERR_NULL;
  return from_hip(launch_csr_add(A->rows, A->cols, A->nnz, A->row_offsets, A->col_idx,
                                 A->col_type == SPOPS_I32, A->values, W, ldw, w_type,
                                 as_stream(hip_stream)));
}

// ------------------------------------------------------- csr_transpose ---

spops_status spops_csr_transpose_workspace_size(int64_t rows, int64_t cols, int64_t nnz,
                                                size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  if (rows < 0 || cols < 0 || nnz < 0 || nnz > INT32_MAX) return SPOPS_ERR_SHAPE;
  *bytes = transpose_workspace_bytes(rows, cols, nnz);
  return SPOPS_OK;
}

spops_status spops_csr_transpose(const spops_csr* A, void* out_values, int32_t* out_row_offsets,
                                 void* out_col_idx, spops_itype out_col_type, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
  spops_status st = check_csr(A, A && A->values != nullptr, false);
  if (st != SPOPS_OK) return st;
  if (!itype_ok(out_col_type)) return SPOPS_ERR_DTYPE;
  if (out_col_type == SPOPS_I16 && A->rows > 32767) return SPOPS_ERR_INDEX_WIDTH;
  if (!out_row_offsets) return SPOPS_ERR_NULL;
  if (A->nnz > 0 && (!out_col_idx || (A->values && !out_values))) return SPOPS_ERR_NULL;
  const size_t need = transpose_workspace_bytes(A->rows, A->cols, A->nnz);
  if (!workspace || workspace_bytes < need) return SPOPS_ERR_WORKSPACE;
  return from_hip(launch_csr_transpose(
      A->rows, A->cols, A->nnz, A->row_offsets, A->col_idx, A->col_type == SPOPS_I32,
      A->values, A->values ? elem_bytes(A->val_type) : 0, out_values, out_row_offsets,
      out_col_idx, out_col_type == SPOPS_I32, workspace, as_stream(hip_stream)));
}

// ------------------------------------------------ transpose permutation ---

static size_t transpose_perm_workspace_bytes(int64_t rows, int64_t cols, int64_t nnz) {
  return align256(transpose_workspace_bytes(rows, cols, nnz)) + align256((size_t)nnz * 4);
}

spops_status spops_csr_transpose_permutation_workspace_size(int64_t rows, int64_t cols,
                                                            int64_t nnz, size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  if (rows < 0 || cols < 0 || nnz < 0 || nnz > INT32_MAX) return SPOPS_ERR_SHAPE;
  *bytes = transpose_perm_workspace_bytes(rows, cols, nnz);
  return SPOPS_OK;
}

spops_status spops_csr_transpose_permutation(const spops_csr* A, int32_t* out_src,
                                             int32_t* out_row_offsets, void* out_col_idx,
                                             spops_itype out_col_type, void* workspace,
                                             size_t workspace_bytes, void* hip_stream) {
  spops_status st = check_csr(A, false, false);
  if (st != SPOPS_OK) return st;
  if (!itype_ok(out_col_type)) return SPOPS_ERR_DTYPE;
  if (out_col_type == SPOPS_I16 && A->rows > 32767) return SPOPS_ERR_INDEX_WIDTH;
  if (!out_row_offsets) return SPOPS_ERR_NULL;
  if (A->nnz > 0 && (!out_col_idx || !out_src)) return SPOPS_ERR_NULL;
  const size_t tws = align256(transpose_workspace_bytes(A->rows, A->cols, A->nnz));
  const size_t need = transpose_perm_workspace_bytes(A->rows, A->cols, A->nnz);
  if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256 != 0))
    return SPOPS_ERR_WORKSPACE;
  return from_hip(launch_csr_transpose_perm(
      A->rows, A->cols, A->nnz, A->row_offsets, A->col_idx, A->col_type == SPOPS_I32, out_src,
      out_row_offsets, out_col_idx, out_col_type == SPOPS_I32, workspace,
      (int32_t*)((char*)workspace + tws), as_stream(hip_stream)));
}

spops_status spops_permute_values(const void* in, int64_t n_in, spops_dtype type,
                                  const int32_t* src, int64_t n, void* out, void* hip_stream) {
  if (!dtype_ok(type)) return SPOPS_ERR_DTYPE;
  if (n < 0 || n_in < 0 || n > INT32_MAX || n_in > INT32_MAX) return SPOPS_ERR_SHAPE;
  if (n == 0) return SPOPS_OK;
  if (!src || !out || (n_in > 0 && !in)) return SPOPS_ERR_NULL;
  return from_hip(launch_permute_values(in, n_in, elem_bytes(type), src, n, out,
                                        as_stream(hip_stream)));
}

// ------------------------------------------------------------ validation ---

spops_status spops_validate_csr_workspace_size(int64_t rows, int64_t cols, int64_t nnz,
                                               size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  if (rows < 0 || cols < 0 || nnz < 0 || rows > INT32_MAX - 1 || cols > INT32_MAX - 1 ||
      nnz > INT32_MAX)
    return SPOPS_ERR_SHAPE;
  *bytes = validate_workspace_bytes(rows, cols, nnz);
  return SPOPS_OK;
}

spops_status spops_validate_csr(const spops_csr* A, int check_duplicates, void* workspace,
                                size_t workspace_bytes, uint32_t* findings, void* hip_stream) {
  if (findings) *findings = 0;
  spops_status st = check_csr(A, false, false);
  if (st != SPOPS_OK) return st;
  if (A->row_idx) {
    if (!itype_ok(A->row_idx_type)) return SPOPS_ERR_DTYPE;
    if (A->row_idx_type == SPOPS_I16 && A->rows > 32767) return SPOPS_ERR_INDEX_WIDTH;
  }
  if (!workspace || workspace_bytes < validate_workspace_bytes(A->rows, A->cols, A->nnz) ||
      (uintptr_t)workspace % 256 != 0)
    return SPOPS_ERR_WORKSPACE;
  uint32_t f = 0;
  hipError_t e = launch_validate(A->rows, A->cols, A->nnz, A->row_offsets, A->col_idx,
                                 A->col_type == SPOPS_I32, A->row_idx,
                                 A->row_idx_type == SPOPS_I32, check_duplicates, workspace, &f,
                                 as_stream(hip_stream));
  if (e != hipSuccess) return SPOPS_ERR_HIP;
  if (findings) *findings = f;
  return f ? SPOPS_ERR_INVALID_INDEX : SPOPS_OK;
}

// ------------------------------------------------- transpose, no allocation ---

// The scratch of spops_csr_transpose_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only names a stand-in); the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (looked up on the first
// call on that device); nullptr on failure.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}
}  // namespace

spops_status spops_csr_transpose_noalloc(const spops_csr* A, void* out_values,
                                         int32_t* out_row_offsets, void* out_col_idx,
                                         spops_itype out_col_type, void* hip_stream) {
  spops_status st = check_csr(A, A && A->values != nullptr, false);
  if (st != SPOPS_OK) return st;
  if (!itype_ok(out_col_type)) return SPOPS_ERR_DTYPE;
  if (out_col_type == SPOPS_I16 && A->rows > 32767) return SPOPS_ERR_INDEX_WIDTH;
  if (!out_row_offsets) return SPOPS_ERR_NULL;
  if (A->nnz > 0 && (!out_col_idx || (A->values && !out_values))) return SPOPS_ERR_NULL;
  if (transpose_workspace_bytes(A->rows, A->cols, A->nnz) > kNoAllocScratchBytes)
    return SPOPS_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return SPOPS_ERR_HIP;
  return from_hip(launch_csr_transpose(
      A->rows, A->cols, A->nnz, A->row_offsets, A->col_idx, A->col_type == SPOPS_I32,
      A->values, A->values ? elem_bytes(A->val_type) : 0, out_values, out_row_offsets,
      out_col_idx, out_col_type == SPOPS_I32, ws, as_stream(hip_stream)));
}

spops_status spops_csr_transpose_noalloc_limit(size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  *bytes = kNoAllocScratchBytes;
  return SPOPS_OK;
}

// ------------------------------------------------------------ row order ---

spops_status spops_sort_rows_by_nnz_workspace_size(int64_t rows, int64_t cols, size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  if (rows < 0 || cols < 0 || rows > INT32_MAX - 1 || cols > INT32_MAX - 1) return SPOPS_ERR_SHAPE;
  *bytes = sort_rows_workspace_bytes(rows, cols);
  return SPOPS_OK;
}

spops_status spops_sort_rows_by_nnz(const int32_t* row_offsets, int64_t rows, int64_t cols,
                                    void* row_idx, spops_itype row_idx_type, void* workspace,
                                    size_t workspace_bytes, void* hip_stream) {
  if (rows < 0 || cols < 0 || rows > INT32_MAX - 1 || cols > INT32_MAX - 1) return SPOPS_ERR_SHAPE;
  if (!itype_ok(row_idx_type)) return SPOPS_ERR_DTYPE;
  if (row_idx_type == SPOPS_I16 && rows > 32767) return SPOPS_ERR_INDEX_WIDTH;
  if (rows == 0) return SPOPS_OK;
  if (!row_offsets || !row_idx) return SPOPS_ERR_NULL;
  if (!workspace || workspace_bytes < sort_rows_workspace_bytes(rows, cols))
    return SPOPS_ERR_WORKSPACE;
  return from_hip(launch_sort_rows(row_offsets, rows, cols, row_idx, row_idx_type == SPOPS_I32,
                                   workspace, as_stream(hip_stream)));
}

// ---------------------------------------------------- conjugate gradients --

static spops_status check_cg(const spops_csr* A, const spops_spmm_plan* plan) {
  spops_status st = check_csr(A, true, true);
  if (st != SPOPS_OK) return st;
  if (A->rows != A->cols) return SPOPS_ERR_SHAPE;
  if (A->val_type != SPOPS_F32) return SPOPS_ERR_DTYPE;
  if (plan && (plan->rows != A->rows || plan->nnz != A->nnz || plan->ro != A->row_offsets ||
               plan->row_idx != A->row_idx))
    return SPOPS_ERR_PLAN;
  return SPOPS_OK;
}

// Entry-range blocks of the fused iteration (0 workgroups: the library's
// SpMV between the direction and update kernels).
static int64_t cg_fused_blocks(const spops_csr* A, const spops_spmm_plan* plan) {
  if (!plan || plan->sch.flat.U <= 0 || !plan->sch.blk_row) return 0;
  return cg_fused_grid(A->nnz, plan->sch.flat.E);
}

spops_status spops_cg_workspace_size(const spops_csr* A, const spops_spmm_plan* plan,
                                     size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  spops_status st = check_cg(A, plan);
  if (st != SPOPS_OK) return st;
  size_t sp = 0;
  spops_spmm_workspace_size(plan, 1, &sp);
  *bytes = cg_workspace_bytes(A->rows, cg_fused_blocks(A, plan), sp);
  return SPOPS_OK;
}

spops_status spops_cg(const spops_csr* A, const void* b, void* x, double rtol, int64_t max_iter,
                      int64_t check_every, const spops_spmm_plan* plan, void* workspace,
                      size_t workspace_bytes, int64_t* iters_out, double* rel_resid_out,
                      void* hip_stream) {
  spops_status st = check_cg(A, plan);
  if (st != SPOPS_OK) return st;
  if (!(rtol >= 0.0) || !isfinite(rtol) || max_iter < 0 || check_every < 1)
    return SPOPS_ERR_ARGUMENT;
  const int64_t m = A->rows;
  if (iters_out) *iters_out = 0;
  if (rel_resid_out) *rel_resid_out = 0.0;
  if (m == 0) return SPOPS_OK;
  if (!b || !x) return SPOPS_ERR_NULL;
  size_t need = 0;
  spops_cg_workspace_size(A, plan, &need);
  if (!workspace || workspace_bytes < need) return SPOPS_ERR_WORKSPACE;
  hipStream_t s = as_stream(hip_stream);
  const int64_t fused = cg_fused_blocks(A, plan);
  const CgBuffers w = carve_cg_workspace(workspace, m, fused);
  // q = A x0, then r = b - q
  const SpmmArgs ax = spmm_args(A, x, SPOPS_F32, 1, 1, w.q, SPOPS_F32, 1, plan, w.spmm_ws);
  hipError_t e = launch_spmm(ax, s);
  if (e == hipSuccess) e = launch_cg_init(m, (const float*)b, w, rtol, s);
  if (e != hipSuccess) return SPOPS_ERR_HIP;
  CgSpmvArgs fa{};
  fa.m = m;
  fa.nnz = A->nnz;
  fa.ro = A->row_offsets;
  fa.col = A->col_idx;
  fa.col_i32 = A->col_type == SPOPS_I32;
  fa.val = (const float*)A->values;
  if (fused > 0) {
    fa.blk_row = plan->sch.blk_row;
    fa.E = plan->sch.flat.E;
    fa.T = plan->sch.flat.T;
    fa.U = plan->sch.flat.U;
  }
  CgState h{};
  int64_t k = 0;
  for (;;) {
    // the first chunk is enqueued without a check: a start that already
    // meets the tolerance stops it at its first kernel
    if (k > 0 || max_iter == 0) {
      if ((e = launch_cg_record(m, k, w, s)) != hipSuccess ||
          (e = hipMemcpyAsync(&h, w.st, sizeof(h), hipMemcpyDeviceToHost, s)) != hipSuccess ||
          (e = hipStreamSynchronize(s)) != hipSuccess)
        return SPOPS_ERR_HIP;
      if (h.done || k >= max_iter) break;
    }
    const int64_t n = std::min<int64_t>(check_every, max_iter - k);
    for (int64_t j = 0; j < n; ++j, ++k) {
      if (fused > 0) {
        fa.k = k;
        e = launch_cg_fused(fa, (float*)x, w, s);
      } else {
        // p sits in the x slots of the (p, r) pairs: leading dimension 2
        const SpmmArgs ap = spmm_args(A, w.pr[(k + 1) & 1], SPOPS_F32, 1, 2, w.q, SPOPS_F32, 1,
                                      plan, w.spmm_ws);
        e = launch_cg_direction(m, k, w, s);
        if (e == hipSuccess) e = launch_spmm(ap, s);
        if (e == hipSuccess) e = launch_cg_dot_update(m, k, (float*)x, w, s);
      }
      if (e != hipSuccess) return SPOPS_ERR_HIP;
    }
  }
  if (iters_out) *iters_out = h.iters;
  if (rel_resid_out) *rel_resid_out = h.bb > 0.0 ? sqrt(h.rr[h.iters & 1] / h.bb) : 0.0;
  return SPOPS_OK;
}

// ----------------------------------------------------------- masked Adam --

spops_status spops_masked_adam(void* values, spops_dtype val_type, int64_t nnz, const void* grad,
                               const int32_t* positions, int64_t ngrad, float* exp_avg,
                               float* exp_avg_sq, int64_t step, double lr, double beta1,
                               double beta2, double eps, int maximize, void* hip_stream) {
  if (!dtype_ok(val_type)) return SPOPS_ERR_DTYPE;
  if (nnz < 0 || ngrad < 0 || nnz > INT32_MAX || ngrad > INT32_MAX) return SPOPS_ERR_SHAPE;
  if (!positions && ngrad != nnz) return SPOPS_ERR_SHAPE;
  if (step < 1 || !(lr >= 0.0) || !isfinite(lr) || !(beta1 >= 0.0 && beta1 < 1.0) ||
      !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0) || !isfinite(eps))
    return SPOPS_ERR_ARGUMENT;
  if (ngrad == 0) return SPOPS_OK;
  if (!values || !grad || !exp_avg || !exp_avg_sq) return SPOPS_ERR_NULL;
  AdamArgs a{};
  a.nnz = nnz;
  a.ngrad = ngrad;
  a.positions = positions;
  a.values = values;
  a.grad = grad;
  a.exp_avg = exp_avg;
  a.exp_avg_sq = exp_avg_sq;
  a.beta1 = (float)beta1;
  a.beta2 = (float)beta2;
  a.one_minus_beta1 = (float)(1.0 - beta1);
  a.one_minus_beta2 = (float)(1.0 - beta2);
  a.alpha_t = (float)(lr * sqrt(1.0 - pow(beta2, (double)step)) / (1.0 - pow(beta1, (double)step)));
  a.eps = (float)eps;
  a.maximize = maximize ? 1 : 0;
  return from_hip(launch_masked_adam(a, val_type, as_stream(hip_stream)));
}

// ------------------------------------------------------ delta-coded rows --

spops_status spops_delta_size_workspace(int64_t rows, size_t* bytes) {
  if (!bytes) return SPOPS_ERR_NULL;
  if (rows < 0 || rows > INT32_MAX - 1) return SPOPS_ERR_SHAPE;
  *bytes = delta_size_workspace_bytes(rows);
  return SPOPS_OK;
}

spops_status spops_delta_size(const spops_csr* A, int32_t* enc_offsets, int64_t* enc_entries,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  spops_status st = check_csr(A, false, false);
  if (st != SPOPS_OK) return st;
  if (!enc_offsets || !enc_entries) return SPOPS_ERR_NULL;
  // every count and offset must fit int32: at most one padding entry per 4
  // columns of each row on top of the stored entries
  if ((double)A->nnz + (double)A->rows * (double)((A->cols + 3) / 4) > (double)INT32_MAX)
    return SPOPS_ERR_SHAPE;
  if (!workspace || workspace_bytes < delta_size_workspace_bytes(A->rows))
    return SPOPS_ERR_WORKSPACE;
  hipStream_t s = as_stream(hip_stream);
  uint32_t tb[2] = {0, 0};
  hipError_t e = launch_delta_size(A->rows, A->cols, A->nnz, A->row_offsets, A->col_idx,
                                   A->col_type == SPOPS_I32, enc_offsets, workspace, tb, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return SPOPS_ERR_HIP;
  if (tb[1]) return SPOPS_ERR_INDEX_ORDER;
  *enc_entries = (int64_t)tb[0];
  return SPOPS_OK;
}

spops_status spops_delta_encode(const spops_csr* A, const int32_t* enc_offsets,
                                int64_t enc_entries, uint32_t* codes, void* enc_values,
                                void* hip_stream) {
  spops_status st = check_csr(A, true, false);
  if (st != SPOPS_OK) return st;
  if (!enc_offsets) return SPOPS_ERR_NULL;
  if (enc_entries < 0 || enc_entries > INT32_MAX) return SPOPS_ERR_SHAPE;
  if (enc_entries > 0 && (!codes || !enc_values)) return SPOPS_ERR_NULL;
  if (A->rows == 0) return SPOPS_OK;
  return from_hip(launch_delta_encode(A->rows, A->nnz, A->row_offsets, A->col_idx,
                                      A->col_type == SPOPS_I32, A->values, A->val_type,
                                      enc_offsets, enc_entries, codes, enc_values,
                                      as_stream(hip_stream)));
}

spops_status spops_delta_spmv(int64_t rows, int64_t cols, const int32_t* enc_offsets,
                              int64_t enc_entries, const uint32_t* codes, const void* enc_values,
                              spops_dtype val_type, const void* x, void* y, spops_dtype y_type,
                              void* hip_stream) {
  if (!dtype_ok(val_type) || !dtype_ok(y_type)) return SPOPS_ERR_DTYPE;
  if (y_type != SPOPS_F32 && y_type != val_type) return SPOPS_ERR_DTYPE;
  if (rows < 0 || cols < 0 || rows > INT32_MAX - 1 || enc_entries < 0 ||
      enc_entries > INT32_MAX)
    return SPOPS_ERR_SHAPE;
  if (rows == 0) return SPOPS_OK;
  if (!enc_offsets || !y) return SPOPS_ERR_NULL;
  if (enc_entries > 0 && cols == 0) return SPOPS_ERR_SHAPE;
  if (enc_entries > 0 && (!codes || !enc_values || !x)) return SPOPS_ERR_NULL;
  if (((uintptr_t)enc_values % 16) != 0) return SPOPS_ERR_SHAPE;
  return from_hip(launch_delta_spmv(rows, cols, enc_offsets, codes, enc_values, val_type,
                                    enc_entries, x, y, y_type, as_stream(hip_stream)));
}

}  // extern "C"

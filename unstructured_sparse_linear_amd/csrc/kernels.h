// kernels.h -- host-side launchers of the gfx950 kernels (internal to libspops).
// The C ABI layer (api.hip) validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spops {

// Round a byte count up to 256 so sub-buffers carved from one workspace stay
// aligned for vector access.
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// ------------------------------------------------------------------ scan --
// Exclusive prefix sum of n uint32 values (in may equal out).  If `total` is
// non-null the grand total is stored there (device pointer).
size_t scan_workspace_bytes(int64_t n);
hipError_t exclusive_scan_u32(const uint32_t* in, uint32_t* out, int64_t n, uint32_t* total,
                              void* ws, hipStream_t s);

// --------------------------------------------------------- csr transpose --
size_t transpose_workspace_bytes(int64_t rows, int64_t cols, int64_t nnz);
hipError_t launch_csr_transpose(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                                const void* col, int col_i32, const void* val, int val_bytes,
                                void* out_val, int32_t* out_ro, void* out_col, int out_col_i32,
                                void* ws, hipStream_t s);
// The transpose's permutation: out_src[j] = source entry of A^T's entry j
// (out_ro / out_col as launch_csr_transpose); iota: nnz int32 of scratch
// beside the transpose workspace ws.
hipError_t launch_csr_transpose_perm(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                                     const void* col, int col_i32, int32_t* out_src,
                                     int32_t* out_ro, void* out_col, int out_col_i32, void* ws,
                                     int32_t* iota, hipStream_t s);
// out[j] = in[src[j]] for j < n (elem_bytes 2 or 4; src outside [0, n_in): 0).
hipError_t launch_permute_values(const void* in, int64_t n_in, int elem_bytes,
                                 const int32_t* src, int64_t n, void* out, hipStream_t s);

// --------------------------------------------------------- row ordering --
size_t sort_rows_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_sort_rows(const int32_t* ro, int64_t rows, int64_t cols, void* row_idx,
                            int row_idx_i32, void* ws, hipStream_t s);

// Stable sort of n keys in [0, 2^bits) with uint32 payload 0..n-1 (the
// source position).  Results land in sorted_keys / sorted_vals.  Used by the
// plans.  Workspace from radix_pairs_workspace_bytes.
size_t radix_pairs_workspace_bytes(int64_t n);
hipError_t radix_sort_u32_iota(const uint32_t* keys, int64_t n, int bits, uint32_t* sorted_keys,
                               uint32_t* sorted_vals, void* ws, hipStream_t s);
// The same sort leaving its results in the workspace: *sorted_keys and
// *sorted_vals point into ws (no copies).
hipError_t radix_sort_u32_iota_ptrs(const uint32_t* keys, int64_t n, int bits, void* ws,
                                    const uint32_t** sorted_keys, const uint32_t** sorted_vals,
                                    hipStream_t s);

// ------------------------------------------------------------------ SpMM --
// Rows with more entries than the plan's split length are cut into chunks of
// the plan's chunk length, one workgroup per chunk.  Split length:
// kSpmmSplitLenSkewed when the row lengths are skewed and at most 1/32 of the
// rows have more entries than that and at most kSpmmSplitLen, else
// kSpmmSplitLen; a call whose row groups span 32 or more lanes takes rows up
// to kSpmmSplitLen whole anyway (their chunk workgroups return at once).
// Chunk length: the longest row rounded up to a power of two, at most
// kSpmmChunkLenMax, when that leaves at least kSpmmMinChunkItems chunks;
// else kSpmmChunkLen.
constexpr int32_t kSpmmSplitLen = 128;
constexpr int32_t kSpmmSplitLenSkewed = 64;
constexpr int32_t kSpmmChunkLen = 512;
constexpr int32_t kSpmmChunkLenMax = 4096;
constexpr int32_t kSpmmMinChunkItems = 128;
static_assert((kSpmmChunkLen & (kSpmmChunkLen - 1)) == 0 &&
                  (kSpmmChunkLenMax & (kSpmmChunkLenMax - 1)) == 0,
              "chunk lengths are powers of two");

struct SpmmArgs {
  int64_t m, k, nnz, N, ldb, ldc;
  const int32_t* ro;
  const void* col;
  int col_i32;
  const void* val;
  const void* row_idx;
  int ri_i32;
  const void* B;
  void* C;
  int dtype;      // value / B dtype
  int out_dtype;  // C dtype
  int natural;          // 1: whole rows in index order (balanced lengths), 0: row_idx order
  int64_t max_row;      // longest row (from the plan; 0 = unknown)
  // row-splitting schedule (P == 0: none)
  int64_t P;            // number of chunk items of split rows
  int64_t S;            // number of split rows
  int32_t T;            // split length: rows longer than T go to the chunk workgroups
  int32_t CLs;          // chunk length = 1 << CLs (a power of two)
  const int32_t* item_pos;    // [P] position in row_idx of the chunk's row
  const int32_t* item_chunk;  // [P] chunk number within its row
  const int32_t* split_pos;   // [S] position in row_idx of each multi-chunk row
  const int32_t* split_start; // [S] first item of each multi-chunk row
  const int32_t* split_end;   // [S] one past its last item
  float* partial;             // [P][N]
  // N == 1 entry-range blocks (blk_row null: none; see SpmvFlat)
  const int32_t* blk_row;     // [nblk + 1] first row each block owns, then m
  int32_t flat_E, flat_T, flat_U;
};
hipError_t launch_spmm(const SpmmArgs& a, hipStream_t s);

// N == 1 on balanced rows with a plan: workgroup b loads the entries
// [b*E, (b+1)*E + T) (U groups of four per lane, E + T <= U * 1024) and
// writes the rows that start in [b*E, (b+1)*E); blk_row[b] is the first of
// them (the last workgroup also owns the empty rows at the end).  T is the
// longest row rounded up to four, so those rows end inside the loaded range.
constexpr int kFlatMaxRow = 128;     // longest row the entry-range blocks take
constexpr int kFlatMinBlocks = 512;  // U is the largest of 4, 2, 1 giving this many blocks
struct SpmvFlat {
  int32_t E = 0, T = 0, U = 0;
  int64_t blocks = 0;
};
SpmvFlat spmv_flat_shape(int64_t m, int64_t nnz, int64_t max_row, int natural, int64_t P);

// Vector kernels' workgroup size, and groups of four entries per lane per
// round of the SpMV on balanced long rows (spmv_row_kernel).
constexpr int kStreamBlock = 256;
constexpr int kStreamQuads = 2;

// Row-splitting schedule for SpMM, built on the device.  chunk = T.
struct SpmmSchedule {
  int64_t P = 0, S = 0, max_row = 0;
  int natural = 0;  // row lengths balanced enough to keep index order (locality)
  int32_t T = 0;
  int32_t CL = kSpmmChunkLen;
  int32_t* item_pos = nullptr;
  int32_t* item_chunk = nullptr;
  int32_t* split_pos = nullptr;
  int32_t* split_start = nullptr;
  int32_t* split_end = nullptr;
  void* mem = nullptr;  // owning allocation
  SpmvFlat flat;                 // entry-range SpMV blocks (flat.U == 0: none)
  int32_t* blk_row = nullptr;    // [flat.blocks + 1], own allocation
};
hipError_t build_spmm_schedule(const int32_t* ro, const void* row_idx, int ri_i32, int64_t m,
                               int64_t nnz, int32_t T, SpmmSchedule* out, hipStream_t s);
void free_spmm_schedule(SpmmSchedule* sch);

// ----------------------------------------------------------------- SDDMM --
// Scalar kernel of the general backend, for K, leading dimensions or
// pointers that do not allow 16-byte vectors along K (mask in CSR order).
struct SddmmArgs {
  int64_t m, n, K, lda, ldbt;
  const int32_t* ro;     // mask row offsets
  int64_t count;         // mask entries (== ro[m])
  const void* col;       // mask column indices
  int col_i32;
  const void* A;
  const void* BT;
  void* out;             // [count], CSR order
  int dtype, out_dtype;
};
hipError_t launch_sddmm_general(const SddmmArgs& a, hipStream_t s);

// Structure-aware SDDMM plan.  Dense tiles are kSddmmTM x kSddmmTN blocks of
// gathered rows x gathered columns; tile t's entries carry the key t, the
// remainder the keys rest_key + column bucket.
constexpr int kMaxBuckets = 8;
constexpr int kSddmmTM = 128;
constexpr int kSddmmTN = 128;

// Counts the plan kernels write to device memory.
struct SddmmPlanScalars {
  int32_t H;             // dense rows
  int32_t mc;            // the other rows
  int32_t Hc;            // dense columns (counted over the other rows)
  int32_t tiles_a;       // tiles of region A (dense rows x all columns)
  int32_t tiles_b_cols;  // tile columns of region B (other rows x dense columns)
  int32_t tiles;         // all tiles
  int32_t tiled;         // entries inside tiles
  int32_t rest;          // remainder entries
  int32_t nb;            // remainder column buckets after the merge decision
  uint32_t rest_count;   // classifier's running count of remainder entries
  int32_t pad[6];
};

struct SddmmPlanDev {
  int64_t m = 0, n = 0, nnz = 0;
  double tau = 0;
  int64_t tiles_a_cols = 0;  // tile columns of region A: cdiv(n, kSddmmTN)
  int64_t max_tiles = 0;     // bound on the tile count (sizes the key space)
  int64_t rest_key = 0;      // first remainder key (max_tiles)
  int nb_max = 1;            // remainder buckets planned before the merge decision
  SddmmPlanScalars* sc = nullptr;  // device
  int32_t* rows = nullptr;         // [m] dense rows, then the other rows
  int32_t* hot_cols = nullptr;     // [n] dense columns
  int32_t* key_start = nullptr;    // [rest_key + nb_max + 1] first sorted entry per key
  int32_t* ent_pos = nullptr;      // [nnz] mask position of each sorted entry
  int32_t* ent_rc = nullptr;       // [nnz] (tile row << 16) | tile column; remainder: row
  int32_t* ent_col = nullptr;      // [nnz] mask column of each sorted entry (as stored)
  // the remainder in row order (its first `rest` entries), for K in pieces
  int32_t* row_pos = nullptr;      // [nnz] mask position
  int32_t* row_rc = nullptr;       // [nnz] row
  int32_t* row_col = nullptr;      // [nnz] mask column
  // host copy of the counts (plans made by spops_sddmm_plan_create)
  bool host_ok = false;
  SddmmPlanScalars h{};
  int64_t bucket_start[kMaxBuckets + 1] = {};  // absolute entry positions of the buckets
  int64_t max_tile_nnz = 0;        // most entries in one tile (host counts)
  int cus = 256;                   // compute units of the device
  void* mem = nullptr;             // owning allocation (null when carved from a workspace)
  // identity of the mask it was built for
  const void* mask_ro = nullptr;
  const void* mask_col = nullptr;
};
// Device memory of a plan (kept) and of its build (temporary).
size_t sddmm_plan_bytes(int64_t m, int64_t n, int64_t nnz);
size_t sddmm_plan_scratch_bytes(int64_t m, int64_t n, int64_t nnz);
// Enqueues the plan's kernels on s (no allocation, no synchronization): the
// plan's arrays are carved from `mem` (sddmm_plan_bytes), temporaries from
// `scratch` (sddmm_plan_scratch_bytes).  Fills *out (counts stay on the
// device; out->host_ok false).  A dense row or column also needs at least
// min_count entries (1 = the tau rule alone).
hipError_t enqueue_sddmm_plan(int64_t m, int64_t n, int64_t nnz, const int32_t* ro,
                              const void* col, int col_i32, double tau, int64_t min_count,
                              void* mem, void* scratch, SddmmPlanDev* out, hipStream_t s);
// Copies the counts to the host (synchronizes s).
hipError_t fetch_sddmm_plan_counts(SddmmPlanDev* p, hipStream_t s);
// Work schedule of the dense tiles for a plan and K, and the fp32 partial
// sums it needs (bytes).
struct SddmmTileSched {
  int splits;     // K splits per tile (1: a tile is one item)
};
SddmmTileSched sddmm_tile_schedule(const SddmmPlanDev& p, int64_t K);
size_t sddmm_split_bytes(const SddmmPlanDev& p, const SddmmTileSched& sched);
// Dense tiles (with several splits: partial sums into part, then their
// fixed-order sum into out).
hipError_t launch_sddmm_tiles(const SddmmPlanDev& p, int64_t K, const void* A, int64_t lda,
                              const void* BT, int64_t ldbt, int dtype, void* out, int out_dtype,
                              const SddmmTileSched& sched, float* part, hipStream_t s);

// General SDDMM over an entry list: entry j is mask position pos[j] in row
// rows[j]; entries of bucket b are [bstart[b], bstart[b+1]) and run on the
// blocks b, b+nb, ... (which share XCD b when nb is 8).
struct SddmmListArgs {
  int64_t m, n, K, lda, ldbt;
  // CSR order when ro is set: entry j is mask position j, its row is found in
  // ro (pos and rows unused, one bucket [0, nnz))
  const int32_t* ro;
  const int32_t* pos;
  const int32_t* rows;
  // column of each list entry as stored in the mask (nullable: col[pos] is
  // loaded instead, one load later)
  const int32_t* cols;
  const void* col;
  int col_i32;
  const void* A;
  const void* BT;
  void* out;
  int dtype, out_dtype;
  int nb;
  int64_t bstart[kMaxBuckets + 1];
  // bucket bounds in device memory instead of bstart (nullable); max_bucket
  // bounds the entries of one bucket
  const int32_t* bstart_dev;
  int64_t max_bucket;
  // K split (ksplit > 1, nb == ksplit): bucket b is piece b of K (kpiece
  // elements at offset b * kpiece) over all entries of bucket 0's range; the
  // piece's fp32 dot products go to part[b * (range length) + entry - start]
  int ksplit;
  int64_t kpiece;
  float* part;
};
hipError_t launch_sddmm_list(const SddmmListArgs& a, hipStream_t s);
// out[pos[j]] = sum over pieces b (in order) of part[b * count + j - start]
// for the entries j in [start, start + count) of a K-split list.
hipError_t launch_sddmm_piece_sum(const float* part, int pieces, int64_t count,
                                  const int32_t* pos, int64_t start, void* out, int out_dtype,
                                  hipStream_t s);

// ------------------------------------------------------------ validation --
// Findings of the CSR validator (bits of a flag word).
constexpr uint32_t kValidateBadOffsets = 1u;
constexpr uint32_t kValidateBadColumn = 2u;
constexpr uint32_t kValidateBadRowIdx = 4u;
constexpr uint32_t kValidateDuplicate = 8u;
size_t validate_workspace_bytes(int64_t rows, int64_t cols, int64_t nnz);
// Runs the checks and copies the flag word to *flags_host (synchronizes s).
hipError_t launch_validate(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                           const void* col, int col_i32, const void* row_idx, int ri_i32,
                           int check_duplicates, void* ws, uint32_t* flags_host,
                           hipStream_t s);

// ------------------------------------------------------------- options --
// Process-wide switches (spops_set_option), read on every call.
enum Option : int {
  kOptSpmmPointerLoads = 0,
  kOptTransposeForceScan = 1,
  kOptTransposeWideRecords = 2,
  kOptSddmmBuckets = 3,
  kOptSddmmSplits = 4,
  kOptSddmmRestSplit = 5,
  kOptCount = 6
};
int64_t option(int o);

// --------------------------------------------------------------- csr_add --
hipError_t launch_csr_add(int64_t m, int64_t n, int64_t nnz, const int32_t* ro, const void* col,
                          int col_i32, const void* val, void* W, int64_t ldw, int dtype,
                          hipStream_t s);

// ------------------------------------------------- conjugate gradients --
// Solver state in device memory (written by the solver's kernels, read by
// the host at its convergence checks).
struct CgState {
  double rr[2];    // r.r after iteration k at rr[k & 1]
  double bb;       // b.b
  double thr;      // rtol^2 * b.b
  int64_t iters;   // iterations completed
  int32_t done;    // 0 running, 1 converged, 2 stopped (p.q not positive)
  int32_t pad;
};
constexpr int kCgMaxParts = 1024;  // most per-workgroup partial sums of a vector kernel
struct CgBuffers {
  float2* pr[2];           // [m] each: (p, r) pairs, alternating between iterations
  float* q;                // [m]
  double* part_pq;         // partials of p.q (one per SpMV row block when fused)
  double* part_rr;         // [kCgMaxParts] partials of r.r
  CgState* st;
  void* spmm_ws;           // the SpMV's own workspace
};
// Workspace of the solver for m unknowns, npq partials of p.q (the fused
// SpMV's grid, else 0) and an SpMV workspace of spmm_ws bytes, and its split
// into buffers (256-byte aligned pieces).
size_t cg_workspace_bytes(int64_t m, int64_t npq, size_t spmm_ws);
CgBuffers carve_cg_workspace(void* ws, int64_t m, int64_t npq);
int cg_parts(int64_t m);
// Set-up once q = A x0 is in w.q: r = b - q, state for iteration 0.
hipError_t launch_cg_init(int64_t m, const float* b, const CgBuffers& w, double rtol,
                          hipStream_t s);
// Records r.r and the iteration count k in the state (before a host check).
hipError_t launch_cg_record(int64_t m, int64_t k, const CgBuffers& w, hipStream_t s);
// Iteration k around the library's SpMV: direction into the p slots of
// w.pr[(k+1)&1], then (after q = A p) p.q and the x / r update.
hipError_t launch_cg_direction(int64_t m, int64_t k, const CgBuffers& w, hipStream_t s);
hipError_t launch_cg_dot_update(int64_t m, int64_t k, float* x, const CgBuffers& w,
                                hipStream_t s);
// Iteration k as row blocks (SpMV fused with the direction and p.q), then
// the update: two launches.  The CSR (f32 values) comes in `a`; the buffer
// fields are filled from w.
struct CgSpmvArgs {
  int64_t m, nnz, k;
  const int32_t* ro;
  const void* col;
  int col_i32;
  const float* val;
  const float2* pr;        // (p_prev, r) pairs read
  float2* pr_next;         // p written to its x slots
  float* q;
  double* part_pq;
  const double* part_rr;
  int nparts_rr;
  CgState* st;
  // entry-range blocks of the plan (SpmvFlat)
  const int32_t* blk_row;
  int32_t E, T, U;
};
// p.q partials of the fused iteration: one per workgroup of the grid.
int64_t cg_fused_grid(int64_t nnz, int32_t E);
hipError_t launch_cg_fused(const CgSpmvArgs& a, float* x, const CgBuffers& w, hipStream_t s);

// ------------------------------------------------------------ masked Adam --
struct AdamArgs {
  int64_t nnz;             // length of values / exp_avg / exp_avg_sq
  int64_t ngrad;           // gradient entries
  const int32_t* positions;  // [ngrad] value index of each gradient entry, or null (j -> j)
  void* values;
  const void* grad;        // [ngrad], values' dtype
  float* exp_avg;
  float* exp_avg_sq;
  float beta1, beta2, one_minus_beta1, one_minus_beta2, alpha_t, eps;
  int maximize;
};
hipError_t launch_masked_adam(const AdamArgs& a, int dtype, hipStream_t s);

// ------------------------------------------------- delta-coded rows --
size_t delta_size_workspace_bytes(int64_t m);
// Encoded row lengths -> enc_offsets[m+1]; copies enc_offsets[m] and a flag
// (columns not strictly ascending / out of range) to total_and_bad[0..1]
// (host memory; valid after the stream synchronizes).
hipError_t launch_delta_size(int64_t m, int64_t n, int64_t nnz, const int32_t* ro,
                             const void* col, int col_i32, int32_t* enc_offsets, void* ws,
                             uint32_t* total_and_bad, hipStream_t s);
hipError_t launch_delta_encode(int64_t m, int64_t nnz, const int32_t* ro, const void* col,
                               int col_i32, const void* val, int dtype, const int32_t* eo,
                               int64_t total, uint32_t* codes, void* out, hipStream_t s);
hipError_t launch_delta_spmv(int64_t m, int64_t n, const int32_t* eo, const uint32_t* codes,
                             const void* val, int dtype, int64_t total, const void* x, void* y,
                             int y_dtype, hipStream_t s);

}  // namespace spops

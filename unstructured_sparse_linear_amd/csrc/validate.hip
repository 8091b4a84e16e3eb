// validate.hip -- device-side checks of a CSR matrix against the layout of
// the spops README (section "Usage": row offsets, column indices, a row_idx
// permutation of the rows; section "Important Notes": index types).
//
// Checks (each sets one bit of a flag word in device memory):
//   kBadOffsets   row_offsets[0] != 0, row_offsets[rows] != nnz, or a row
//                 whose end lies before its start;
//   kBadColumn    a column index outside [0, cols);
//   kBadRowIdx    row_idx holds a value outside [0, rows) or a row twice
//                 (then some row is missing: not a permutation);
//   kDuplicate    a (row, column) pair stored twice.
// Every read stays inside the lengths passed in: row offsets are clamped to
// [0, nnz] before they index anything.  Duplicates are found on the
// transpose of the pattern (a stable sort by column keeps each column's
// source rows in ascending order, so a repeated pair shows up as two equal
// neighbours); that step runs only when offsets and columns are valid.
#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

__global__ void validate_init_kernel(uint32_t* flags) {
  if (threadIdx.x == 0) flags[0] = 0u;
}

// One thread per row r in [0, rows]: offsets monotone, ends match.
__global__ void validate_offsets_kernel(const int32_t* ro, int64_t rows, int64_t nnz,
                                        uint32_t* flags) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r > rows) return;
  bool bad = false;
  if (r == 0) bad |= ro[0] != 0;
  if (r == rows) bad |= (int64_t)ro[rows] != nnz;
  if (r < rows) bad |= ro[r + 1] < ro[r] || ro[r] < 0 || (int64_t)ro[r + 1] > nnz;
  if (bad) atomicOr(flags, kValidateBadOffsets);
}

// One thread per stored entry: column in range.
template <typename IT>
__global__ void validate_cols_kernel(const IT* col, int64_t nnz, int64_t cols, uint32_t* flags) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= nnz) return;
  const int64_t c = (int64_t)col[p];
  if (c < 0 || c >= cols) atomicOr(flags, kValidateBadColumn);
}

__global__ void validate_zero_kernel(uint32_t* cnt, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) cnt[i] = 0u;
}

// row_idx: each value in range, counted.
template <typename IT>
__global__ void validate_perm_count_kernel(const IT* ri, int64_t rows, uint32_t* cnt,
                                           uint32_t* flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  const int64_t v = (int64_t)ri[i];
  if (v < 0 || v >= rows)
    atomicOr(flags, kValidateBadRowIdx);
  else
    atomicAdd(&cnt[v], 1u);
}

__global__ void validate_perm_check_kernel(const uint32_t* cnt, int64_t rows, uint32_t* flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < rows && cnt[i] != 1u) atomicOr(flags, kValidateBadRowIdx);
}

// On the transposed pattern (rows of A^T = columns of A, entries = source
// rows in ascending order): equal neighbours inside a column are a
// duplicate (row, column) pair.  Skipped unless offsets and columns passed.
template <typename OT>
__global__ void validate_dup_kernel(const int32_t* ro_t, const OT* ci_t, int64_t cols,
                                    int64_t nnz, uint32_t* flags) {
  if (flags[0] & (kValidateBadOffsets | kValidateBadColumn)) return;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nnz || q == 0) return;
  // q and q - 1 in the same output row?  Find q's row by the offsets of
  // its neighbours: a boundary lies between them when some ro_t[c] == q.
  // Binary search for the largest c with ro_t[c] <= q - 1.
  int64_t lo = 0, hi = cols;  // ro_t[0] = 0 <= q - 1
  while (hi - lo > 1) {
    const int64_t mid = lo + ((hi - lo) >> 1);
    if ((int64_t)ro_t[mid] <= q - 1)
      lo = mid;
    else
      hi = mid;
  }
  const bool same_col = (int64_t)ro_t[lo + 1] > q;  // q - 1 and q both in column lo
  if (same_col && ci_t[q] == ci_t[q - 1]) atomicOr(flags, kValidateDuplicate);
}

struct ValidateWs {
  uint32_t* flags;
  uint32_t* cnt;
  int32_t* ro_t;
  int32_t* ci_t;
  void* tws;
};

ValidateWs carve(void* ws, int64_t rows, int64_t cols, int64_t nnz) {
  char* p = (char*)ws;
  ValidateWs w{};
  w.flags = (uint32_t*)p;
  p += 256;
  w.cnt = (uint32_t*)p;
  p += align256((size_t)(rows > 0 ? rows : 1) * 4);
  w.ro_t = (int32_t*)p;
  p += align256((size_t)(cols + 1) * 4);
  w.ci_t = (int32_t*)p;
  p += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  w.tws = p;
  return w;
}

}  // namespace

size_t validate_workspace_bytes(int64_t rows, int64_t cols, int64_t nnz) {
  return 256 + align256((size_t)(rows > 0 ? rows : 1) * 4) + align256((size_t)(cols + 1) * 4) +
         align256((size_t)(nnz > 0 ? nnz : 1) * 4) +
         align256(transpose_workspace_bytes(rows, cols, nnz));
}

hipError_t launch_validate(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                           const void* col, int col_i32, const void* row_idx, int ri_i32,
                           int check_duplicates, void* ws, uint32_t* flags_host,
                           hipStream_t s) {
  ValidateWs w = carve(ws, rows, cols, nnz);
  hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, s, w.flags);
  hipLaunchKernelGGL(validate_offsets_kernel, dim3((unsigned)cdiv(rows + 1, 256)), dim3(256), 0,
                     s, ro, rows, nnz, w.flags);
  if (nnz > 0) {
    const dim3 g((unsigned)cdiv(nnz, 256));
    if (col_i32)
      hipLaunchKernelGGL(validate_cols_kernel<int32_t>, g, dim3(256), 0, s,
                         (const int32_t*)col, nnz, cols, w.flags);
    else
      hipLaunchKernelGGL(validate_cols_kernel<int16_t>, g, dim3(256), 0, s,
                         (const int16_t*)col, nnz, cols, w.flags);
  }
  if (row_idx && rows > 0) {
    const dim3 g((unsigned)cdiv(rows, 256));
    hipLaunchKernelGGL(validate_zero_kernel, g, dim3(256), 0, s, w.cnt, rows);
    if (ri_i32)
      hipLaunchKernelGGL(validate_perm_count_kernel<int32_t>, g, dim3(256), 0, s,
                         (const int32_t*)row_idx, rows, w.cnt, w.flags);
    else
      hipLaunchKernelGGL(validate_perm_count_kernel<int16_t>, g, dim3(256), 0, s,
                         (const int16_t*)row_idx, rows, w.cnt, w.flags);
    hipLaunchKernelGGL(validate_perm_check_kernel, g, dim3(256), 0, s, w.cnt, rows, w.flags);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (check_duplicates && nnz > 1 && cols > 0) {
    // The transpose reads the offsets and columns, so it may run only on
    // valid ones: read the flags first.
    uint32_t f = 0;
    if ((e = hipMemcpyAsync(&f, w.flags, 4, hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    if (!(f & (kValidateBadOffsets | kValidateBadColumn))) {
      if ((e = launch_csr_transpose(rows, cols, nnz, ro, col, col_i32, nullptr, 0, nullptr,
                                    w.ro_t, w.ci_t, 1, w.tws, s)) != hipSuccess)
        return e;
      hipLaunchKernelGGL(validate_dup_kernel<int32_t>, dim3((unsigned)cdiv(nnz, 256)), dim3(256),
                         0, s, w.ro_t, w.ci_t, cols, nnz, w.flags);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if ((e = hipMemcpyAsync(flags_host, w.flags, 4, hipMemcpyDeviceToHost, s)) != hipSuccess)
    return e;
  return hipStreamSynchronize(s);
}

}  // namespace spops

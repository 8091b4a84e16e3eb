// csr_add.hip -- W += A in place for a CSR matrix A and a dense row-major W
// on gfx950 (spops README, section "Sparse Addition").
//
// Each stored entry (r, c, v) is an independent read-modify-write of one
// element of W: the sum is formed in fp32 and rounded once to W's format.
// For f16 and bf16 that equals the correctly rounded sum, since an fp32
// intermediate (24 bits) is at least 2p+1 bits for p = 11 or 8 (Figueroa,
// "When is double rounding innocuous?", 1995); for f32 it is the single
// rounding itself.  Entries are spread evenly over lanes (one entry per lane
// per round, consecutive entries on consecutive lanes), which keeps rows of
// any length balanced; each lane finds its row by a binary search between the
// rows of the wave's first and last entries.  Entries are unique within a row, so no two
// lanes touch the same element.
#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int kBlock = 256;

template <typename VT, typename IT, int kRounds>
__global__ __launch_bounds__(kBlock) void csr_add_kernel(int64_t m, int64_t n, int64_t nnz,
                                                         const int32_t* ro, const IT* col,
                                                         const VT* val, VT* W, int64_t ldw) {
  const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int64_t wb = wave * (kWave * kRounds);
  if (wb >= nnz) return;
  const int64_t we = (wb + kWave * kRounds < nnz ? wb + kWave * kRounds : nnz) - 1;
  // rows of the wave's first and last entries (64-way searches), then each
  // lane's row by binary search between them: a bounded number of loads
  // however many empty rows the wave's entries span
  const int64_t rf = wave_upper_row(ro, m, wb);
  const int64_t rl = wave_upper_row(ro, m, we);
  const int lane = lane_id();
  // all loads of W first (positions are distinct), then the stores
  int64_t off[kRounds];
  float add[kRounds];
  VT old[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int64_t p = wb + q * kWave + lane;
    off[q] = -1;
    add[q] = 0.f;
    if (p < nnz) {
      const int64_t r = upper_row(ro, rf, rl + 1, p);
      const int c = (int)col[p];
      if ((unsigned)c < (unsigned)n) {
        off[q] = r * ldw + c;
        add[q] = to_f32(val[p]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kRounds; ++q)
    if (off[q] >= 0) old[q] = W[off[q]];
#pragma unroll
  for (int q = 0; q < kRounds; ++q)
    if (off[q] >= 0) W[off[q]] = from_f32<VT>(to_f32(old[q]) + add[q]);
}

template <typename VT, int kRounds>
hipError_t launch_vtr(int64_t m, int64_t n, int64_t nnz, const int32_t* ro, const void* col,
                      int col_i32, const void* val, void* W, int64_t ldw, hipStream_t s) {
  const int64_t waves = (nnz + kWave * kRounds - 1) / (kWave * kRounds);
  const dim3 grid((unsigned)((waves * kWave + kBlock - 1) / kBlock));
  if (col_i32)
    hipLaunchKernelGGL((csr_add_kernel<VT, int32_t, kRounds>), grid, dim3(kBlock), 0, s, m, n,
                       nnz, ro, (const int32_t*)col, (const VT*)val, (VT*)W, ldw);
  else
    hipLaunchKernelGGL((csr_add_kernel<VT, int16_t, kRounds>), grid, dim3(kBlock), 0, s, m, n,
                       nnz, ro, (const int16_t*)col, (const VT*)val, (VT*)W, ldw);
  return hipGetLastError();
}

// One entry per lane: the kernel is bound by the latency of its dependent
// loads (row search, W read), so more waves in flight beat more entries per
// lane (measured 1, 2, 4, 8 entries per lane on MI355X; 1 was fastest).
template <typename VT>
hipError_t launch_vt(int64_t m, int64_t n, int64_t nnz, const int32_t* ro, const void* col,
                     int col_i32, const void* val, void* W, int64_t ldw, hipStream_t s) {
  return launch_vtr<VT, 1>(m, n, nnz, ro, col, col_i32, val, W, ldw, s);
}

}  // namespace

hipError_t launch_csr_add(int64_t m, int64_t n, int64_t nnz, const int32_t* ro, const void* col,
                          int col_i32, const void* val, void* W, int64_t ldw, int dtype,
                          hipStream_t s) {
  if (nnz <= 0 || m <= 0) return hipSuccess;
  switch (dtype) {
    case kF32: return launch_vt<float>(m, n, nnz, ro, col, col_i32, val, W, ldw, s);
    case kF16: return launch_vt<_Float16>(m, n, nnz, ro, col, col_i32, val, W, ldw, s);
    case kBF16: return launch_vt<bf16_t>(m, n, nnz, ro, col, col_i32, val, W, ldw, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spops

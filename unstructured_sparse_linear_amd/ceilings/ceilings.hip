// ceilings.hip -- measurement kernels for bench.py (a separate library,
// libspops_ceilings.so; nothing in libspops uses it).
//
// The SpMM and SDDMM kernels are bound by how fast the chip can gather whole
// operand rows (16-byte lanes, one row per wave per step) from L2 or from the
// Infinity Cache, not by HBM streaming.  These kernels measure that rate for
// the row sizes the operations use, so the benchmark can report each
// kernel's rate against it next to the HBM roofline:
//   * gather_kernel<ROWB, SLICED>: every wave gathers `per_wave` rows of ROWB
//     bytes at the given indices; with SLICED each workgroup reads only the
//     slice of the source that belongs to its XCD (workgroup b runs on XCD
//     b mod 8), so the slice can stay in that XCD's L2; without it all
//     workgroups share the whole source.  Lanes fold what they load into one
//     word each, stored once, so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBlock = 256;
constexpr int kWave = 64;
constexpr int kInFlight = 8;  // rows whose loads a lane issues together

// Rows of 512 bytes take half a wave each (two rows per step); larger rows
// take the whole wave, ROWB / 1024 loads per lane.
template <int ROWB, bool SLICED>
__global__ __launch_bounds__(kBlock) void gather_kernel(const uint4* src, int64_t slice_rows,
                                                        const int32_t* idx, int64_t per_wave,
                                                        uint32_t* sink) {
  constexpr int kLanesPerRow = ROWB / 16 < kWave ? ROWB / 16 : kWave;
  constexpr int kRowsPerStep = kWave / kLanesPerRow;
  constexpr int kVecs = ROWB / 16 / kLanesPerRow;  // 16-byte loads per lane per row
  const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int lane = threadIdx.x % kWave;
  const int sub = lane / kLanesPerRow, ln = lane % kLanesPerRow;
  const uint4* base = SLICED ? src + (int64_t)(blockIdx.x % 8) * slice_rows * (ROWB / 16) : src;
  const int32_t* my = idx + wave * per_wave;
  uint32_t acc = 0;
  for (int64_t i = 0; i < per_wave; i += kInFlight * kRowsPerStep) {
    uint4 v[kInFlight][kVecs];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t row = my[i + u * kRowsPerStep + sub];
      const uint4* p = base + row * (ROWB / 16) + ln;
#pragma unroll
      for (int q = 0; q < kVecs; ++q) v[u][q] = p[q * kLanesPerRow];
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
#pragma unroll
      for (int q = 0; q < kVecs; ++q) acc ^= v[u][q].x ^ v[u][q].y ^ v[u][q].z ^ v[u][q].w;
  }
  sink[(int64_t)blockIdx.x * kBlock + threadIdx.x] = acc;
}

}  // namespace

// Gathers: blocks x 256 threads, each wave `per_wave` rows (a multiple of 16)
// of row_bytes (512, 1024 or 4096) from src at idx[wave * per_wave + i] (row
// numbers below slice_rows).  sliced != 0: workgroup b reads slice b mod 8
// (slice_rows rows each).  sink: blocks * 256 words.  Returns 0, or -1 for
// an unsupported row size.
extern "C" int spops_ceil_gather(const void* src, int64_t slice_rows, int row_bytes, int sliced,
                                 const int32_t* idx, int64_t per_wave, int blocks, void* sink,
                                 void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const uint4* p = (const uint4*)src;
  uint32_t* o = (uint32_t*)sink;
  if (per_wave % (2 * kInFlight) != 0) return -1;
#define LAUNCH(RB, SL)                                                                        \
  hipLaunchKernelGGL((gather_kernel<RB, SL>), dim3(blocks), dim3(kBlock), 0, s, p, slice_rows, \
                     idx, per_wave, o)
  if (row_bytes == 512) {
    if (sliced) LAUNCH(512, true); else LAUNCH(512, false);
  } else if (row_bytes == 1024) {
    if (sliced) LAUNCH(1024, true); else LAUNCH(1024, false);
  } else if (row_bytes == 4096) {
    if (sliced) LAUNCH(4096, true); else LAUNCH(4096, false);
  } else {
    return -1;
  }
#undef LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

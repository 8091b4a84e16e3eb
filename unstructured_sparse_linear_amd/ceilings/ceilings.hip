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
// and the on-chip rates the kernels' inner loops run against:
//   * lds_kernel: 16-byte LDS reads, consecutive lanes at consecutive
//     16-byte words (no bank conflicts), eight per lane per step;
//   * fma_kernel: v_fma_f32, eight independent chains per lane;
//   * dot2_kernel: v_dot2_f32_f16 (two products and their sum into an fp32
//     accumulator), eight independent chains per lane.
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

constexpr int kLdsVecs = 1024;  // 16 KiB of LDS per workgroup

__global__ __launch_bounds__(kBlock) void lds_kernel(int64_t iters, uint32_t* sink) {
  __shared__ uint4 buf[kLdsVecs];
  const int t = threadIdx.x;
  for (int i = t; i < kLdsVecs; i += kBlock) buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
  __syncthreads();
  uint32_t acc = 0;
  for (int64_t i = 0; i < iters; ++i) {
    const int base = t + (int)(i & 3) * 32;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = buf[(base + u * 128) & (kLdsVecs - 1)];
      acc += v.x + v.y + v.z + v.w;
    }
  }
  sink[(int64_t)blockIdx.x * kBlock + t] = acc;
}

__global__ __launch_bounds__(kBlock) void fma_kernel(int64_t iters, float x, float y,
                                                     float* sink) {
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (float)threadIdx.x * 1e-3f + (float)j;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = __builtin_fmaf(a[j], x, y);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  sink[(int64_t)blockIdx.x * kBlock + threadIdx.x] = s;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kBlock) void dot2_kernel(int64_t iters, uint32_t xbits,
                                                      float* sink) {
  const half2v x = __builtin_bit_cast(half2v, xbits);
  half2v b[8];
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    b[j] = half2v{(_Float16)(threadIdx.x & 15), (_Float16)j};
    a[j] = (float)j;
  }
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = __builtin_amdgcn_fdot2(b[j], x, a[j], false);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  sink[(int64_t)blockIdx.x * kBlock + threadIdx.x] = s;
}

}  // namespace

// LDS reads: blocks x 256 threads, each iters x 8 reads of 16 bytes (iters x
// 128 bytes per thread).  sink: blocks * 256 words.
extern "C" int spops_ceil_lds(int blocks, int64_t iters, void* sink, void* stream) {
  if (blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(lds_kernel, dim3(blocks), dim3(kBlock), 0, (hipStream_t)stream, iters,
                     (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// VALU rates: blocks x 256 threads, each iters x 32 instructions; kind 0:
// v_fma_f32 (2 flops each), kind 1: v_dot2_f32_f16 (4 flops each).  sink:
// blocks * 256 floats.
extern "C" int spops_ceil_valu(int kind, int blocks, int64_t iters, void* sink, void* stream) {
  if (blocks <= 0 || iters <= 0) return -1;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(fma_kernel, dim3(blocks), dim3(kBlock), 0, s, iters, 0.999f, 1e-3f,
                       (float*)sink);
  else if (kind == 1)
    hipLaunchKernelGGL(dot2_kernel, dim3(blocks), dim3(kBlock), 0, s, iters, 0x3bff3bffu,
                       (float*)sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

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

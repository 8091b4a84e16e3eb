// spmm.hip -- C = A * B for a CSR matrix A and a dense row-major B on gfx950
// (spops README, section "Sparse Matrix Multiplication (SpMM)").
//
// Work mapping.  Rows are visited in row_idx order (section "Usage": rows
// sorted by entry count), so neighbouring groups of lanes get rows of similar
// length and the longest rows start first.  A group of LPR lanes owns one row
// and a window of LPR*VEC columns of C; each lane keeps VEC fp32 accumulators
// and streams the row's entries, loading 16-byte vectors of the B rows it
// needs (coalesced across the group) and multiplying by the entry value.
//
// Long rows.  A plan (see build_spmm_schedule) lists the rows longer than
// kSpmmSplitLen in row_idx order and cuts each into chunks of kChunkLen entries.
// Each chunk is one workgroup: its groups take contiguous slices of the chunk
// and are summed in LDS in group order.  A row with one chunk is written
// directly; a row with several writes fp32 partial rows that a second kernel
// adds in chunk order.  All sums therefore have a fixed order and results are
// bitwise reproducible.
//
// N == 1 (SpMV) uses a different split: the lanes of a group stride over the
// row's entries and are combined with a fixed xor-shuffle tree.
#include "common.h"
#include "kernels.h"

namespace spops {

constexpr int32_t kChunkLen = kSpmmChunkLen;

namespace {

constexpr int kBlock = 256;


template <typename T>
struct Vec16;  // 16 bytes of elements
template <>
struct Vec16<float> {
  static constexpr int n = 4;
};
template <>
struct Vec16<_Float16> {
  static constexpr int n = 8;
};
template <>
struct Vec16<bf16_t> {
  static constexpr int n = 8;
};

// acc[e] += v * B[e] for one 16-byte vector of B.
template <typename VT>
__device__ __forceinline__ void fma_vec(float* acc, float v, const uint4& w) {
  if constexpr (Vec16<VT>::n == 4) {
    acc[0] = __builtin_fmaf(v, __uint_as_float(w.x), acc[0]);
    acc[1] = __builtin_fmaf(v, __uint_as_float(w.y), acc[1]);
    acc[2] = __builtin_fmaf(v, __uint_as_float(w.z), acc[2]);
    acc[3] = __builtin_fmaf(v, __uint_as_float(w.w), acc[3]);
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = __builtin_fmaf(v, lo_f32(ws[q], (VT*)nullptr), acc[2 * q]);
      acc[2 * q + 1] = __builtin_fmaf(v, hi_f32(ws[q], (VT*)nullptr), acc[2 * q + 1]);
    }
  }
}

template <typename OT, int VEC>
__device__ __forceinline__ void store_vec(OT* dst, const float* acc) {
  if constexpr (sizeof(OT) == 4) {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q)
      *(float4*)(dst + 4 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2],
                                            acc[4 * q + 3]);
  } else {
    static_assert(VEC == 8, "16-bit outputs use 8-wide vectors");
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)bits16(from_f32<OT>(acc[2 * q])) |
             ((uint32_t)bits16(from_f32<OT>(acc[2 * q + 1])) << 16);
    *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ int64_t load_row(const void* ri, int ri_i32, int64_t i) {
  return ri_i32 ? (int64_t)((const int32_t*)ri)[i] : (int64_t)((const int16_t*)ri)[i];
}

// Row r's entry range, clamped to [0, nnz].
__device__ __forceinline__ void row_range(const int32_t* ro, int64_t r, int64_t nnz,
                                          int64_t& p0, int64_t& p1) {
  p0 = ro[r];
  p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > nnz ? nnz : p1);
}

// Accumulate entries [p0, p1) into acc for columns [j, j+VEC).
template <typename VT, typename IT, int VEC, bool ALIGNED>
__device__ __forceinline__ void accumulate(const SpmmArgs& a, int64_t p0, int64_t p1, int64_t j,
                                           float* acc) {
  const IT* col = (const IT*)a.col;
  const VT* val = (const VT*)a.val;
  const VT* B = (const VT*)a.B;
  const int64_t k = a.k;
  if constexpr (ALIGNED) {
    if (j >= a.N) return;
    constexpr int U = 4;
    int64_t p = p0;
    for (; p + U <= p1; p += U) {
      int c[U];
      float v[U];
      uint4 b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        c[u] = (int)col[p + u];
        v[u] = to_f32(val[p + u]);
        if ((unsigned)c[u] >= (unsigned)k) {
          c[u] = 0;
          v[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = *(const uint4*)(B + (int64_t)c[u] * a.ldb + j);
#pragma unroll
      for (int u = 0; u < U; ++u) fma_vec<VT>(acc, v[u], b[u]);
    }
    for (; p < p1; ++p) {
      int c = (int)col[p];
      float v = to_f32(val[p]);
      if ((unsigned)c >= (unsigned)k) {
        c = 0;
        v = 0.f;
      }
      uint4 b = *(const uint4*)(B + (int64_t)c * a.ldb + j);
      fma_vec<VT>(acc, v, b);
    }
  } else {
    static_assert(VEC == 1, "unaligned path is scalar");
    if (j >= a.N) return;
    for (int64_t p = p0; p < p1; ++p) {
      int c = (int)col[p];
      if ((unsigned)c >= (unsigned)k) continue;
      acc[0] = __builtin_fmaf(to_f32(val[p]), to_f32(B[(int64_t)c * a.ldb + j]), acc[0]);
    }
  }
}

template <typename OT, int VEC, bool ALIGNED>
__device__ __forceinline__ void write_out(OT* dst, int64_t j, int64_t N, const float* acc) {
  if (j >= N) return;
  if constexpr (ALIGNED) {
    store_vec<OT, VEC>(dst + j, acc);
  } else {
    dst[j] = from_f32<OT>(acc[0]);
  }
}

// Blocks [0, P): one chunk of a long row each.  Blocks [P, ...): kBlock/LPR
// whole rows each (rows longer than the split length are skipped there).
template <typename VT, typename OT, typename IT, int LPR, int VEC, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void spmm_kernel(SpmmArgs a) {
  constexpr int GPB = kBlock / LPR;  // groups per block
  const int grp = threadIdx.x / LPR;
  const int gl = threadIdx.x % LPR;
  const int64_t j = (int64_t)blockIdx.y * (LPR * VEC) + (int64_t)gl * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  if ((int64_t)blockIdx.x < a.P) {
    __shared__ float red[GPB > 1 ? GPB - 1 : 1][LPR * VEC];
    const int64_t g = blockIdx.x;
    const int64_t i = a.item_pos[g];
    const int64_t ch = a.item_chunk[g];
    const int64_t r = load_row(a.row_idx, a.ri_i32, i);
    int64_t rs = 0, re = 0;
    if (r >= 0 && r < a.m) row_range(a.ro, r, a.nnz, rs, re);
    const int64_t c0 = rs + ch * kChunkLen;
    const int64_t c1 = (c0 + kChunkLen < re) ? c0 + kChunkLen : re;
    const int64_t len = c1 > c0 ? c1 - c0 : 0;
    const int64_t sub = cdiv(len, GPB);
    int64_t q0 = c0 + grp * sub;
    int64_t q1 = q0 + sub;
    q0 = q0 < c1 ? q0 : c1;
    q1 = q1 < c1 ? q1 : c1;
    accumulate<VT, IT, VEC, ALIGNED>(a, q0, q1, j, acc);
    if (grp > 0) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) red[grp - 1][gl * VEC + e] = acc[e];
    }
    __syncthreads();
    if (grp == 0) {
      for (int q = 0; q < GPB - 1; ++q) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += red[q][gl * VEC + e];
      }
      const int64_t nch = cdiv(re - rs, kChunkLen);
      if (nch <= 1) {
        if (r >= 0 && r < a.m) write_out<OT, VEC, ALIGNED>((OT*)a.C + r * a.ldc, j, a.N, acc);
      } else {
        write_out<float, VEC, ALIGNED>(a.partial + g * a.N, j, a.N, acc);
      }
    }
    return;
  }
  const int64_t i = ((int64_t)blockIdx.x - a.P) * GPB + grp;
  if (i >= a.m) return;
  const int64_t r = load_row(a.row_idx, a.ri_i32, i);
  if (r < 0 || r >= a.m) return;
  int64_t p0, p1;
  row_range(a.ro, r, a.nnz, p0, p1);
  if (a.P > 0 && p1 - p0 > a.T) return;  // handled by the chunk blocks
  accumulate<VT, IT, VEC, ALIGNED>(a, p0, p1, j, acc);
  write_out<OT, VEC, ALIGNED>((OT*)a.C + r * a.ldc, j, a.N, acc);
}

// N == 1: LPR lanes share a row, striding over its entries.
template <typename VT, typename OT, typename IT, int LPR>
__global__ __launch_bounds__(kBlock) void spmv_kernel(SpmmArgs a) {
  constexpr int GPB = kBlock / LPR;
  const IT* col = (const IT*)a.col;
  const VT* val = (const VT*)a.val;
  const VT* x = (const VT*)a.B;
  const int64_t k = a.k;
  const int64_t ldx = a.ldb;
  const int grp = threadIdx.x / LPR;
  const int gl = threadIdx.x % LPR;

  if ((int64_t)blockIdx.x < a.P) {
    __shared__ float red[kBlock / kWave];
    const int64_t g = blockIdx.x;
    const int64_t i = a.item_pos[g];
    const int64_t ch = a.item_chunk[g];
    const int64_t r = load_row(a.row_idx, a.ri_i32, i);
    int64_t rs = 0, re = 0;
    if (r >= 0 && r < a.m) row_range(a.ro, r, a.nnz, rs, re);
    const int64_t c0 = rs + ch * kChunkLen;
    const int64_t c1 = (c0 + kChunkLen < re) ? c0 + kChunkLen : re;
    float s = 0.f;
    for (int64_t p = c0 + threadIdx.x; p < c1; p += kBlock) {
      int c = (int)col[p];
      if ((unsigned)c < (unsigned)k) s = __builtin_fmaf(to_f32(val[p]), to_f32(x[c * ldx]), s);
    }
    s = group_sum<kWave>(s);
    if (lane_id() == 0) red[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = red[0];
      for (int q = 1; q < kBlock / kWave; ++q) t += red[q];
      const int64_t nch = cdiv(re - rs, kChunkLen);
      if (nch <= 1) {
        if (r >= 0 && r < a.m) ((OT*)a.C)[r * a.ldc] = from_f32<OT>(t);
      } else {
        a.partial[g] = t;
      }
    }
    return;
  }
  const int64_t i = ((int64_t)blockIdx.x - a.P) * GPB + grp;
  int64_t r = -1, p0 = 0, p1 = 0;
  if (i < a.m) {
    r = load_row(a.row_idx, a.ri_i32, i);
    if (r >= 0 && r < a.m) row_range(a.ro, r, a.nnz, p0, p1);
    else r = -1;
    if (a.P > 0 && p1 - p0 > a.T) r = -1;
  }
  if (r < 0) p1 = p0;
  float s = 0.f;
  constexpr int U = 4;
  int64_t p = p0 + gl;
  for (; p + (U - 1) * LPR < p1; p += U * LPR) {
    int c[U];
    float v[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      c[u] = (int)col[p + u * LPR];
      v[u] = to_f32(val[p + u * LPR]);
      if ((unsigned)c[u] >= (unsigned)k) {
        c[u] = 0;
        v[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) xv[u] = to_f32(x[(int64_t)c[u] * ldx]);
#pragma unroll
    for (int u = 0; u < U; ++u) s = __builtin_fmaf(v[u], xv[u], s);
  }
  for (; p < p1; p += LPR) {
    int c = (int)col[p];
    if ((unsigned)c < (unsigned)k) s = __builtin_fmaf(to_f32(val[p]), to_f32(x[c * ldx]), s);
  }
  s = group_sum<LPR>(s);
  if (gl == 0 && r >= 0) ((OT*)a.C)[r * a.ldc] = from_f32<OT>(s);
}

// Sum the partial rows of each multi-chunk row in chunk order.
template <typename OT>
__global__ __launch_bounds__(kBlock) void spmm_fixup_kernel(SpmmArgs a) {
  const int64_t s = blockIdx.x;
  const int64_t j = (int64_t)blockIdx.y * kBlock + threadIdx.x;
  if (j >= a.N) return;
  const int64_t i = a.split_pos[s];
  const int64_t r = load_row(a.row_idx, a.ri_i32, i);
  if (r < 0 || r >= a.m) return;
  const int64_t g0 = a.split_start[s], g1 = a.split_end[s];
  float t = 0.f;
  for (int64_t g = g0; g < g1; ++g) t += a.partial[g * a.N + j];
  ((OT*)a.C)[r * a.ldc + j] = from_f32<OT>(t);
}

// ------------------------------------------------------------ dispatch ---

template <typename VT, typename OT, typename IT, int LPR>
hipError_t launch_rows(const SpmmArgs& a, bool aligned, hipStream_t s) {
  constexpr int VEC = Vec16<VT>::n;
  constexpr int GPB = kBlock / LPR;
  const int64_t bx = a.P + cdiv(a.m, GPB);
  if (bx == 0) return hipSuccess;
  if (aligned) {
    dim3 grid((unsigned)bx, (unsigned)cdiv(a.N, LPR * VEC));
    hipLaunchKernelGGL((spmm_kernel<VT, OT, IT, LPR, VEC, true>), grid, dim3(kBlock), 0, s, a);
  } else {
    // scalar path: 64 lanes per row, one column each
    constexpr int G = kBlock / 64;
    dim3 grid((unsigned)(a.P + cdiv(a.m, G)), (unsigned)cdiv(a.N, 64));
    hipLaunchKernelGGL((spmm_kernel<VT, OT, IT, 64, 1, false>), grid, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

template <typename VT, typename OT, typename IT>
hipError_t launch_typed(const SpmmArgs& a, hipStream_t s) {
  constexpr int VEC = Vec16<VT>::n;
  hipError_t e;
  if (a.N == 1) {
    // lanes per row from the mean row length
    const int64_t mean = a.m > 0 ? a.nnz / a.m : 0;
    int lpr = 2;
    while (lpr < 64 && lpr * 4 < mean) lpr *= 2;
    const int gpb = kBlock / lpr;
    const dim3 grid((unsigned)(a.P + cdiv(a.m, gpb)));
    if (grid.x == 0) return hipSuccess;
    switch (lpr) {
      case 2: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 2>), grid, dim3(kBlock), 0, s, a); break;
      case 4: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 4>), grid, dim3(kBlock), 0, s, a); break;
      case 8: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 8>), grid, dim3(kBlock), 0, s, a); break;
      case 16: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 16>), grid, dim3(kBlock), 0, s, a); break;
      case 32: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 32>), grid, dim3(kBlock), 0, s, a); break;
      default: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 64>), grid, dim3(kBlock), 0, s, a); break;
    }
    e = hipGetLastError();
  } else {
    const bool aligned = (a.N % VEC == 0) && (a.ldb % VEC == 0) && (a.ldc % VEC == 0) &&
                         ((uintptr_t)a.B % 16 == 0) && ((uintptr_t)a.C % 16 == 0) &&
                         ((uintptr_t)a.partial % 16 == 0);
    const int64_t nv = cdiv(a.N, VEC);
    if (nv <= 4) e = launch_rows<VT, OT, IT, 4>(a, aligned, s);
    else if (nv <= 8) e = launch_rows<VT, OT, IT, 8>(a, aligned, s);
    else if (nv <= 16) e = launch_rows<VT, OT, IT, 16>(a, aligned, s);
    else if (nv <= 32) e = launch_rows<VT, OT, IT, 32>(a, aligned, s);
    else e = launch_rows<VT, OT, IT, 64>(a, aligned, s);
  }
  if (e != hipSuccess) return e;
  if (a.S > 0) {
    dim3 grid((unsigned)a.S, (unsigned)cdiv(a.N, kBlock));
    hipLaunchKernelGGL(spmm_fixup_kernel<OT>, grid, dim3(kBlock), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

template <typename VT>
hipError_t launch_vt(const SpmmArgs& a, hipStream_t s) {
  if (a.out_dtype == kF32) {
    return a.col_i32 ? launch_typed<VT, float, int32_t>(a, s)
                     : launch_typed<VT, float, int16_t>(a, s);
  }
  if constexpr (sizeof(VT) == 2) {
    return a.col_i32 ? launch_typed<VT, VT, int32_t>(a, s) : launch_typed<VT, VT, int16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------- schedule ---

__global__ __launch_bounds__(256) void sched_count_kernel(const int32_t* ro, const void* ri,
                                                          int ri_i32, int64_t m, int64_t nnz,
                                                          int32_t T, uint32_t* nch,
                                                          uint32_t* multi, int32_t* maxlen) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const int64_t r = load_row(ri, ri_i32, i);
  int64_t p0 = 0, p1 = 0;
  if (r >= 0 && r < m) row_range(ro, r, nnz, p0, p1);
  const int64_t len = p1 - p0;
  const uint32_t c = len > T ? (uint32_t)cdiv(len, kChunkLen) : 0u;
  nch[i] = c;
  multi[i] = c > 1 ? 1u : 0u;
  atomicMax(maxlen, (int32_t)len);
}

__global__ __launch_bounds__(256) void sched_fill_kernel(const uint32_t* nch, const uint32_t* off,
                                                         const uint32_t* multi_rank, int64_t m,
                                                         int32_t* item_pos, int32_t* item_chunk,
                                                         int32_t* split_pos, int32_t* split_start) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const uint32_t c = nch[i];
  const uint32_t o = off[i];
  for (uint32_t q = 0; q < c; ++q) {
    item_pos[o + q] = (int32_t)i;
    item_chunk[o + q] = (int32_t)q;
  }
  if (c > 1) {
    const uint32_t s = multi_rank[i];
    split_pos[s] = (int32_t)i;
    split_start[s] = (int32_t)o;
  }
}

// split_end[s] = one past the last item of multi-chunk row s
__global__ __launch_bounds__(256) void sched_ends_kernel(const uint32_t* nch, const uint32_t* off,
                                                         const int32_t* split_pos, int64_t S,
                                                         int32_t* split_end) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const int64_t i = split_pos[s];
  split_end[s] = (int32_t)(off[i] + nch[i]);
}

}  // namespace

hipError_t launch_spmm(const SpmmArgs& a, hipStream_t s) {
  switch (a.dtype) {
    case kF32: return launch_vt<float>(a, s);
    case kF16: return launch_vt<_Float16>(a, s);
    case kBF16: return launch_vt<bf16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t build_spmm_schedule(const int32_t* ro, const void* row_idx, int ri_i32, int64_t m,
                               int64_t nnz, int32_t T, SpmmSchedule* out, hipStream_t s) {
  *out = SpmmSchedule{};
  out->T = T;
  if (m <= 0) return hipSuccess;
  const size_t nb = align256((size_t)m * 4);
  const size_t sw = scan_workspace_bytes(m);
  char* tmp = nullptr;
  hipError_t e = hipMalloc(&tmp, 4 * nb + sw + 256);
  if (e != hipSuccess) return e;
  uint32_t* nch = (uint32_t*)tmp;
  uint32_t* off = (uint32_t*)(tmp + nb);
  uint32_t* multi = (uint32_t*)(tmp + 2 * nb);
  uint32_t* mrank = (uint32_t*)(tmp + 3 * nb);
  int32_t* dev_misc = (int32_t*)(tmp + 4 * nb);  // [0] maxlen, [1] P, [2] S
  void* sws = tmp + 4 * nb + 256;
  int32_t host_misc[3] = {0, 0, 0};
  const unsigned g = (unsigned)cdiv(m, 256);
  do {
    if ((e = hipMemcpyAsync(dev_misc, host_misc, 12, hipMemcpyHostToDevice, s)) != hipSuccess) break;
    hipLaunchKernelGGL(sched_count_kernel, dim3(g), dim3(256), 0, s, ro, row_idx, ri_i32, m, nnz,
                       T, nch, multi, dev_misc);
    if ((e = hipGetLastError()) != hipSuccess) break;
    if ((e = exclusive_scan_u32(nch, off, m, (uint32_t*)dev_misc + 1, sws, s)) != hipSuccess) break;
    if ((e = exclusive_scan_u32(multi, mrank, m, (uint32_t*)dev_misc + 2, sws, s)) != hipSuccess)
      break;
    if ((e = hipMemcpyAsync(host_misc, dev_misc, 12, hipMemcpyDeviceToHost, s)) != hipSuccess) break;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
    out->max_row = host_misc[0];
    out->P = host_misc[1];
    out->S = host_misc[2];
    if (out->P > 0) {
      const size_t pb = align256((size_t)out->P * 4), sb = align256((size_t)(out->S + 1) * 4);
      char* mem = nullptr;
      if ((e = hipMalloc(&mem, 2 * pb + 3 * sb)) != hipSuccess) break;
      out->mem = mem;
      out->item_pos = (int32_t*)mem;
      out->item_chunk = (int32_t*)(mem + pb);
      out->split_pos = (int32_t*)(mem + 2 * pb);
      out->split_start = (int32_t*)(mem + 2 * pb + sb);
      out->split_end = (int32_t*)(mem + 2 * pb + 2 * sb);
      hipLaunchKernelGGL(sched_fill_kernel, dim3(g), dim3(256), 0, s, nch, off, mrank, m,
                         out->item_pos, out->item_chunk, out->split_pos, out->split_start);
      if ((e = hipGetLastError()) != hipSuccess) break;
      if (out->S > 0) {
        hipLaunchKernelGGL(sched_ends_kernel, dim3((unsigned)cdiv(out->S, 256)), dim3(256), 0, s,
                           nch, off, out->split_pos, out->S, out->split_end);
        if ((e = hipGetLastError()) != hipSuccess) break;
      }
    }
    e = hipStreamSynchronize(s);
  } while (0);
  hipFree(tmp);
  if (e != hipSuccess) free_spmm_schedule(out);
  return e;
}

void free_spmm_schedule(SpmmSchedule* sch) {
  if (sch->mem) hipFree(sch->mem);
  *sch = SpmmSchedule{};
}

}  // namespace spops

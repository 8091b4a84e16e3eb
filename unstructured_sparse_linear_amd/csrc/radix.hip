// radix.hip -- prefix sums and stable LSD radix sorting on gfx950, and the
// two operations built from them:
//   * csr_transpose (spops README, section "CSR Transpose"): a stable sort of
//     the stored entries by column; the output row offsets are the column
//     boundaries of the sorted keys;
//   * the row_idx order (section "Usage"): rows sorted by entry count, most
//     first, ties by ascending row -- a stable sort on (cols - count).
//
// Sorting is least-significant-digit radix with 8-bit digits, in three
// kernels per pass: per-tile digit counts, one exclusive scan over the
// digit-major count table, and a stable scatter.  Inside a tile the rank of
// each key among equal digits is found with wave ballots (64-lane match on
// the digit bits) plus per-wave digit counts in LDS, so no atomics decide
// any position and the output is deterministic.  No kernel waits on another
// block, so no launch order assumptions are made.
#include "common.h"
#include "kernels.h"

namespace spops {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;
constexpr int kTile = kThreads * kItems;  // keys per tile
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;

// ================================================================= scan ==

// Exclusive scan inside each block of kTile elements; block totals to `sums`.
__global__ __launch_bounds__(kThreads) void scan_local_kernel(const uint32_t* in, uint32_t* out,
                                                              int64_t n, uint32_t* sums,
                                                              uint32_t* total) {
  __shared__ uint32_t wave_tot[kThreads / kWave];
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)t * kItems;
  uint32_t v[kItems];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    v[i] = (base + i < n) ? in[base + i] : 0u;
    s += v[i];
  }
  // inclusive scan of per-thread sums inside the wave
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane_id() >= o) x += y;
  }
  const int w = t / kWave;
  if (lane_id() == kWave - 1) wave_tot[w] = x;
  __syncthreads();
  uint32_t wave_off = 0, blk = 0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) {
    uint32_t wt = wave_tot[i];
    if (i < w) wave_off += wt;
    blk += wt;
  }
  uint32_t run = wave_off + x - s;  // exclusive prefix of this thread
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
  if (t == 0) {
    if (sums) sums[blockIdx.x] = blk;
    if (total && gridDim.x == 1) *total = blk;
  }
}

// Whole exclusive scan in one workgroup of 1024 threads for n up to 16384:
// each thread scans a contiguous chunk of at most 16 values.
constexpr int kSingleThreads = 1024;
constexpr int64_t kSingleMax = 16384;

__global__ __launch_bounds__(kSingleThreads) void scan_single_kernel(const uint32_t* in,
                                                                     uint32_t* out, int64_t n,
                                                                     uint32_t* total) {
  __shared__ uint32_t wave_tot[kSingleThreads / kWave];
  const int t = threadIdx.x;
  constexpr int kPer = kSingleMax / kSingleThreads;
  const int64_t b0 = (int64_t)t * kPer;
  uint32_t v[kPer];
  uint32_t s = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    v[q] = (b0 + q < n) ? in[b0 + q] : 0u;
    s += v[q];
  }
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane_id() >= o) x += y;
  }
  const int w = t / kWave;
  if (lane_id() == kWave - 1) wave_tot[w] = x;
  __syncthreads();
  uint32_t run = 0, blk = 0;
  for (int i = 0; i < kSingleThreads / kWave; ++i) {
    const uint32_t wt = wave_tot[i];
    if (i < w) run += wt;
    blk += wt;
  }
  run += x - s;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (b0 + q < n) out[b0 + q] = run;
    run += v[q];
  }
  if (t == 0 && total) *total = blk;
}

__global__ __launch_bounds__(kThreads) void scan_add_kernel(uint32_t* out, int64_t n,
                                                            const uint32_t* offs) {
  const uint32_t add = offs[blockIdx.x];
  const int64_t base = (int64_t)blockIdx.x * kTile + (int64_t)threadIdx.x * kItems;
#pragma unroll
  for (int i = 0; i < kItems; ++i)
    if (base + i < n) out[base + i] += add;
}

// ========================================================== radix sort ==

// Key sources: a typed index list clamped to [0, kmax]; row lengths turned
// into descending-order keys; a plain uint32 array.
template <typename I>
struct KeyFromIndex {
  const I* p;
  int32_t kmax;
  __device__ uint32_t operator()(int64_t i) const {
    int v = (int)p[i];
    v = v < 0 ? 0 : (v > kmax ? kmax : v);
    return (uint32_t)v;
  }
};

struct KeyFromRowLength {
  const int32_t* ro;
  int32_t cols;
  __device__ uint32_t operator()(int64_t i) const {
    int64_t c = (int64_t)ro[i + 1] - (int64_t)ro[i];
    c = c < 0 ? 0 : (c > cols ? cols : c);
    return (uint32_t)(cols - c);
  }
};

struct KeyFromU32 {
  const uint32_t* p;
  __device__ uint32_t operator()(int64_t i) const { return p[i]; }
};

struct ValIota {
  __device__ uint32_t operator()(int64_t i) const { return (uint32_t)i; }
};

struct ValFromU32 {
  const uint32_t* p;
  __device__ uint32_t operator()(int64_t i) const { return p[i]; }
};

// Per-tile digit histogram, stored digit-major: counts[d * ntiles + tile].
// Thread t takes kItems consecutive keys.
template <class KS>
__global__ __launch_bounds__(kThreads) void radix_count_kernel(KS ks, int64_t n, int shift,
                                                               uint32_t mask, uint32_t* counts,
                                                               int64_t ntiles) {
  __shared__ uint32_t hist[kRadix];
  const int t = threadIdx.x;
  hist[t] = 0;
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kTile + (int64_t)t * kItems;
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int64_t i = i0 + q;
    if (i < n) atomicAdd(&hist[(ks(i) >> shift) & mask], 1u);
  }
  __syncthreads();
  counts[(int64_t)t * ntiles + blockIdx.x] = hist[t];
}

// Stable scatter.  Keys of a tile are taken in rounds of kThreads (round-major,
// then thread order == index order).  In a round each wave finds the lanes
// holding the same digit with ballots; the lowest such lane publishes the
// count; digit offsets per wave then follow from the running per-digit base.
template <class KS, class VS>
__global__ __launch_bounds__(kThreads) void radix_scatter_kernel(
    KS ks, VS vs, int64_t n, int shift, int nbits, const uint32_t* offs, int64_t ntiles,
    uint32_t* kout, uint32_t* vout) {
  __shared__ uint32_t base_d[kRadix];
  __shared__ uint32_t wcnt[kThreads / kWave][kRadix];
  const int t = threadIdx.x;
  const int w = t / kWave;
  const uint32_t mask = (1u << nbits) - 1u;
  base_d[t] = offs[(int64_t)t * ntiles + blockIdx.x];
  const int64_t tbase = (int64_t)blockIdx.x * kTile;
  const uint64_t lt = lanemask_lt();
  for (int r = 0; r < kItems; ++r) {
#pragma unroll
    for (int ww = 0; ww < kThreads / kWave; ++ww) wcnt[ww][t] = 0;
    __syncthreads();
    const int64_t i = tbase + r * kThreads + t;
    const bool valid = i < n;
    const uint32_t key = valid ? ks(i) : 0u;
    const uint32_t d = (key >> shift) & mask;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & lt);
    if (valid && rank == 0) wcnt[w][d] = (uint32_t)__popcll(peers);
    __syncthreads();
    {
      // thread t owns digit t: turn per-wave counts into per-wave offsets
      uint32_t run = base_d[t];
#pragma unroll
      for (int ww = 0; ww < kThreads / kWave; ++ww) {
        uint32_t c = wcnt[ww][t];
        wcnt[ww][t] = run;
        run += c;
      }
      base_d[t] = run;
    }
    __syncthreads();
    if (valid) {
      const uint32_t dst = wcnt[w][d] + rank;
      kout[dst] = key;
      vout[dst] = vs(i);
    }
    __syncthreads();
  }
}

struct RadixWs {
  uint32_t* keys[2];
  uint32_t* vals[2];
  uint32_t* counts;
  void* scan_ws;
};

size_t radix_ws_bytes_for(int64_t n) {
  const int64_t ntiles = cdiv(n > 0 ? n : 1, kTile);
  return 4 * align256((size_t)n * 4) + align256((size_t)ntiles * kRadix * 4) +
         scan_workspace_bytes(ntiles * kRadix);
}

RadixWs carve_radix_ws(void* ws, int64_t n) {
  const int64_t ntiles = cdiv(n > 0 ? n : 1, kTile);
  char* p = (char*)ws;
  RadixWs r;
  for (int i = 0; i < 2; ++i) {
    r.keys[i] = (uint32_t*)p;
    p += align256((size_t)n * 4);
    r.vals[i] = (uint32_t*)p;
    p += align256((size_t)n * 4);
  }
  r.counts = (uint32_t*)p;
  p += align256((size_t)ntiles * kRadix * 4);
  r.scan_ws = p;
  return r;
}

int bit_length(uint64_t v) {
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

// Sorts n keys (all < 2^bits) stably; the first pass reads `ks0` and produces
// payload iota.  Returns the buffer index holding the result.
template <class KS0>
hipError_t radix_sort_iota(KS0 ks0, int64_t n, int bits, const RadixWs& R, int* result,
                           hipStream_t s) {
  const int64_t ntiles = cdiv(n, kTile);
  if (bits < 1) bits = 1;
  int cur = -1;  // -1: source functor; else buffer index holding current keys
  int dst = 0;
  for (int shift = 0; shift < bits; shift += kRadixBits) {
    const int nb = (bits - shift) < kRadixBits ? (bits - shift) : kRadixBits;
    const uint32_t mask = (1u << nb) - 1u;
    if (cur < 0) {
      hipLaunchKernelGGL(radix_count_kernel<KS0>, dim3(ntiles), dim3(kThreads), 0, s, ks0, n,
                         shift, mask, R.counts, ntiles);
    } else {
      hipLaunchKernelGGL(radix_count_kernel<KeyFromU32>, dim3(ntiles), dim3(kThreads), 0, s,
                         KeyFromU32{R.keys[cur]}, n, shift, mask, R.counts, ntiles);
    }
    hipError_t e = exclusive_scan_u32(R.counts, R.counts, ntiles * kRadix, nullptr, R.scan_ws, s);
    if (e != hipSuccess) return e;
    if (cur < 0) {
      hipLaunchKernelGGL((radix_scatter_kernel<KS0, ValIota>), dim3(ntiles), dim3(kThreads), 0,
                         s, ks0, ValIota{}, n, shift, nb, R.counts, ntiles, R.keys[dst],
                         R.vals[dst]);
    } else {
      hipLaunchKernelGGL((radix_scatter_kernel<KeyFromU32, ValFromU32>), dim3(ntiles),
                         dim3(kThreads), 0, s, KeyFromU32{R.keys[cur]}, ValFromU32{R.vals[cur]},
                         n, shift, nb, R.counts, ntiles, R.keys[dst], R.vals[dst]);
    }
    cur = dst;
    dst ^= 1;
  }
  *result = cur;
  return hipGetLastError();
}

// ============================================================= transpose ==

// rows_of[p] = row owning position p; 16 lanes per row.
__global__ __launch_bounds__(256) void expand_rows_kernel(const int32_t* ro, int64_t m,
                                                          int64_t nnz, uint32_t* rows_of) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  if (r >= m) return;
  int64_t p0 = ro[r], p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : p0;
  p1 = p1 > nnz ? nnz : p1;
  for (int64_t p = p0 + sub; p < p1; p += 16) rows_of[p] = (uint32_t)r;
}

// Output row offsets from the sorted column keys, and gather of row indices
// and values through the sorted payload (source positions).
template <typename OI, int VB>
__global__ __launch_bounds__(256) void transpose_finish_kernel(
    const uint32_t* keys, const uint32_t* src, const uint32_t* rows_of, int64_t nnz, int64_t n,
    const uint8_t* val, uint8_t* out_val, int32_t* out_ro, OI* out_col) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q > nnz) return;
  const int64_t kprev = q == 0 ? -1 : (int64_t)keys[q - 1];
  const int64_t kcur = q == nnz ? n : (int64_t)keys[q];
  for (int64_t c = kprev + 1; c <= kcur; ++c) out_ro[c] = (int32_t)q;
  if (q == nnz) return;
  const uint32_t p = src[q];
  out_col[q] = (OI)rows_of[p];
  if constexpr (VB == 4) {
    ((uint32_t*)out_val)[q] = ((const uint32_t*)val)[p];
  } else if constexpr (VB == 2) {
    ((uint16_t*)out_val)[q] = ((const uint16_t*)val)[p];
  }
}

template <typename OI>
hipError_t finish_transpose(const uint32_t* keys, const uint32_t* src, const uint32_t* rows_of,
                            int64_t nnz, int64_t n, const void* val, int vb, void* out_val,
                            int32_t* out_ro, void* out_col, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(nnz + 1, 256));
  if (vb == 4)
    hipLaunchKernelGGL((transpose_finish_kernel<OI, 4>), grid, dim3(256), 0, s, keys, src,
                       rows_of, nnz, n, (const uint8_t*)val, (uint8_t*)out_val, out_ro,
                       (OI*)out_col);
  else if (vb == 2)
    hipLaunchKernelGGL((transpose_finish_kernel<OI, 2>), grid, dim3(256), 0, s, keys, src,
                       rows_of, nnz, n, (const uint8_t*)val, (uint8_t*)out_val, out_ro,
                       (OI*)out_col);
  else
    hipLaunchKernelGGL((transpose_finish_kernel<OI, 0>), grid, dim3(256), 0, s, keys, src,
                       rows_of, nnz, n, (const uint8_t*)val, (uint8_t*)out_val, out_ro,
                       (OI*)out_col);
  return hipGetLastError();
}

// Row order of up to kBlockSortMax rows in one workgroup: LSD radix sort of
// 16-bit keys (cols - count) packed above 16-bit row ids, two 8-bit passes
// through LDS.  Ranks among equal digits come from wave ballots, rounds of
// 1024 rows are taken in index order, so the sort is stable.
constexpr int kBlockSortThreads = 1024;
constexpr int64_t kBlockSortMax = 16384;
// measured: one workgroup beats the multi-kernel sort only for small counts
constexpr int64_t kBlockSortUse = 4096;

template <typename OI>
__global__ __launch_bounds__(kBlockSortThreads) void sort_rows_block_kernel(const int32_t* ro,
                                                                           int64_t m,
                                                                           int32_t cols,
                                                                           OI* out) {
  constexpr int NW = kBlockSortThreads / kWave;
  __shared__ uint32_t buf[2][kBlockSortMax];
  __shared__ uint32_t cnt[NW][kRadix];
  __shared__ uint32_t base_d[kRadix];
  const int t = threadIdx.x, w = t / kWave;
  const uint64_t lt = lanemask_lt();
  for (int64_t i = t; i < m; i += kBlockSortThreads) {
    int64_t c = (int64_t)ro[i + 1] - (int64_t)ro[i];
    c = c < 0 ? 0 : (c > cols ? cols : c);
    buf[0][i] = ((uint32_t)(cols - c) << 16) | (uint32_t)i;
  }
  int cur = 0;
  for (int shift = 16; shift < 32; shift += 8) {
    if (t < kRadix) base_d[t] = 0;
    __syncthreads();
    for (int64_t i = t; i < m; i += kBlockSortThreads)
      atomicAdd(&base_d[(buf[cur][i] >> shift) & 0xffu], 1u);
    __syncthreads();
    if (t == 0) {
      uint32_t run = 0;
      for (int d = 0; d < kRadix; ++d) {
        const uint32_t c = base_d[d];
        base_d[d] = run;
        run += c;
      }
    }
    __syncthreads();
    for (int64_t r0 = 0; r0 < m; r0 += kBlockSortThreads) {
      for (int q = t; q < NW * kRadix; q += kBlockSortThreads) (&cnt[0][0])[q] = 0;
      __syncthreads();
      const int64_t i = r0 + t;
      const bool valid = i < m;
      const uint32_t item = valid ? buf[cur][i] : 0u;
      const uint32_t d = (item >> shift) & 0xffu;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      const uint32_t rank = (uint32_t)__popcll(peers & lt);
      if (valid && rank == 0) cnt[w][d] = (uint32_t)__popcll(peers);
      __syncthreads();
      if (t < kRadix) {
        uint32_t run = base_d[t];
        for (int ww = 0; ww < NW; ++ww) {
          const uint32_t c = cnt[ww][t];
          cnt[ww][t] = run;
          run += c;
        }
        base_d[t] = run;
      }
      __syncthreads();
      if (valid) buf[cur ^ 1][cnt[w][d] + rank] = item;
      __syncthreads();
    }
    cur ^= 1;
  }
  for (int64_t i = t; i < m; i += kBlockSortThreads) out[i] = (OI)(buf[cur][i] & 0xffffu);
}

// row_idx output from the sorted payload
template <typename OI>
__global__ __launch_bounds__(256) void store_perm_kernel(const uint32_t* src, int64_t m, OI* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < m) out[i] = (OI)src[i];
}

}  // namespace

// ================================================================ public ==

size_t scan_workspace_bytes(int64_t n) {
  size_t b = 0;
  while (n > kTile) {
    n = cdiv(n, kTile);
    b += align256((size_t)n * 4);
  }
  return b + 256;
}

hipError_t exclusive_scan_u32(const uint32_t* in, uint32_t* out, int64_t n, uint32_t* total,
                              void* ws, hipStream_t s) {
  if (n <= 0) {
    if (total) return hipMemsetAsync(total, 0, 4, s);
    return hipSuccess;
  }
  const int64_t nb = cdiv(n, kTile);
  if (nb == 1) {
    hipLaunchKernelGGL(scan_local_kernel, dim3(1), dim3(kThreads), 0, s, in, out, n, nullptr,
                       total);
    return hipGetLastError();
  }
  if (n <= kSingleMax) {
    hipLaunchKernelGGL(scan_single_kernel, dim3(1), dim3(kSingleThreads), 0, s, in, out, n,
                       total);
    return hipGetLastError();
  }
  uint32_t* sums = (uint32_t*)ws;
  void* rest = (char*)ws + align256((size_t)nb * 4);
  hipLaunchKernelGGL(scan_local_kernel, dim3((unsigned)nb), dim3(kThreads), 0, s, in, out, n,
                     sums, nullptr);
  hipError_t e = exclusive_scan_u32(sums, sums, nb, total, rest, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)nb), dim3(kThreads), 0, s, out, n, sums);
  return hipGetLastError();
}

size_t radix_pairs_workspace_bytes(int64_t n) { return radix_ws_bytes_for(n); }

hipError_t radix_sort_u32_iota(const uint32_t* keys, int64_t n, int bits, uint32_t* sorted_keys,
                               uint32_t* sorted_vals, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  RadixWs R = carve_radix_ws(ws, n);
  int res = 0;
  hipError_t e = radix_sort_iota(KeyFromU32{keys}, n, bits, R, &res, s);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(sorted_keys, R.keys[res], (size_t)n * 4, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  return hipMemcpyAsync(sorted_vals, R.vals[res], (size_t)n * 4, hipMemcpyDeviceToDevice, s);
}

size_t transpose_workspace_bytes(int64_t rows, int64_t cols, int64_t nnz) {
  (void)rows;
  (void)cols;
  return radix_ws_bytes_for(nnz) + align256((size_t)nnz * 4);
}

hipError_t launch_csr_transpose(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                                const void* col, int col_i32, const void* val, int val_bytes,
                                void* out_val, int32_t* out_ro, void* out_col, int out_col_i32,
                                void* ws, hipStream_t s) {
  RadixWs R = carve_radix_ws(ws, nnz);
  uint32_t* rows_of = (uint32_t*)((char*)ws + radix_ws_bytes_for(nnz));
  const uint32_t* skeys = nullptr;
  const uint32_t* svals = nullptr;
  if (nnz > 0) {
    hipLaunchKernelGGL(expand_rows_kernel, dim3((unsigned)cdiv(rows * 16, 256)), dim3(256),
                       0, s, ro, rows, nnz, rows_of);
    const int bits = bit_length((uint64_t)(cols - 1));
    int res = 0;
    hipError_t e;
    if (col_i32)
      e = radix_sort_iota(KeyFromIndex<int32_t>{(const int32_t*)col, (int32_t)(cols - 1)}, nnz,
                          bits, R, &res, s);
    else
      e = radix_sort_iota(KeyFromIndex<int16_t>{(const int16_t*)col, (int32_t)(cols - 1)}, nnz,
                          bits, R, &res, s);
    if (e != hipSuccess) return e;
    skeys = R.keys[res];
    svals = R.vals[res];
  }
  const int vb = val ? val_bytes : 0;
  if (out_col_i32)
    return finish_transpose<int32_t>(skeys, svals, rows_of, nnz, cols, val, vb, out_val, out_ro,
                                     out_col, s);
  return finish_transpose<int16_t>(skeys, svals, rows_of, nnz, cols, val, vb, out_val, out_ro,
                                   out_col, s);
}

size_t sort_rows_workspace_bytes(int64_t rows, int64_t cols) {
  (void)cols;
  return radix_ws_bytes_for(rows);
}

hipError_t launch_sort_rows(const int32_t* ro, int64_t rows, int64_t cols, void* row_idx,
                            int row_idx_i32, void* ws, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows <= kBlockSortUse && cols <= 65535) {
    if (row_idx_i32)
      hipLaunchKernelGGL(sort_rows_block_kernel<int32_t>, dim3(1), dim3(kBlockSortThreads), 0, s,
                         ro, rows, (int32_t)cols, (int32_t*)row_idx);
    else
      hipLaunchKernelGGL(sort_rows_block_kernel<int16_t>, dim3(1), dim3(kBlockSortThreads), 0, s,
                         ro, rows, (int32_t)cols, (int16_t*)row_idx);
    return hipGetLastError();
  }
  RadixWs R = carve_radix_ws(ws, rows);
  int res = 0;
  const int bits = bit_length((uint64_t)cols);
  hipError_t e = radix_sort_iota(KeyFromRowLength{ro, (int32_t)cols}, rows, bits, R, &res, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)cdiv(rows, 256));
  if (row_idx_i32)
    hipLaunchKernelGGL(store_perm_kernel<int32_t>, grid, dim3(256), 0, s, R.vals[res], rows,
                       (int32_t*)row_idx);
  else
    hipLaunchKernelGGL(store_perm_kernel<int16_t>, grid, dim3(256), 0, s, R.vals[res], rows,
                       (int16_t*)row_idx);
  return hipGetLastError();
}

}  // namespace spops

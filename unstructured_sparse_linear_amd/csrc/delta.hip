// delta.hip -- rows with 2-bit delta-coded columns (encode, SpMV) on gfx950.
//
// The UST news page (section "Formatos menos comuns") converts a matrix to a
// 2-bit delta-compressed format: rows stay a dense level, column coordinates
// inside a row are stored as differences; its MACKO experiment (section
// "Performance") multiplies such matrices with a vector at low sparsity,
// padding only up to the end of each row.  Layout (the page shows none):
// entry e of the encoded stream has a 2-bit code d, its column is the
// previous entry's column + d + 1 (from -1 at a row start); a gap above 4 is
// bridged by zero-valued padding entries (code 3) every 4 columns; nothing
// is padded after a row's last entry.  enc_offsets[m+1] delimit the rows;
// codes are packed 16 per uint32 (entry e in bits 2(e mod 16) of word e/16);
// the value array is padded with zeros to a multiple of 16 entries, so a
// word's 16 values can always be loaded whole.
//
// Index storage drops from 16 or 32 bits to 2 bits per entry (plus padding,
// rare at the densities the format is for), so an SpMV that streams the
// matrix from HBM moves about half the bytes of CSR for f16 values.
//
// SpMV: one wave per row.  Lane l takes one code word (16 entries) and its
// 16 values (two or four 16-byte loads); it decodes its 16 column steps, the
// wave turns the per-lane step totals into each lane's starting column with
// a DPP prefix sum, and the lane gathers x at its columns and accumulates in
// fp32.  A row spans as many 1024-entry wave rounds as it needs; the column
// carries over between rounds, and the next round's word and values are
// loaded while a round is computed.  When x fits (48 KiB) each workgroup
// first copies it into LDS, so the gathers are LDS reads; workgroups then
// loop over rows.  Entries whose decoded column is outside [0, n) (codes
// that do not belong to a valid matrix) are skipped.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

__device__ __forceinline__ uint32_t wave_last(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Encoded length of every row (stored entries + padding); flags rows whose
// columns are not strictly ascending or out of [0, n).
template <typename IT>
__global__ __launch_bounds__(kBlock) void delta_count_kernel(int64_t m, int64_t n, int64_t nnz,
                                                             const int32_t* ro, const IT* col,
                                                             uint32_t* len, uint32_t* bad) {
  const int64_t r = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  const int l = lane_id();
  if (blockIdx.x == 0 && threadIdx.x == 0) len[m] = 0;
  if (r >= m) return;
  int64_t p0 = ro[r], p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > nnz ? nnz : p1);
  uint32_t cnt = 0, err = 0;
  for (int64_t p = p0 + l; p < p1; p += kWave) {
    const int64_t c = (int64_t)col[p];
    const int64_t cp = p > p0 ? (int64_t)col[p - 1] : -1;
    const int64_t gap = c - cp;
    if (gap < 1 || c >= n) {
      err = 1;
      cnt += 1;
    } else {
      cnt += (uint32_t)((gap - 1) >> 2) + 1;
    }
  }
  for (int o = kWave / 2; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if (l == 0) len[r] = cnt;
  if (err) atomicOr(bad, 1u);
}

__global__ __launch_bounds__(kBlock) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename VT>
__global__ __launch_bounds__(kBlock) void fill_values_kernel(VT* p, int64_t from, int64_t to) {
  const int64_t i = from + (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < to) p[i] = VT{};
}

// Writes the encoded stream: one wave per row, 64 stored entries per round;
// each lane's entry and its padding take (gap - 1) / 4 + 1 slots, placed by
// a wave prefix sum.  Codes are OR-ed into zeroed words (a word can hold
// codes of two rows, which different waves write).
template <typename VT, typename IT>
__global__ __launch_bounds__(kBlock) void delta_encode_kernel(int64_t m, int64_t nnz,
                                                              const int32_t* ro, const IT* col,
                                                              const VT* val, const int32_t* eo,
                                                              int64_t total, uint32_t* codes,
                                                              VT* out) {
  const int64_t r = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  const int l = lane_id();
  if (r >= m) return;
  int64_t p0 = ro[r], p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > nnz ? nnz : p1);
  int64_t slot0 = eo[r];
  for (int64_t b = p0; b < p1; b += kWave) {
    const int64_t p = b + l;
    uint32_t cnt = 0, pad = 0, code = 0;
    if (p < p1) {
      const int64_t c = (int64_t)col[p];
      const int64_t cp = p > p0 ? (int64_t)col[p - 1] : -1;
      const int64_t gap = c - cp;
      if (gap >= 1) {
        pad = (uint32_t)((gap - 1) >> 2);
        code = (uint32_t)(gap - 1 - 4 * (int64_t)pad);
      }
      cnt = pad + 1;
    }
    const uint32_t incl = wave_inclusive_sum(cnt);
    const int64_t start = slot0 + (incl - cnt);
    if (p < p1) {
      for (uint32_t j = 0; j < pad; ++j) {
        const int64_t s = start + j;
        if (s < total) {
          out[s] = VT{};
          atomicOr(codes + (s >> 4), 3u << (2 * (s & 15)));
        }
      }
      const int64_t s = start + pad;
      if (s < total) {
        out[s] = val[p];
        if (code) atomicOr(codes + (s >> 4), code << (2 * (s & 15)));
      }
    }
    slot0 += wave_last(incl);
  }
}

// 16 values of one code word.
template <typename VT>
__device__ __forceinline__ void load16(const VT* p, float (&v)[16]) {
  if constexpr (sizeof(VT) == 4) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint4 w = q[h];
      v[4 * h + 0] = __uint_as_float(w.x);
      v[4 * h + 1] = __uint_as_float(w.y);
      v[4 * h + 2] = __uint_as_float(w.z);
      v[4 * h + 3] = __uint_as_float(w.w);
    }
  } else {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 w = q[h];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * h + 2 * k] = lo_f32(ws[k], (VT*)nullptr);
        v[8 * h + 2 * k + 1] = hi_f32(ws[k], (VT*)nullptr);
      }
    }
  }
}

// x in LDS when it fits this many bytes (then every gather is an LDS read
// and the next round's loads can be in flight while a round is computed)
constexpr int64_t kDeltaXLds = 48 * 1024;
// most workgroups; each copies x into its LDS once and loops over rows
constexpr int64_t kDeltaMaxBlocks = 1024;

template <typename VT, typename OT, bool XLDS>
__global__ __launch_bounds__(kBlock) void delta_spmv_kernel(int64_t m, int64_t n,
                                                            const int32_t* eo,
                                                            const uint32_t* codes, const VT* val,
                                                            int64_t total, const VT* x, OT* y) {
  extern __shared__ __align__(16) unsigned char xs_raw[];
  const VT* xr = x;
  if constexpr (XLDS) {
    VT* xs = (VT*)xs_raw;
    for (int64_t i = threadIdx.x; i < n; i += kBlock) xs[i] = x[i];
    __syncthreads();
    xr = xs;
  }
  const int l = lane_id();
  for (int64_t r = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave; r < m;
       r += (int64_t)gridDim.x * kWaves) {
    int64_t e0 = eo[r], e1 = eo[r + 1];
    e0 = e0 < 0 ? 0 : (e0 > total ? total : e0);
    e1 = e1 < e0 ? e0 : (e1 > total ? total : e1);
    float acc0 = 0.f, acc1 = 0.f;
    int64_t colc = -1;  // column before the first entry of this round
    const int64_t wfirst = e0 >> 4;
    // round 0's word and values; later rounds are loaded one round ahead
    // (the value array is padded to whole words; lanes past the row load
    // the row's first word)
    int64_t w = wfirst + l;
    uint32_t word = 0;
    float v[16];
    {
      const int64_t wl = w * 16 < e1 ? w : wfirst;
      if (e0 < e1) {
        word = codes[wl];
        load16(val + wl * 16, v);
      }
    }
    for (int64_t wb = wfirst; wb * 16 < e1; wb += kWave, w += kWave) {
      const int64_t eb = w * 16;  // first entry of this lane's word
      const bool any = eb < e1;
      uint32_t nword = 0;
      float nv[16];
      const int64_t wn = w + kWave;
      if ((wb + kWave) * 16 < e1) {
        const int64_t wl = wn * 16 < e1 ? wn : wfirst;
        nword = codes[wl];
        load16(val + wl * 16, nv);
      }
      // column steps of this lane's entries that belong to the row
      uint32_t step[16];
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t e = eb + j;
        step[j] = (any && e >= e0 && e < e1) ? ((word >> (2 * j)) & 3u) + 1u : 0u;
        tot += step[j];
      }
      const uint32_t incl = wave_inclusive_sum(tot);
      int64_t c = colc + (int64_t)(incl - tot);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        c += step[j];
        const bool ok = step[j] != 0 && c < n;
        const float xv = to_f32(xr[ok ? c : 0]);
        const float vv = ok ? v[j] : 0.f;  // entries of other rows
        if (j & 1)
          acc1 = __builtin_fmaf(vv, xv, acc1);
        else
          acc0 = __builtin_fmaf(vv, xv, acc0);
      }
      colc += (int64_t)wave_last(incl);
      word = nword;
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = nv[j];
    }
    float acc = group_sum<kWave>(acc0 + acc1);
    if (l == 0) y[r] = from_f32<OT>(acc);
  }
}

template <typename IT>
hipError_t count_it(int64_t m, int64_t n, int64_t nnz, const int32_t* ro, const void* col,
                    uint32_t* len, uint32_t* bad, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(m, kWaves));
  hipLaunchKernelGGL(delta_count_kernel<IT>, grid, dim3(kBlock), 0, s, m, n, nnz, ro,
                     (const IT*)col, len, bad);
  return hipGetLastError();
}

template <typename VT>
hipError_t encode_vt(int64_t m, int64_t nnz, const int32_t* ro, const void* col, int col_i32,
                     const void* val, const int32_t* eo, int64_t total, uint32_t* codes,
                     void* out, hipStream_t s) {
  const int64_t words = cdiv(total, 16);
  const int64_t padded = words * 16;
  if (words > 0) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)cdiv(words, kBlock)), dim3(kBlock), 0, s,
                       codes, words, 0u);
    if (padded > total)
      hipLaunchKernelGGL(fill_values_kernel<VT>, dim3(1), dim3(kBlock), 0, s, (VT*)out, total,
                         padded);
  }
  const dim3 grid((unsigned)cdiv(m, kWaves));
  if (col_i32)
    hipLaunchKernelGGL((delta_encode_kernel<VT, int32_t>), grid, dim3(kBlock), 0, s, m, nnz, ro,
                       (const int32_t*)col, (const VT*)val, eo, total, codes, (VT*)out);
  else
    hipLaunchKernelGGL((delta_encode_kernel<VT, int16_t>), grid, dim3(kBlock), 0, s, m, nnz, ro,
                       (const int16_t*)col, (const VT*)val, eo, total, codes, (VT*)out);
  return hipGetLastError();
}

template <typename VT, typename OT>
void spmv_launch(int64_t m, int64_t n, const int32_t* eo, const uint32_t* codes, const void* val,
                 int64_t total, const void* x, void* y, hipStream_t s) {
  const dim3 grid((unsigned)std::min<int64_t>(cdiv(m, kWaves), kDeltaMaxBlocks));
  const int64_t xbytes = n * (int64_t)sizeof(VT);
  if (xbytes <= kDeltaXLds)
    hipLaunchKernelGGL((delta_spmv_kernel<VT, OT, true>), grid, dim3(kBlock), (size_t)xbytes, s,
                       m, n, eo, codes, (const VT*)val, total, (const VT*)x, (OT*)y);
  else
    hipLaunchKernelGGL((delta_spmv_kernel<VT, OT, false>), grid, dim3(kBlock), 0, s, m, n, eo,
                       codes, (const VT*)val, total, (const VT*)x, (OT*)y);
}

template <typename VT>
hipError_t spmv_vt(int64_t m, int64_t n, const int32_t* eo, const uint32_t* codes,
                   const void* val, int64_t total, const void* x, void* y, int y_dtype,
                   hipStream_t s) {
  if (y_dtype == kF32)
    spmv_launch<VT, float>(m, n, eo, codes, val, total, x, y, s);
  else
    spmv_launch<VT, VT>(m, n, eo, codes, val, total, x, y, s);
  return hipGetLastError();
}

}  // namespace

size_t delta_size_workspace_bytes(int64_t m) {
  return align256((size_t)(m + 1) * 4) + align256(4) + scan_workspace_bytes(m + 1);
}

hipError_t launch_delta_size(int64_t m, int64_t n, int64_t nnz, const int32_t* ro,
                             const void* col, int col_i32, int32_t* enc_offsets, void* ws,
                             uint32_t* total_and_bad, hipStream_t s) {
  char* c = (char*)ws;
  uint32_t* len = (uint32_t*)c;
  uint32_t* bad = (uint32_t*)(c + align256((size_t)(m + 1) * 4));
  void* scan_ws = c + align256((size_t)(m + 1) * 4) + align256(4);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(kBlock), 0, s, bad, (int64_t)1, 0u);
  hipError_t e = col_i32 ? count_it<int32_t>(m, n, nnz, ro, col, len, bad, s)
                         : count_it<int16_t>(m, n, nnz, ro, col, len, bad, s);
  if (e != hipSuccess) return e;
  e = exclusive_scan_u32(len, (uint32_t*)enc_offsets, m + 1, nullptr, scan_ws, s);
  if (e != hipSuccess) return e;
  // total (enc_offsets[m]) and the flag, for the host to read back
  if ((e = hipMemcpyAsync(total_and_bad, enc_offsets + m, 4, hipMemcpyDeviceToHost, s)) !=
      hipSuccess)
    return e;
  return hipMemcpyAsync(total_and_bad + 1, bad, 4, hipMemcpyDeviceToHost, s);
}

hipError_t launch_delta_encode(int64_t m, int64_t nnz, const int32_t* ro, const void* col,
                               int col_i32, const void* val, int dtype, const int32_t* eo,
                               int64_t total, uint32_t* codes, void* out, hipStream_t s) {
  switch (dtype) {
    case kF32: return encode_vt<float>(m, nnz, ro, col, col_i32, val, eo, total, codes, out, s);
    case kF16:
      return encode_vt<_Float16>(m, nnz, ro, col, col_i32, val, eo, total, codes, out, s);
    case kBF16: return encode_vt<bf16_t>(m, nnz, ro, col, col_i32, val, eo, total, codes, out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_delta_spmv(int64_t m, int64_t n, const int32_t* eo, const uint32_t* codes,
                             const void* val, int dtype, int64_t total, const void* x, void* y,
                             int y_dtype, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  switch (dtype) {
    case kF32: return spmv_vt<float>(m, n, eo, codes, val, total, x, y, kF32, s);
    case kF16: return spmv_vt<_Float16>(m, n, eo, codes, val, total, x, y, y_dtype, s);
    case kBF16: return spmv_vt<bf16_t>(m, n, eo, codes, val, total, x, y, y_dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spops

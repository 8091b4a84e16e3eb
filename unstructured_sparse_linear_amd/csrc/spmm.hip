// spmm.hip -- C = A * B for a CSR matrix A and a dense row-major B on gfx950
// (spops README, section "Sparse Matrix Multiplication (SpMM)").
//
// Kernels, chosen per call from N and the data layout:
// * spmm_kernel (N > 1): a group of LPR lanes owns one row and a window of
//   LPR*VEC columns; lanes load 16-byte vectors of B rows.  The entries'
//   columns and values are loaded once per group (a few lanes load a batch
//   of 8, the rest fetch them with ds_swizzle) and B, col_idx and values are
//   read through buffer resources, whose range check turns padding entries
//   into loads of zero that touch no memory.  LPR is halved while one
//   window's share of B would overflow an XCD's L2.
// * spmv_flat_kernel, spmv_row_kernel, spmv_kernel (N == 1).
//
// Row order.  Work visits rows in row_idx order (section "Usage": rows sorted
// by entry count) so that neighbouring waves get rows of similar length and
// the longest start first.  When the plan finds the lengths balanced (longest
// row at most twice the mean plus 32) whole rows are visited in index order
// instead, each XCD taking one contiguous range of rows, which keeps the B
// rows of banded matrices in L2; results are identical either way.
//
// Long rows.  The plan (build_spmm_schedule) lists the rows longer than its
// split length (kSpmmSplitLen, or kSpmmSplitLenSkewed when the lengths are
// not balanced and at most 1/32 of the rows fall between the two) in row_idx
// order and cuts each into chunks of the plan's chunk length (the longest
// row rounded up to a power of two, up to 4096 entries, when that leaves at
// least 128 chunks, else 512 entries); each chunk is one workgroup whose
// waves take contiguous slices and are summed through LDS in wave order.  A
// launch with wide row groups raises the split length back to
// kSpmmSplitLen: its chunk workgroups for shorter rows return at once and
// the row path takes those rows.  A row with several chunks writes fp32
// partial rows that spmm_fixup_kernel adds in chunk order.  Every sum has a
// fixed order, so results are bitwise reproducible.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace spops {

namespace {

constexpr int kBlock = 256;
// entries whose B vectors are loaded together (bytes in flight per lane:
// kUnroll * 16); the gathers are latency-bound, so deeper is faster
constexpr int kUnroll = 8;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

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

// ------------------------------------------------------- narrow-N groups --

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

// Store VEC fp32 results (or their rounding to 16 bits) at dst[0..VEC).
template <typename OT, int VEC>
__device__ __forceinline__ void store_vec(OT* dst, const float* acc) {
  if constexpr (sizeof(OT) == 4) {
    if constexpr (VEC == 1) {
      *dst = acc[0];
    } else if constexpr (VEC == 2) {
      *(float2*)dst = make_float2(acc[0], acc[1]);
    } else {
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q)
        *(float4*)(dst + 4 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2],
                                              acc[4 * q + 3]);
    }
  } else {
    uint32_t w[VEC / 2];
#pragma unroll
    for (int q = 0; q < VEC / 2; ++q)
      w[q] = (uint32_t)bits16(from_f32<OT>(acc[2 * q])) |
             ((uint32_t)bits16(from_f32<OT>(acc[2 * q + 1])) << 16);
    if constexpr (VEC == 2) {
      *(uint32_t*)dst = w[0];
    } else if constexpr (VEC == 4) {
      *(uint2*)dst = make_uint2(w[0], w[1]);
    } else {
      *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Accumulate entries [p0, p1) into acc for columns [j, j+VEC).
// A wave that owns a whole row (64 lanes per row): every entry is the same
// in all lanes, so its column and value are moved to scalar registers
// (readfirstlane) and the B row address is formed with scalar arithmetic; a
// lane only adds its fixed 32-bit byte offset within the row.
template <typename VT, typename IT>
__device__ __forceinline__ void accumulate_wave(const SpmmArgs& a, int64_t p0_, int64_t p1_,
                                                int64_t j, float* acc) {
  if (j >= a.N) return;
  const int p0 = __builtin_amdgcn_readfirstlane((int)p0_);
  const int p1 = __builtin_amdgcn_readfirstlane((int)p1_);
  const IT* col = (const IT*)a.col;
  const VT* val = (const VT*)a.val;
  const char* B = (const char*)a.B;
  const int64_t ldb_bytes = a.ldb * (int64_t)sizeof(VT);
  const uint32_t off = (uint32_t)(j * (int64_t)sizeof(VT));
  const uint32_t k = (uint32_t)a.k;
  constexpr int U = kUnroll;
  int p = p0;
  for (; p + U <= p1; p += U) {
    int c[U];
    float v[U];
    uint4 b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      c[u] = __builtin_amdgcn_readfirstlane((int)col[p + u]);
      v[u] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(to_f32(val[p + u]))));
      if ((uint32_t)c[u] >= k) {
        c[u] = 0;
        v[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = *(const uint4*)(B + (int64_t)c[u] * ldb_bytes + off);
#pragma unroll
    for (int u = 0; u < U; ++u) fma_vec<VT>(acc, v[u], b[u]);
  }
  for (; p < p1; ++p) {
    int c = __builtin_amdgcn_readfirstlane((int)col[p]);
    float v = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(to_f32(val[p]))));
    if ((uint32_t)c >= k) {
      c = 0;
      v = 0.f;
    }
    const uint4 b = *(const uint4*)(B + (int64_t)c * ldb_bytes + off);
    fma_vec<VT>(acc, v, b);
  }
}

template <typename VT, typename IT, int VEC, bool ALIGNED>
__device__ __forceinline__ void accumulate(const SpmmArgs& a, int64_t p0, int64_t p1, int64_t j,
                                           float* acc) {
  const IT* col = (const IT*)a.col;
  const VT* val = (const VT*)a.val;
  const VT* B = (const VT*)a.B;
  const int64_t k = a.k;
  if (j >= a.N) return;
  if constexpr (ALIGNED) {
    constexpr int U = kUnroll;
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

// ------------------------------------------------------- buffer loads --

template <int BYTES>
struct BufLoad;
template <>
struct BufLoad<4> {
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                              uint32_t* w) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  }
};
template <>
struct BufLoad<8> {
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                              uint32_t* w) {
    auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    w[0] = v[0];
    w[1] = v[1];
  }
};
template <>
struct BufLoad<16> {
  __device__ static void load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                              uint32_t* w) {
    auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
    w[3] = v[3];
  }
};


__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, _Float16*) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c,
                                false);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, bf16_t*) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, a),
                                         __builtin_bit_cast(bf162v, b), c, false);
}


// Group path with buffer loads (B, col_idx and values each under 2 GiB).
// Entries go in batches of 8.  The group's lanes share a batch's metadata:
// lane gl loads column and value of entry p + (gl mod W) (W = min(LPR, 8);
// groups of 4 lanes load two entries each), turns the column into a byte
// offset into B, and the other lanes fetch offsets and values with
// ds_swizzle.  Entries outside [q0, q1) and columns outside [0, k) get an
// offset past the end of the buffer, which reads zeros without touching
// memory, and a zero value; so every load is unconditional and the loop has
// no branch but its exit.  The next batch's metadata is requested after this
// batch's B vectors and arrives while they are consumed.

template <int LPR>
struct BatchMeta {
  static constexpr int W = LPR < 8 ? LPR : 8;  // lanes holding metadata
  static constexpr int T = 8 / W;              // entries per holding lane
  uint32_t c[T];    // column (raw bits of IT)
  uint32_t raw[T];  // value bits (fp32, or the 16-bit value)
};

template <typename T>
__device__ __forceinline__ uint32_t buf_load_elem(__amdgpu_buffer_rsrc_t rs, uint32_t i) {
  if constexpr (sizeof(T) == 2)
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, i * 2u, 0, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b32(rs, i * 4u, 0, 0);
}

template <typename VT, typename IT, int LPR>
__device__ __forceinline__ void load_meta(__amdgpu_buffer_rsrc_t crs, __amdgpu_buffer_rsrc_t vrs,
                                          int p, int gl, BatchMeta<LPR>& m) {
  using M = BatchMeta<LPR>;
#pragma unroll
  for (int t = 0; t < M::T; ++t) {
    const uint32_t e = (uint32_t)(p + gl % M::W + M::W * t);
    m.c[t] = buf_load_elem<IT>(crs, e);
    m.raw[t] = buf_load_elem<VT>(vrs, e);
  }
}

// Value of lane src (< W) of this lane's group, by ds_swizzle in bit-mask
// mode: within each half-wave, lane i reads lane (i & and_mask) | src, the
// and-mask keeping the bits that number the group.  Groups of 64 lanes work
// as two halves whose lanes 0..W-1 hold the same metadata.
template <int LPR, int SRC>
__device__ __forceinline__ uint32_t group_bcast(uint32_t v) {
  constexpr int kAnd = LPR >= 32 ? 0 : (31 & ~(LPR - 1));
  static_assert(SRC < (LPR < 32 ? LPR : 32), "source lane outside the group");
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, kAnd | (SRC << 5));
}

template <int LPR, int W, int U>
struct Bcast {  // entry U of a batch: lane U mod W, slot U / W
  __device__ static uint32_t get(const uint32_t* x) { return group_bcast<LPR, U % W>(x[U / W]); }
};

template <typename VT>
struct GroupBatch {
  static constexpr int NV = sizeof(VT) == 2 ? 4 : 8;  // 16-bit values go in pairs
  uint4 b[8];
  uint32_t v[NV];
};

// f(integral_constant<int, i>) for i = 0 .. N-1 (compile-time indices).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Check the batch at entry p (metadata in m) and request its B vectors.
template <typename VT, typename IT, int LPR>
__device__ __forceinline__ void issue_group(__amdgpu_buffer_rsrc_t brs, int64_t k, uint32_t ldbb,
                                            const BatchMeta<LPR>& m, int p, int q1, int gl,
                                            uint32_t joff, GroupBatch<VT>& x) {
  using M = BatchMeta<LPR>;
  uint32_t off[M::T], vb[M::T];
#pragma unroll
  for (int t = 0; t < M::T; ++t) {
    const int c = sizeof(IT) == 2 ? (int)(int16_t)m.c[t] : (int)m.c[t];
    const bool ok = p + gl % M::W + M::W * t < q1 && (unsigned)c < (unsigned)k;
    off[t] = ok ? (uint32_t)c * ldbb : kOob;
    vb[t] = ok ? m.raw[t] : 0u;
    if constexpr (sizeof(VT) == 2) {
      // even lanes pack their value with the next lane's: one v_dot2 pair
      const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)vb[t], 0xF5, 0xF, 0xF, false);
      vb[t] |= nb << 16;
    }
  }
  static_for<8>([&](auto u) {
    const uint32_t o = Bcast<LPR, M::W, decltype(u)::value>::get(off);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(brs, o + joff, 0, 0);
    x.b[u] = make_uint4(v[0], v[1], v[2], v[3]);
  });
  static_for<GroupBatch<VT>::NV>([&](auto q) {
    // the entry (32-bit values) or the first entry of the pair (16-bit)
    constexpr int e = sizeof(VT) == 2 ? 2 * decltype(q)::value : decltype(q)::value;
    x.v[q] = Bcast<LPR, M::W, e>::get(vb);
  });
}

template <typename VT>
__device__ __forceinline__ void consume_group(const GroupBatch<VT>& x, float* acc) {
  if constexpr (sizeof(VT) == 4) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = __uint_as_float(x.v[u]);
      acc[0] = __builtin_fmaf(v, __uint_as_float(x.b[u].x), acc[0]);
      acc[1] = __builtin_fmaf(v, __uint_as_float(x.b[u].y), acc[1]);
      acc[2] = __builtin_fmaf(v, __uint_as_float(x.b[u].z), acc[2]);
      acc[3] = __builtin_fmaf(v, __uint_as_float(x.b[u].w), acc[3]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w0[4] = {x.b[2 * t].x, x.b[2 * t].y, x.b[2 * t].z, x.b[2 * t].w};
      const uint32_t w1[4] = {x.b[2 * t + 1].x, x.b[2 * t + 1].y, x.b[2 * t + 1].z,
                              x.b[2 * t + 1].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = __builtin_amdgcn_perm(w1[d], w0[d], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(w1[d], w0[d], 0x07060302u);
        acc[2 * d] = dot2(lo, x.v[t], acc[2 * d], (VT*)nullptr);
        acc[2 * d + 1] = dot2(hi, x.v[t], acc[2 * d + 1], (VT*)nullptr);
      }
    }
  }
}

// Buffer resources of the group path.
struct GroupBufs {
  __amdgpu_buffer_rsrc_t b, c, v;
};

// Entries [q0, q1) of one row into this lane's 16 bytes of columns (byte
// offset joff within a B row).
template <typename VT, typename IT, int LPR>
__device__ __forceinline__ void accumulate_buf(const SpmmArgs& a, const GroupBufs& rs,
                                               uint32_t ldbb, int q0, int q1, int gl,
                                               uint32_t joff, float* acc) {
  if (q0 >= q1) return;
  BatchMeta<LPR> m;
  load_meta<VT, IT, LPR>(rs.c, rs.v, q0, gl, m);
  for (int p = q0; p < q1; p += 8) {
    GroupBatch<VT> x;
    issue_group<VT, IT, LPR>(rs.b, a.k, ldbb, m, p, q1, gl, joff, x);
    __builtin_amdgcn_sched_barrier(0);
    load_meta<VT, IT, LPR>(rs.c, rs.v, p + 8, gl, m);
    __builtin_amdgcn_sched_barrier(0);
    consume_group<VT>(x, acc);
  }
}

// Blocks [0, P): one chunk of a long row each.  Blocks [P, ...): kBlock/LPR
// whole rows each (rows longer than the split length are skipped there).
// Column windows: window w of LPR*VEC columns runs on blocks w, w+nwin, ...
// which the dispatcher places on the same XCD(s), so each XCD's L2 serves a
// fixed slice of B.
// BUF: B, col_idx and values are read through buffer resources (each under
// 2 GiB) with the group-shared metadata of accumulate_buf.
template <typename VT, typename OT, typename IT, int LPR, int VEC, bool ALIGNED, bool BUF>
__global__ __launch_bounds__(kBlock) void spmm_kernel(SpmmArgs a, int64_t nwin) {
  static_assert(!BUF || (ALIGNED && VEC * sizeof(VT) == 16), "buffer path loads 16 bytes");
  constexpr int GPB = kBlock / LPR;  // groups per block
  const int grp = threadIdx.x / LPR;
  const int gl = threadIdx.x % LPR;
  // Window w runs on the XCD(s) w mod 8 (block b is on XCD b mod 8).  With
  // more than 8 windows (a multiple of 8), XCD x takes its windows x, x + 8,
  // ... one after the other rather than interleaved, so its L2 holds one
  // window's share of B at a time.
  const int64_t nblk = (int64_t)gridDim.x / nwin;  // blocks per window
  int64_t bx, win;
  if (nwin > 8 && nwin % 8 == 0) {
    const int64_t k = (int64_t)blockIdx.x / 8;
    win = (int64_t)blockIdx.x % 8 + 8 * (k / nblk);
    bx = k % nblk;
  } else {
    bx = (int64_t)blockIdx.x / nwin;
    win = (int64_t)blockIdx.x % nwin;
  }
  const int64_t j = win * (LPR * VEC) + (int64_t)gl * VEC;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  // buffer path: lanes past column N read column 0 (results not stored)
  const uint32_t ldbb = (uint32_t)(a.ldb * (int64_t)sizeof(VT));
  const uint32_t joff = (uint32_t)((j < a.N ? j : 0) * (int64_t)sizeof(VT));
  GroupBufs brs;
  brs.b = make_rsrc(a.B, BUF ? (uint32_t)(a.k * a.ldb * (int64_t)sizeof(VT)) : 0u);
  brs.c = make_rsrc(a.col, BUF ? (uint32_t)(a.nnz * (int64_t)sizeof(IT)) : 0u);
  brs.v = make_rsrc(a.val, BUF ? (uint32_t)(a.nnz * (int64_t)sizeof(VT)) : 0u);

  if (bx < a.P) {
    __shared__ float red[GPB > 1 ? GPB - 1 : 1][LPR * VEC];
    const int64_t g = bx;
    const int64_t i = a.item_pos[g];
    const int64_t ch = a.item_chunk[g];
    const int64_t r = load_row(a.row_idx, a.ri_i32, i);
    int64_t rs = 0, re = 0;
    if (r >= 0 && r < a.m) row_range(a.ro, r, a.nnz, rs, re);
    // a row within this launch's split length is the row path's (uniform
    // over the workgroup: one item per workgroup)
    if (re - rs <= a.T) return;
    // chunk lengths are powers of two: shifts, no division
    const int64_t c0 = rs + (ch << a.CLs);
    const int64_t c1 = (c0 + ((int64_t)1 << a.CLs) < re) ? c0 + ((int64_t)1 << a.CLs) : re;
    const int64_t len = c1 > c0 ? c1 - c0 : 0;
    const int64_t sub = cdiv(len, GPB);
    int64_t q0 = c0 + grp * sub;
    int64_t q1 = q0 + sub;
    q0 = q0 < c1 ? q0 : c1;
    q1 = q1 < c1 ? q1 : c1;
    if constexpr (BUF)
      accumulate_buf<VT, IT, LPR>(a, brs, ldbb, (int)q0, (int)q1, gl, joff, acc);
    else
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
      const int64_t nch = (re - rs + ((int64_t)1 << a.CLs) - 1) >> a.CLs;
      if (nch <= 1) {
        if (r >= 0 && r < a.m) write_out<OT, VEC, ALIGNED>((OT*)a.C + r * a.ldc, j, a.N, acc);
      } else {
        write_out<float, VEC, ALIGNED>(a.partial + g * a.N, j, a.N, acc);
      }
    }
    return;
  }
  const int64_t nbw = nblk - a.P;
  const int64_t i = row_block(bx - a.P, nbw, a.natural) * GPB + grp;
  if (i >= a.m) return;
  const int64_t r = a.natural ? i : load_row(a.row_idx, a.ri_i32, i);
  if (r < 0 || r >= a.m) return;
  int64_t p0, p1;
  row_range(a.ro, r, a.nnz, p0, p1);
  if (a.P > 0 && p1 - p0 > a.T) return;  // handled by the chunk blocks
  if constexpr (BUF)
    accumulate_buf<VT, IT, LPR>(a, brs, ldbb, (int)p0, (int)p1, gl, joff, acc);
  else if constexpr (LPR == kWave && ALIGNED)
    accumulate_wave<VT, IT>(a, p0, p1, j, acc);
  else
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
    if (re - rs <= a.T) return;  // the row path's (uniform over the workgroup)
    const int64_t c0 = rs + (ch << a.CLs);
    const int64_t c1 = (c0 + ((int64_t)1 << a.CLs) < re) ? c0 + ((int64_t)1 << a.CLs) : re;
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
      const int64_t nch = (re - rs + ((int64_t)1 << a.CLs) - 1) >> a.CLs;
      if (nch <= 1) {
        if (r >= 0 && r < a.m) ((OT*)a.C)[r * a.ldc] = from_f32<OT>(t);
      } else {
        a.partial[g] = t;
      }
    }
    return;
  }
  const int64_t nbw = (int64_t)gridDim.x - a.P;
  const int64_t i = row_block((int64_t)blockIdx.x - a.P, nbw, a.natural) * GPB + grp;
  int64_t r = -1, p0 = 0, p1 = 0;
  if (i < a.m) {
    r = a.natural ? i : load_row(a.row_idx, a.ri_i32, i);
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

// N == 1 on balanced rows: entry-range blocks.  Workgroup b takes the
// entries [b*E, (b+1)*E) and writes the rows that start there (rows are
// owned by their first entry; the plan lists each block's first row in
// blk_row).  Its loads need no row offsets: it requests its entries, plus the
// T that follow so that its last rows end inside what it loaded, as U groups
// of four consecutive entries per lane (16-byte loads) right away, and looks
// up its rows' offsets while they are in flight.  Products val * x[col] go to
// LDS as 16-byte groups; then thread t adds row t's products in stored
// order.  This is the LDS staging of Greathouse and Daga's CSR-Stream (SC
// 2014) over an entry-balanced split of the kind Merrill and Garland use
// (merge-based SpMV, SC 2016), with each row left whole to one block instead
// of carried between blocks.  Row offsets that do not match the plan (a row
// ending past the loaded range) send the block's rows to a wave-per-row path
// that reads them from memory, so results stay the product and no access
// leaves the buffers.
// UNIT: x has a leading dimension of 1.
template <typename VT, typename OT, typename IT, int U, bool QUAD, bool UNIT>
__global__ __launch_bounds__(kBlock) void spmv_flat_kernel(SpmmArgs a) {
  extern __shared__ __align__(16) float prod[];  // E + T + 8 floats
  const IT* col = (const IT*)a.col;
  const VT* val = (const VT*)a.val;
  const VT* x = (const VT*)a.B;
  // entry positions and rows fit in 32 bits, with room for E + T past the
  // last entry (the plan takes this path only when nnz + 8192 < 2^31)
  const int k = (int)a.k, nnz = (int)a.nnz, m = (int)a.m;
  const int64_t ldx = UNIT ? 1 : a.ldb;
  const int E = a.flat_E, T = a.flat_T;
  const int nblk = (nnz + E - 1) / E;
  const int b = (int)row_block(blockIdx.x, gridDim.x, 1);
  if (b >= nblk) return;
  const int t = threadIdx.x;
  const int e0 = b * E;  // a multiple of four
  const int e1 = min(e0 + E, nnz);
  const int eL = min(e1 + T, nnz);
  // the entries first: groups of four [4g, 4g+4) inside the arrays, clamped
  // (the last group may stick out of [e0, eL); the slots past eL are
  // written but never read)
  const int gbeg = e0 >> 2;
  const int gend = QUAD ? min(nnz >> 2, (eL + 3) >> 2) : gbeg;
  IT c[U][4];
  VT v[U][4];
  if (gend > gbeg) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gq = min(gbeg + t + u * kBlock, gend - 1);
      load_quad(col + 4 * gq, c[u]);
      load_quad(val + 4 * gq, v[u]);
    }
  }
  // the owned rows [rb, re) and their offsets, while the entries arrive
  const int rb = min(max(a.blk_row[b], 0), m);
  const int re = min(max(a.blk_row[b + 1], rb), m);
  const int lo = a.ro[rb], hi = a.ro[re];
  const int r = rb + t;
  const int rl = min(r < re ? r : rb, m - 1);
  const int o0 = a.ro[rl], o1 = a.ro[rl + 1];
  const bool has_x = k > 0;  // x[0] stands in for an invalid column
  int p_done = e0;
  if (gend > gbeg) {
    p_done = max(e0, 4 * gend);
    float xv[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ci = (int)c[u][q];
        const bool ok = (unsigned)ci < (unsigned)k;
        const int xi = ok ? ci : 0;
        const float xl = has_x ? to_f32(UNIT ? x[xi] : x[(int64_t)xi * ldx]) : 0.f;
        xv[u][q] = ok ? xl : 0.f;
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = gbeg + t + u * kBlock;
      if (gu < gend) {
        float4 pr;
        pr.x = to_f32(v[u][0]) * xv[u][0];
        pr.y = to_f32(v[u][1]) * xv[u][1];
        pr.z = to_f32(v[u][2]) * xv[u][2];
        pr.w = to_f32(v[u][3]) * xv[u][3];
        *reinterpret_cast<float4*>(prod + (4 * gu - e0)) = pr;
      }
    }
  }
  // entries one at a time: everything without the 4-entry loads, else the
  // at most three past the arrays' last whole group
  for (int pp = p_done + t; pp < eL; pp += kBlock) {
    const int ci = (int)col[pp];
    const bool ok = (unsigned)ci < (unsigned)k;
    const int xi = ok ? ci : 0;
    const float xl = has_x ? to_f32(UNIT ? x[xi] : x[(int64_t)xi * ldx]) : 0.f;
    prod[pp - e0] = ok ? to_f32(val[pp]) * xl : 0.f;
  }
  __syncthreads();
  if (lo >= e0 && hi <= eL) {
    for (int rr = r; rr < re; rr += kBlock) {
      const int a0 = rr == r ? o0 : a.ro[rr];
      const int a1 = rr == r ? o1 : a.ro[rr + 1];
      const int q0 = a0 < e0 ? e0 : (a0 > eL ? eL : a0);
      const int q1 = a1 < q0 ? q0 : (a1 > eL ? eL : a1);
      float s = 0.f;
#pragma unroll 4
      for (int pp = q0; pp < q1; ++pp) s += prod[pp - e0];
      ((OT*)a.C)[(int64_t)rr * a.ldc] = from_f32<OT>(s);
    }
  } else {
    // offsets that do not match the plan: a wave per owned row
    const int w = t / kWave, l = lane_id();
    for (int rr = rb + w; rr < re; rr += kBlock / kWave) {
      int64_t p0, p1;
      row_range(a.ro, rr, nnz, p0, p1);
      float s = 0.f;
      for (int64_t p = p0 + l; p < p1; p += kWave) {
        const int ci = (int)col[p];
        if ((unsigned)ci < (unsigned)k) s = __builtin_fmaf(to_f32(val[p]), to_f32(x[ci * ldx]), s);
      }
      s = group_sum<kWave>(s);
      if (l == 0) ((OT*)a.C)[(int64_t)rr * a.ldc] = from_f32<OT>(s);
    }
  }
}

// N == 1 on balanced long rows (every row above the row-block limit): one
// workgroup per row, rows in index order with one contiguous range per XCD.
// Lanes stream the row's entries with the same clamped 4-entry loads as the
// row-block kernel and keep two fp32 sums; the workgroup adds its lanes'
// sums in a fixed order.
template <typename VT, typename OT, typename IT, bool QUAD>
__global__ __launch_bounds__(kBlock) void spmv_row_kernel(SpmmArgs a) {
  __shared__ float red[kBlock / kWave];
  const IT* col = (const IT*)a.col;
  const VT* val = (const VT*)a.val;
  const VT* x = (const VT*)a.B;
  const int k = (int)a.k, nnz = (int)a.nnz;
  const int64_t ldx = a.ldb;
  const int64_t r = row_block(blockIdx.x, gridDim.x, 1);
  if (r >= a.m) return;
  const int t = threadIdx.x;
  int base = a.ro[r], end = a.ro[r + 1];
  base = base < 0 ? 0 : (base > nnz ? nnz : base);
  end = end < base ? base : (end > nnz ? nnz : end);
  const bool has_x = k > 0;
  float acc0 = 0.f, acc1 = 0.f;
  int p_done = base;
  if constexpr (QUAD) {
    constexpr int U = kStreamQuads;
    const int gend = min(nnz >> 2, (end + 3) >> 2);
    const int gbeg = base >> 2;
    if (gend > gbeg) {
      p_done = max(base, 4 * gend);
      for (int g = gbeg + t; g < gend; g += kBlock * U) {
        IT c[U][4];
        VT v[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int gq = min(g + u * kBlock, gend - 1);
          load_quad(col + 4 * gq, c[u]);
          load_quad(val + 4 * gq, v[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int gu = g + u * kBlock;
            const int pp = 4 * gu + q;
            const int ci = (int)c[u][q];
            const bool ok = gu < gend && pp >= base && pp < end && (unsigned)ci < (unsigned)k;
            const float xl = has_x ? to_f32(x[(int64_t)(ok ? ci : 0) * ldx]) : 0.f;
            const float pr = ok ? to_f32(v[u][q]) * xl : 0.f;
            if (q & 1)
              acc1 += pr;
            else
              acc0 += pr;
          }
      }
    }
  }
  for (int pp = p_done + t; pp < end; pp += kBlock) {
    const int ci = (int)col[pp];
    const bool ok = (unsigned)ci < (unsigned)k;
    const float xl = has_x ? to_f32(x[(int64_t)(ok ? ci : 0) * ldx]) : 0.f;
    acc0 += ok ? to_f32(val[pp]) * xl : 0.f;
  }
  float s = group_sum<kWave>(acc0 + acc1);
  if (lane_id() == 0) red[t / kWave] = s;
  __syncthreads();
  if (t == 0) {
    float tot = red[0];
    for (int w = 1; w < kBlock / kWave; ++w) tot += red[w];
    ((OT*)a.C)[r * a.ldc] = from_f32<OT>(tot);
  }
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
  const float* pj = a.partial + j;
  float t = 0.f;
  int64_t g = g0;
  for (; g + 4 <= g1; g += 4) {  // four loads in flight, added in chunk order
    const float v0 = pj[g * a.N], v1 = pj[(g + 1) * a.N], v2 = pj[(g + 2) * a.N],
                v3 = pj[(g + 3) * a.N];
    t += v0;
    t += v1;
    t += v2;
    t += v3;
  }
  for (; g < g1; ++g) t += pj[g * a.N];
  ((OT*)a.C)[r * a.ldc + j] = from_f32<OT>(t);
}

// ------------------------------------------------------------ dispatch ---

int64_t pad8(int64_t x) { return (x + 7) & ~(int64_t)7; }

// Row groups of 32 or more lanes take rows up to kSpmmSplitLen whole (a
// wide group gains little from splitting shorter rows); narrower groups use
// the plan's split length.
inline SpmmArgs with_split_len(const SpmmArgs& a, bool wide) {
  SpmmArgs b = a;
  if (wide && b.T < kSpmmSplitLen) b.T = kSpmmSplitLen;
  return b;
}

template <typename VT, typename OT, typename IT, int LPR>
hipError_t launch_rows(const SpmmArgs& a0, bool aligned, hipStream_t s) {
  constexpr int VEC = Vec16<VT>::n;
  const SpmmArgs a = with_split_len(a0, LPR >= 32 || !aligned);
  if (aligned) {
    constexpr int GPB = kBlock / LPR;
    const int64_t nbw = a.natural ? pad8(cdiv(a.m, GPB)) : cdiv(a.m, GPB);
    const int64_t nwin = cdiv(a.N, LPR * VEC);
    const int64_t blocks = (a.P + nbw) * nwin;
    if (blocks == 0) return hipSuccess;
    // the pointer-load path runs for operands of 2 GiB and more, or when the
    // kOptSpmmPointerLoads switch asks for it (for its test)
    const int64_t esz = sizeof(VT) > sizeof(IT) ? sizeof(VT) : sizeof(IT);
    const bool buf = option(kOptSpmmPointerLoads) == 0 &&
                     a.k * a.ldb * (int64_t)sizeof(VT) < ((int64_t)1 << 31) &&
                     (a.nnz + 64) * esz < ((int64_t)1 << 31);
    if (buf)
      hipLaunchKernelGGL((spmm_kernel<VT, OT, IT, LPR, VEC, true, true>), dim3((unsigned)blocks),
                         dim3(kBlock), 0, s, a, nwin);
    else
      hipLaunchKernelGGL((spmm_kernel<VT, OT, IT, LPR, VEC, true, false>),
                         dim3((unsigned)blocks), dim3(kBlock), 0, s, a, nwin);
  } else {
    // scalar path: 64 lanes per row, one column each
    constexpr int G = kBlock / 64;
    const int64_t nbw = a.natural ? pad8(cdiv(a.m, G)) : cdiv(a.m, G);
    const int64_t nwin = cdiv(a.N, 64);
    const int64_t blocks = (a.P + nbw) * nwin;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((spmm_kernel<VT, OT, IT, 64, 1, false, false>), dim3((unsigned)blocks),
                       dim3(kBlock), 0, s, a, nwin);
  }
  return hipGetLastError();
}

template <typename VT, typename OT, typename IT>
hipError_t launch_typed(const SpmmArgs& a, hipStream_t s) {
  constexpr int VEC = Vec16<VT>::n;
  hipError_t e;
  bool whole_rows = false;  // every row written by one workgroup (no fixup)
  if (a.N == 1 && a.blk_row && a.flat_U > 0 && a.flat_E > 0 && a.nnz > 0) {
    // balanced rows with a plan: entry-range blocks
    const int64_t nblk = cdiv(a.nnz, (int64_t)a.flat_E);
    const dim3 grid((unsigned)pad8(nblk));
    const size_t lds = (size_t)(a.flat_E + a.flat_T + 8) * sizeof(float);
    const bool quad = ((uintptr_t)a.col % (4 * sizeof(IT)) == 0) &&
                      ((uintptr_t)a.val % (4 * sizeof(VT)) == 0);
    if (a.flat_E + a.flat_T > a.flat_U * 4 * kBlock ||
        a.nnz + a.flat_E + a.flat_T >= INT32_MAX)
      return hipErrorInvalidValue;
#define FLAT(U, Q)                                                                              \
  do {                                                                                          \
    if (a.ldb == 1)                                                                             \
      hipLaunchKernelGGL((spmv_flat_kernel<VT, OT, IT, U, Q, true>), grid, dim3(kBlock), lds, s, \
                         a);                                                                    \
    else                                                                                        \
      hipLaunchKernelGGL((spmv_flat_kernel<VT, OT, IT, U, Q, false>), grid, dim3(kBlock), lds,   \
                         s, a);                                                                 \
  } while (0)
    switch (a.flat_U) {
      case 1: if (quad) FLAT(1, true); else FLAT(1, false); break;
      case 2: if (quad) FLAT(2, true); else FLAT(2, false); break;
      case 4: if (quad) FLAT(4, true); else FLAT(4, false); break;
      default: return hipErrorInvalidValue;
    }
#undef FLAT
    e = hipGetLastError();
  } else if (a.N == 1 && a.natural && a.max_row > kFlatMaxRow) {
    // balanced long rows: a workgroup per row (the plan's row splits are not
    // used, so there is nothing to fix up)
    whole_rows = true;
    const dim3 grid((unsigned)pad8(a.m));
    const bool quad = ((uintptr_t)a.col % (4 * sizeof(IT)) == 0) &&
                      ((uintptr_t)a.val % (4 * sizeof(VT)) == 0);
    if (quad)
      hipLaunchKernelGGL((spmv_row_kernel<VT, OT, IT, true>), grid, dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((spmv_row_kernel<VT, OT, IT, false>), grid, dim3(kBlock), 0, s, a);
    e = hipGetLastError();
  } else if (a.N == 1) {
    // lanes per row from the mean row length
    const int64_t mean = a.m > 0 ? a.nnz / a.m : 0;
    int lpr = 2;
    while (lpr < 64 && lpr * 4 < mean) lpr *= 2;
    const int gpb = kBlock / lpr;
    const int64_t nbw = a.natural ? pad8(cdiv(a.m, gpb)) : cdiv(a.m, gpb);
    const dim3 grid((unsigned)(a.P + nbw));
    if (grid.x == 0) return hipSuccess;
    const SpmmArgs b = with_split_len(a, true);
    switch (lpr) {
      case 2: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 2>), grid, dim3(kBlock), 0, s, b); break;
      case 4: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 4>), grid, dim3(kBlock), 0, s, b); break;
      case 8: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 8>), grid, dim3(kBlock), 0, s, b); break;
      case 16: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 16>), grid, dim3(kBlock), 0, s, b); break;
      case 32: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 32>), grid, dim3(kBlock), 0, s, b); break;
      default: hipLaunchKernelGGL((spmv_kernel<VT, OT, IT, 64>), grid, dim3(kBlock), 0, s, b); break;
    }
    e = hipGetLastError();
  } else {
    const bool aligned = (a.N % VEC == 0) && (a.ldb % VEC == 0) && (a.ldc % VEC == 0) &&
                         ((uintptr_t)a.B % 16 == 0) && ((uintptr_t)a.C % 16 == 0) &&
                         ((uintptr_t)a.partial % 16 == 0);
    // lanes per row: enough for N (at most a wave), then halved (not below
    // 16) while the B columns one window reads exceed an XCD's 4 MB L2, so
    // that the windows the dispatcher spreads over the XCDs stay cached
    int64_t nv = cdiv(a.N, VEC);
    int64_t lpr = 4;
    while (lpr < 64 && lpr < nv) lpr *= 2;
    while (lpr > 16 && a.k * lpr * 16 > ((int64_t)4 << 20)) lpr /= 2;
    nv = lpr;
    if (nv <= 4) e = launch_rows<VT, OT, IT, 4>(a, aligned, s);
    else if (nv <= 8) e = launch_rows<VT, OT, IT, 8>(a, aligned, s);
    else if (nv <= 16) e = launch_rows<VT, OT, IT, 16>(a, aligned, s);
    else if (nv <= 32) e = launch_rows<VT, OT, IT, 32>(a, aligned, s);
    else e = launch_rows<VT, OT, IT, 64>(a, aligned, s);
  }
  if (e != hipSuccess) return e;
  if (a.S > 0 && !whole_rows) {
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
                                                          int32_t T, int32_t CL, uint32_t* nch,
                                                          uint32_t* multi, int32_t* maxlen) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const int64_t r = load_row(ri, ri_i32, i);
  int64_t p0 = 0, p1 = 0;
  if (r >= 0 && r < m) row_range(ro, r, nnz, p0, p1);
  const int64_t len = p1 - p0;
  const uint32_t c = len > T ? (uint32_t)cdiv(len, (int64_t)CL) : 0u;
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

SpmvFlat spmv_flat_shape(int64_t m, int64_t nnz, int64_t max_row, int natural, int64_t P) {
  SpmvFlat f;
  if (!(m > 0 && nnz > 0 && natural && P == 0 && max_row > 0 && max_row <= kFlatMaxRow &&
        nnz + 8192 < (int64_t)INT32_MAX))
    return f;
  // the largest blocks that still give every CU about two: fewer, larger
  // blocks measured faster on the banded 123440-row matrix (U = 4: 13.3 us,
  // 2: 14.3, 1: 14.5 cold), down to about 500 blocks
  const int32_t T = (int32_t)((max_row + 3) & ~(int64_t)3);
  for (int U = 4; U >= 1; U /= 2) {
    f.U = U;
    f.T = T;
    f.E = U * 4 * kStreamBlock - T;
    f.blocks = cdiv(nnz, (int64_t)f.E);
    if (f.blocks >= kFlatMinBlocks) break;
  }
  return f;
}

hipError_t launch_spmm(const SpmmArgs& a, hipStream_t s) {
  switch (a.dtype) {
    case kF32: return launch_vt<float>(a, s);
    case kF16: return launch_vt<_Float16>(a, s);
    case kBF16: return launch_vt<bf16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

namespace {
// blk_row[b] = first row r in [0, m] with ro[r] >= b * E for b < blocks;
// blk_row[blocks] = m.
__global__ void flat_rows_kernel(const int32_t* ro, int64_t m, int64_t E, int64_t blocks,
                                 int32_t* blk_row) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b > blocks) return;
  if (b == blocks) {
    blk_row[b] = (int32_t)m;
    return;
  }
  const int64_t e = b * E;
  int64_t lo = 0, hi = m;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if ((int64_t)ro[mid] < e) lo = mid + 1;
    else hi = mid;
  }
  blk_row[b] = (int32_t)lo;
}
}  // namespace

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
  // chunk counts, their offsets and the split rows' ranks for split length t
  // and chunk length cl
  auto count = [&](int32_t t, int32_t cl) -> hipError_t {
    host_misc[0] = host_misc[1] = host_misc[2] = 0;
    hipError_t r = hipMemcpyAsync(dev_misc, host_misc, 12, hipMemcpyHostToDevice, s);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(sched_count_kernel, dim3(g), dim3(256), 0, s, ro, row_idx, ri_i32, m, nnz,
                       t, cl, nch, multi, dev_misc);
    if ((r = hipGetLastError()) != hipSuccess) return r;
    if ((r = exclusive_scan_u32(nch, off, m, (uint32_t*)dev_misc + 1, sws, s)) != hipSuccess)
      return r;
    if ((r = exclusive_scan_u32(multi, mrank, m, (uint32_t*)dev_misc + 2, sws, s)) != hipSuccess)
      return r;
    if ((r = hipMemcpyAsync(host_misc, dev_misc, 12, hipMemcpyDeviceToHost, s)) != hipSuccess)
      return r;
    return hipStreamSynchronize(s);
  };
  int32_t CL = kSpmmChunkLen;
  out->CL = CL;
  do {
    if ((e = count(T, CL)) != hipSuccess) break;
    out->max_row = host_misc[0];
    // balanced lengths: keep index order for locality
    out->natural = (out->max_row <= 2 * (nnz / m) + 32) ? 1 : 0;
    // skewed lengths: rows from the shorter split length on get their own
    // workgroups too, for the narrow row groups that can use them, when the
    // rows this adds (one chunk each) are rare stragglers among short rows;
    // where they are common, a workgroup each costs more than it saves
    if (!out->natural && T > kSpmmSplitLenSkewed) {
      const int64_t p_long = host_misc[1];
      if ((e = count(kSpmmSplitLenSkewed, CL)) != hipSuccess) break;
      if ((host_misc[1] - p_long) * 32 <= m)
        out->T = T = kSpmmSplitLenSkewed;
      else if ((e = count(T, CL)) != hipSuccess)
        break;
    }
    // rows up to kSpmmChunkLenMax entries whole in one workgroup each (no
    // partial rows to add up afterwards) while that still leaves at least
    // kSpmmMinChunkItems chunk workgroups; else kSpmmChunkLen
    if (out->max_row > CL) {
      int32_t cl = CL;
      while (cl < out->max_row && cl < kSpmmChunkLenMax) cl *= 2;
      if ((e = count(T, cl)) != hipSuccess) break;
      if (host_misc[1] >= kSpmmMinChunkItems)
        out->CL = CL = cl;
      else if ((e = count(T, CL)) != hipSuccess)
        break;
    }
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
    out->flat = spmv_flat_shape(m, nnz, out->max_row, out->natural, out->P);
    if (out->flat.U > 0) {
      const int64_t nb = out->flat.blocks;
      if ((e = hipMalloc(&out->blk_row, (size_t)(nb + 1) * 4)) != hipSuccess) break;
      hipLaunchKernelGGL(flat_rows_kernel, dim3((unsigned)cdiv(nb + 1, 256)), dim3(256), 0, s, ro,
                         m, (int64_t)out->flat.E, nb, out->blk_row);
      if ((e = hipGetLastError()) != hipSuccess) break;
    }
    e = hipStreamSynchronize(s);
  } while (0);
  (void)hipFree(tmp);  // e already reports the schedule's outcome
  if (e != hipSuccess) free_spmm_schedule(out);
  return e;
}

void free_spmm_schedule(SpmmSchedule* sch) {
  // teardown: nothing to report
  if (sch->mem) (void)hipFree(sch->mem);
  if (sch->blk_row) (void)hipFree(sch->blk_row);
  *sch = SpmmSchedule{};
}

}  // namespace spops

// common.h -- device helpers shared by the gfx950 kernels of libspops.
//
// Element formats: f32 (float), f16 (IEEE binary16, _Float16) and bf16
// (bfloat16 kept as its 16-bit pattern).  All arithmetic is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spops {

constexpr int kWave = 64;  // CDNA wavefront width

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct bf16_t {
  uint16_t bits;
};

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float((uint32_t)x.bits << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// v_cvt_f16_f32 rounds to nearest even and keeps subnormals.
template <>
__device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// Round to nearest even on the bit pattern; NaN stays a quiet NaN.
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  bf16_t r;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    r.bits = (uint16_t)((u >> 16) | 0x40u);
  } else {
    r.bits = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  return r;
}

// Unpack 16-bit pairs held in one 32-bit word.
__device__ __forceinline__ float lo_f32(uint32_t w, _Float16*) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_f32(uint32_t w, _Float16*) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float lo_f32(uint32_t w, bf16_t*) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w, bf16_t*) {
  return __uint_as_float(w & 0xffff0000u);
}

template <typename T>
__device__ __forceinline__ uint16_t bits16(T x) {
  return __builtin_bit_cast(uint16_t, x);
}
template <>
__device__ __forceinline__ uint16_t bits16<bf16_t>(bf16_t x) { return x.bits; }

// --------------------------------------------------------------- indices --

// Index lists are int16 or int32.  Negative (or >= extent) values are
// treated as out of range by the callers.
template <typename I>
__device__ __forceinline__ int load_index(const I* p, int64_t i) {
  return (int)p[i];
}

// --------------------------------------------------------- buffer loads --

// Raw buffer resource over `bytes` bytes at p (dword 3 as for untyped 32-bit
// data on gfx9).  Loads at offsets at or past `bytes` return zeros without a
// memory access, which the kernels use to mask entries without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}
// An offset past the end of every buffer the kernels read this way (each is
// under 2 GiB).
constexpr uint32_t kOob = 0x80000000u;

// ------------------------------------------------------------ wave tools --

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

template <typename T>
__device__ __forceinline__ T wave_uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}

// Sum over aligned groups of G lanes (G a power of two <= 64), fixed order:
// every lane of the group ends up with the same value.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with six DPP adds and no
// LDS traffic: shifts by 1, 2, 4 and 8 lanes inside each 16-lane row (lanes
// shifted in from outside the row read 0), then lane 15 of rows 0 and 2 is
// added to rows 1 and 3 (row_bcast:15) and lane 31 to rows 2 and 3
// (row_bcast:31).  Every lane gets the sum of lanes 0..itself.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp_u32<0x111, 0xF>(v);  // row_shr:1
  v += dpp_u32<0x112, 0xF>(v);  // row_shr:2
  v += dpp_u32<0x114, 0xF>(v);  // row_shr:4
  v += dpp_u32<0x118, 0xF>(v);  // row_shr:8
  v += dpp_u32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Largest r in [lo, hi) with ro[r] <= p, assuming ro nondecreasing on that
// range and ro[lo] <= p.  Used to find the row owning position p.
__device__ __forceinline__ int64_t upper_row(const int32_t* ro, int64_t lo, int64_t hi,
                                             int64_t p) {
  // invariant: ro[lo] <= p, answer in [lo, hi)
  while (hi - lo > 1) {
    int64_t mid = lo + ((hi - lo) >> 1);
    if ((int64_t)ro[mid] <= p)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Wave-cooperative version of upper_row over [0, m): every lane probes one
// of 64 evenly spaced offsets per step, so the range shrinks 64-fold per
// dependent load instead of 2-fold.  All lanes must call it with the same p;
// all get the same (wave-uniform) answer.
__device__ __forceinline__ int64_t wave_upper_row(const int32_t* ro, int64_t m, int64_t p) {
  int64_t lo = 0, hi = m;  // answer in [lo, hi), ro[lo] <= p assumed
  const int lane = lane_id();
  while (hi - lo > 1) {
    const int64_t step = cdiv(hi - lo, kWave);
    const int64_t idx = lo + (int64_t)lane * step;
    const bool le = idx < hi && (int64_t)ro[idx] <= p;
    const uint64_t mask = __ballot(le);
    const int last = mask ? 63 - __builtin_clzll(mask) : 0;
    lo = lo + (int64_t)last * step;
    const int64_t nhi = lo + step;
    hi = nhi < hi ? nhi : hi;
  }
  return wave_uniform((int)lo);
}

// Whole-row block index -> first row position.  In index order each XCD gets
// one contiguous range of row blocks (blocks b, b+8, ... share an XCD); grids
// for this mapping are padded to a multiple of 8 blocks.
__device__ __forceinline__ int64_t row_block(int64_t bw, int64_t nbw_padded, int natural) {
  if (!natural) return bw;
  const int64_t per = nbw_padded / 8;
  return (bw % 8) * per + bw / 8;
}

template <int BYTES>
struct QuadLoad;
template <>
struct QuadLoad<16> {
  typedef uint4 type;
};
template <>
struct QuadLoad<8> {
  typedef uint2 type;
};

// Four consecutive elements from a 4-element-aligned address.
template <typename T>
__device__ __forceinline__ void load_quad(const T* p, T (&out)[4]) {
  typedef typename QuadLoad<4 * sizeof(T)>::type Q;
  const Q q = *reinterpret_cast<const Q*>(p);
  __builtin_memcpy(out, &q, sizeof(Q));
}

}  // namespace spops

// sddmm.hip -- general SDDMM on gfx950 (spops README, section "Sampled
// Dense-Dense Matrix Multiplication (SDDMM)", the kernel for any pattern):
//     out[p] = sum_k A[r][k] * BT[c][k]   for each stored position p = (r, c).
//
// Two kernels:
//   * sddmm_list_kernel, for 16-byte vectors along K: a wave takes a run of
//     consecutive entries (of the mask in CSR order for the general backend,
//     or of the structure-aware plan's remainder list) and computes their dot
//     products with its lanes split along K (details at the kernel);
//   * sddmm_scalar_kernel, for K, leading dimensions or pointers that do not
//     allow 16-byte vectors: a wave per group of 8 entries, lane l takes
//     k = l, l+64, ...
// Dots use v_dot2_f32_f16 / v_dot2_f32_bf16 (two products per lane per
// instruction, fp32 accumulation) or v_fma_f32, and each entry's partial sums
// are combined in a fixed order, so results are deterministic.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int kBlock = 256;


typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

template <typename VT>
struct Traits;
template <>
struct Traits<float> {
  static constexpr int vec = 4;
  __device__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = __builtin_fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = __builtin_fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = __builtin_fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = __builtin_fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
    return acc;
  }
};
template <>
struct Traits<_Float16> {
  static constexpr int vec = 8;
  __device__ static float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b),
                                  acc, false);
  }
  __device__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = dot2(a.x, b.x, acc);
    acc = dot2(a.y, b.y, acc);
    acc = dot2(a.z, b.z, acc);
    acc = dot2(a.w, b.w, acc);
    return acc;
  }
};
template <>
struct Traits<bf16_t> {
  static constexpr int vec = 8;
  __device__ static float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, a),
                                           __builtin_bit_cast(bf162v, b), acc, false);
  }
  __device__ static float dot(const uint4& a, const uint4& b, float acc) {
    acc = dot2(a.x, b.x, acc);
    acc = dot2(a.y, b.y, acc);
    acc = dot2(a.z, b.z, acc);
    acc = dot2(a.w, b.w, acc);
    return acc;
  }
};

// Scalar path for K, leading dims or pointers that do not allow 16-byte
// vectors: a wave takes 8 consecutive entries of the mask in CSR order and
// computes them one after the other, lane l taking k = l, l+64, ...
template <typename VT, typename OT, typename IT>
__global__ __launch_bounds__(kBlock) void sddmm_scalar_kernel(SddmmArgs a) {
  constexpr int E = 8;
  const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
  const int lane = lane_id();
  const int64_t wb = wave * E;
  if (wb >= a.count) return;
  const int64_t we = (wb + E < a.count) ? wb + E : a.count;
  const int64_t m = a.m;
  int64_t r = wave_upper_row(a.ro, m, wb);
  const VT* A = (const VT*)a.A;
  const VT* BT = (const VT*)a.BT;
  const IT* col = (const IT*)a.col;
  for (int64_t e = wb; e < we; ++e) {
    r = upper_row(a.ro, r, m, e);  // a binary search past any empty rows
    const int c = (int)col[e];
    float s = 0.f;
    if ((unsigned)c < (unsigned)a.n) {
      for (int64_t k = lane; k < a.K; k += kWave)
        s = __builtin_fmaf(to_f32(A[r * a.lda + k]), to_f32(BT[(int64_t)c * a.ldbt + k]), s);
    }
    s = group_sum<kWave>(s);
    if (lane == 0) ((OT*)a.out)[e] = from_f32<OT>(s);
  }
}

template <typename VT, typename OT, typename IT>
hipError_t launch_typed(const SddmmArgs& a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(cdiv(a.count, 8) * kWave, kBlock));
  hipLaunchKernelGGL((sddmm_scalar_kernel<VT, OT, IT>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------- entry lists --

// Cross-lane exchanges without LDS.  For a partner offset o <= 8 a DPP
// move gives every lane the value of a lane in the other half of its aligned
// 2o-lane block (o = 1, 2: lane ^ o; o = 4: mirror inside 8 lanes; o = 8:
// mirror inside 16 lanes).  For o = 16 and 32 gfx950's v_permlane16_swap and
// v_permlane32_swap swap odd 16-lane rows of x with even rows of y, and the
// upper 32 lanes of x with the lower 32 of y; adding the two results gives,
// in the lower half of every 2o-lane block, x summed with its partner lane
// and, in the upper half, y summed with its partner lane.
template <int O>
__device__ __forceinline__ float dpp_partner(float v) {
  constexpr int ctrl = O == 1 ? 0xB1 : O == 2 ? 0x4E : O == 4 ? 0x141 : 0x140;
  static_assert(O == 1 || O == 2 || O == 4 || O == 8, "DPP partner offsets are 1, 2, 4, 8");
  return __uint_as_float(
      __builtin_amdgcn_update_dpp(0u, __float_as_uint(v), ctrl, 0xF, 0xF, false));
}
template <int O>
__device__ __forceinline__ float swap_sum(float x, float y) {
  static_assert(O == 16 || O == 32, "swap offsets are 16, 32");
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// One halving step at offset O: lanes whose bit O is clear keep values
// [0, H) and add their partner's; the others keep [H, 2H).
template <int O, int H, int U>
__device__ __forceinline__ void halve(float (&w)[U], int gl) {
#pragma unroll
  for (int j = 0; j < H; ++j) {
    if constexpr (O >= 16) {
      w[j] = swap_sum<O>(w[j], w[j + H]);
    } else {
      const bool up = (gl & O) != 0;
      const float send = up ? w[j] : w[j + H];
      const float keep = up ? w[j + H] : w[j];
      w[j] = keep + dpp_partner<O>(send);
    }
  }
}
template <int O>
__device__ __forceinline__ float pair_sum(float v) {
  if constexpr (O >= 16)
    return swap_sum<O>(v, v);
  else
    return v + dpp_partner<O>(v);
}

// Sum of U values over aligned groups of LPN lanes in log2(LPN) exchange
// steps instead of U*log2(LPN): log2(U) halving steps at offsets LPN/2,
// LPN/4, ... leave one value per lane, then pair sums over the remaining
// LPN/U lanes.  On return lane gl of a group holds the total of value
// gl / (LPN/U).  The order of additions is fixed for every lane.
template <int LPN, int U>
__device__ __forceinline__ float group_sum_multi(const float (&v)[U], int gl) {
  static_assert(U >= 1 && U <= 4 && U <= LPN && (U & (U - 1)) == 0, "U in {1, 2, 4}, U <= LPN");
  float w[U];
#pragma unroll
  for (int j = 0; j < U; ++j) w[j] = v[j];
  if constexpr (U >= 2) halve<LPN / 2, U / 2>(w, gl);
  if constexpr (U >= 4) halve<LPN / 4, U / 4>(w, gl);
  constexpr int S = LPN / U;
  float t = w[0];
  if constexpr (S >= 64) t = pair_sum<32>(t);
  if constexpr (S >= 32) t = pair_sum<16>(t);
  if constexpr (S >= 16) t = pair_sum<8>(t);
  if constexpr (S >= 8) t = pair_sum<4>(t);
  if constexpr (S >= 4) t = pair_sum<2>(t);
  if constexpr (S >= 2) t = pair_sum<1>(t);
  return t;
}

// Entry list (the structure-aware plan's remainder): entry j is mask position
// pos[j] in row rows[j]; rows ascend inside a bucket.  Bucket b = blockIdx % nb
// (its blocks share XCD b), so the BT rows gathered by one XCD come from one
// column range.
//
// A wave takes E consecutive entries of its bucket and first loads one
// entry's row, position and column per lane, so the loop below issues only
// operand loads.  The wave is cut into groups of LPN lanes that split K into
// 16-byte vectors (lane l holds vectors v*LPN + l, so a group's loads of a row
// are contiguous); group g owns entries [g*E/G, (g+1)*E/G).  A step of a group
// takes up to U consecutive entries of one row: A's row slice is loaded into
// registers when the row changes and reused otherwise, the U rows of BT are
// loaded together, and the U dot products are reduced together.  When K needs
// more than one pass of LPN*KV vectors, A is reloaded per pass.
template <typename VT, typename OT, typename IT, int LPN, int KV, int U, int E, bool FULL>
__global__ __launch_bounds__(kWave) void sddmm_list_kernel(SddmmListArgs a) {
  static_assert(E <= kWave && E % (kWave / LPN) == 0, "one entry per lane");
  using TR = Traits<VT>;
  constexpr int VEC = TR::vec;
  constexpr int G = kWave / LPN;
  constexpr int EG = E / G;
  // One wave per workgroup: the wave index is blockIdx, a scalar, so the
  // loop bounds and the rows derived from it stay in scalar registers.
  // The grid is a multiple of nb; a wave takes chunks wave, wave + per, ...
  const bool split = a.ksplit > 1;
  // buckets: b = blockIdx mod nb (bucket b on XCD b mod 8); with more than
  // 8 K pieces, the first 8 * per workgroups take pieces 0..7 (piece x on
  // XCD x), the next 8 * per pieces 8..15, and so on, so each XCD works
  // through its pieces one after the other
  const int64_t per = gridDim.x / (unsigned)a.nb;
  const bool seq = split && a.nb > 8;
  const int b = seq ? (int)(blockIdx.x % 8 + 8 * ((blockIdx.x / 8) / per))
                    : (int)(blockIdx.x % (unsigned)a.nb);
  const int64_t w0 = seq ? (int64_t)((blockIdx.x / 8) % per) : (int64_t)(blockIdx.x / a.nb);
  const int bb = split ? 0 : b;  // K pieces share bucket 0's entry range
  const int64_t bs = a.bstart_dev ? (int64_t)a.bstart_dev[bb] : a.bstart[bb];
  const int64_t be = a.bstart_dev ? (int64_t)a.bstart_dev[bb + 1] : a.bstart[bb + 1];
  for (int64_t wave = w0; bs + wave * E < be; wave += per) {
  const int64_t wb = bs + wave * E;
  const int nw = (int)((be - wb < E) ? be - wb : E);
  const int lane = lane_id();
  const int g = G == 1 ? 0 : lane / LPN;
  const int gl = G == 1 ? lane : lane % LPN;
  const int n = (int)a.n;
  const IT* col = (const IT*)a.col;

  int my_r = 0, my_p = 0, my_c = -1;
  if (a.ro) {
    // CSR order: rows of the wave's first and last entries by a 64-way
    // search, then each lane's row by binary search between them
    const int64_t rf = wave_upper_row(a.ro, a.m, wb);
    const int64_t rl = wave_upper_row(a.ro, a.m, wb + nw - 1);
    if (lane < nw) {
      my_p = (int)(wb + lane);
      my_r = (int)upper_row(a.ro, rf, rl + 1, wb + lane);
    }
  } else if (lane < nw) {
    my_r = a.rows[wb + lane];
    my_p = a.pos[wb + lane];
  }
  // raw column (validated where it is used, so the first A load below need
  // not wait for it); a list with its own columns saves the dependent load
  if (lane < nw) my_c = (!a.ro && a.cols) ? a.cols[wb + lane] : (int)col[my_p];
  // from here on my_p is the output index: the mask position, or with a K
  // split the entry's index in the range (into this piece's partial sums)
  if (split) my_p = (int)(wb + lane - bs);

  const int g0 = g * EG;
  const int g1 = (g0 + EG < nw) ? g0 + EG : nw;  // may be <= g0
  const int64_t kvec = a.K / VEC;
  const int64_t npass = cdiv(kvec, (int64_t)LPN * KV);
  const VT* A = (const VT*)a.A + (split ? b * a.kpiece : 0);
  const VT* BT = (const VT*)a.BT + (split ? b * a.kpiece : 0);
  OT* out = split ? (OT*)(a.part + (int64_t)b * (be - bs)) : (OT*)a.out;
  const bool cache_a = FULL || npass == 1;

  // FULL: K is exactly one pass (kvec == LPN * KV), so no vector is out of
  // range and the loads of a row differ only by constant offsets.
  auto load_slice = [&](const VT* rowp, int64_t pass, uint4* dst) {
    if constexpr (FULL) {
      const uint4* q = (const uint4*)rowp + gl;
#pragma unroll
      for (int v = 0; v < KV; ++v) dst[v] = q[v * LPN];
    } else {
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        const int64_t kv = (pass * KV + v) * LPN + gl;
        dst[v] = kv < kvec ? *(const uint4*)(rowp + kv * VEC) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // entry q's row, column and position (q is group-uniform)
  auto fetch = [&](int src, int& r, int& c, int& p) {
    if constexpr (G == 1) {
      r = __builtin_amdgcn_readlane(my_r, src);
      c = __builtin_amdgcn_readlane(my_c, src);
      p = __builtin_amdgcn_readlane(my_p, src);
    } else {
      r = __shfl(my_r, src, 64);
      c = __shfl(my_c, src, 64);
      p = __shfl(my_p, src, 64);
    }
  };

  // The first A row is requested right after the column loads, so its
  // latency overlaps theirs (vector loads complete in issue order).
  int rcur = -1;
  uint4 acur[KV];
  if (cache_a) {
    const int r0 = G == 1 ? __builtin_amdgcn_readlane(my_r, 0) : __shfl(my_r, g0, 64);
    if (g0 < g1) {
      load_slice(A + (int64_t)r0 * a.lda, 0, acur);
      rcur = r0;
    }
  }
  int i = g0;
  while (true) {
    const bool act = i < g1;
    if constexpr (G == 1) {
      if (!act) break;
    } else {
      if (__ballot(act) == 0) break;
    }
    int r[U], c[U], p[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = i + u;
      fetch(q < g1 ? q : g0, r[u], c[u], p[u]);
      if ((unsigned)c[u] >= (unsigned)n) c[u] = -1;
    }
    ok[0] = act;
#pragma unroll
    for (int u = 1; u < U; ++u) ok[u] = ok[u - 1] && (i + u < g1) && r[u] == r[0];
    float s[U];
    uint4 bv[U][KV];
    if (cache_a) {
      if (act && r[0] != rcur) {
        load_slice(A + (int64_t)r[0] * a.lda, 0, acur);
        rcur = r[0];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ok[u]) load_slice(BT + (int64_t)(c[u] >= 0 ? c[u] : 0) * a.ldbt, 0, bv[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u] = 0.f;
        if (ok[u]) {
#pragma unroll
          for (int v = 0; v < KV; ++v) s[u] = TR::dot(acur[v], bv[u][v], s[u]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) s[u] = 0.f;
      for (int64_t pass = 0; pass < npass; ++pass) {
        if (act) load_slice(A + (int64_t)r[0] * a.lda, pass, acur);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ok[u]) load_slice(BT + (int64_t)(c[u] >= 0 ? c[u] : 0) * a.ldbt, pass, bv[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (ok[u]) {
#pragma unroll
            for (int v = 0; v < KV; ++v) s[u] = TR::dot(acur[v], bv[u][v], s[u]);
          }
        }
      }
    }
    const float t = group_sum_multi<LPN, U>(s, gl);
    constexpr int SUB = LPN / U;
    const int uo = gl / SUB;
    int po = p[0];
    bool oko = ok[0], cvo = c[0] >= 0;
#pragma unroll
    for (int u = 1; u < U; ++u)
      if (uo == u) {
        po = p[u];
        oko = ok[u];
        cvo = c[u] >= 0;
      }
    if (gl % SUB == 0 && oko) out[po] = from_f32<OT>(cvo ? t : 0.f);
    int taken = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) taken += ok[u] ? 1 : 0;
    i += taken;
  }
  }
}

template <typename VT, typename OT, typename IT, int LPN, int KV, int U, int E>
hipError_t launch_list_ue(const SddmmListArgs& a, hipStream_t s) {
  int64_t most = 0;
  if (a.ksplit > 1) {
    most = a.bstart_dev ? a.max_bucket : a.bstart[1] - a.bstart[0];
  } else if (a.bstart_dev) {
    most = a.max_bucket;  // bucket bounds on the device: a host-side bound
  } else {
    for (int b = 0; b < a.nb; ++b) {
      const int64_t cnt = a.bstart[b + 1] - a.bstart[b];
      most = cnt > most ? cnt : most;
    }
  }
  // one wave per chunk of E entries, capped so the grid stays well inside
  // its limits (waves then loop over several chunks); with bounds only known
  // on the device, at most 8192 waves loop over the buckets' chunks
  int64_t waves_per_bucket = cdiv(most, E);
  if (waves_per_bucket == 0) return hipSuccess;
  const int64_t cap = a.bstart_dev ? (int64_t)8192 : (int64_t)1 << 22;
  if (waves_per_bucket * a.nb > cap) waves_per_bucket = cap / a.nb;
  constexpr int VEC = Traits<VT>::vec;
  const dim3 grid((unsigned)(waves_per_bucket * a.nb));
  if (a.K == (int64_t)LPN * KV * VEC)
    hipLaunchKernelGGL((sddmm_list_kernel<VT, OT, IT, LPN, KV, U, E, true>), grid, dim3(kWave), 0,
                       s, a);
  else
    hipLaunchKernelGGL((sddmm_list_kernel<VT, OT, IT, LPN, KV, U, E, false>), grid, dim3(kWave),
                       0, s, a);
  return hipGetLastError();
}

// U = 4 entries per step and 16 entries per wave were the fastest of
// U in {1, 2, 4} x E in {8, 16, 32, 64} on the K = 2048 and K = 256
// remainders measured (MI355X, cold caches); for K = 32 (8-lane groups) 64
// entries per wave beat 16.
template <typename VT, typename OT, typename IT, int LPN, int KV>
hipError_t launch_list(const SddmmListArgs& a, hipStream_t s) {
  // 16 entries per wave for 32- and 64-lane groups; narrower groups (small
  // K) take 64 so that each group still gets several entries
  constexpr int E = LPN >= 32 ? 16 : kWave;
  return launch_list_ue<VT, OT, IT, LPN, KV, (LPN < 4 ? LPN : 4), E>(a, s);
}

template <typename VT, typename OT, typename IT>
hipError_t launch_list_typed(const SddmmListArgs& a, hipStream_t s) {
  constexpr int VEC = Traits<VT>::vec;
  const int64_t kvec = a.K / VEC;
  if (kvec <= 4) return launch_list<VT, OT, IT, 4, 1>(a, s);
  if (kvec <= 8) return launch_list<VT, OT, IT, 8, 1>(a, s);
  if (kvec <= 16) return launch_list<VT, OT, IT, 16, 1>(a, s);
  if (kvec <= 32) return launch_list<VT, OT, IT, 32, 1>(a, s);
  if (kvec <= 64) return launch_list<VT, OT, IT, 64, 1>(a, s);
  if (kvec <= 128) return launch_list<VT, OT, IT, 64, 2>(a, s);
  if (kvec <= 256) return launch_list<VT, OT, IT, 64, 4>(a, s);
  return launch_list<VT, OT, IT, 64, 8>(a, s);
}

template <typename VT>
hipError_t launch_list_vt(const SddmmListArgs& a, hipStream_t s) {
  if (a.out_dtype == kF32)
    return a.col_i32 ? launch_list_typed<VT, float, int32_t>(a, s)
                     : launch_list_typed<VT, float, int16_t>(a, s);
  if constexpr (sizeof(VT) == 2)
    return a.col_i32 ? launch_list_typed<VT, VT, int32_t>(a, s)
                     : launch_list_typed<VT, VT, int16_t>(a, s);
  return hipErrorInvalidValue;
}

template <typename VT>
hipError_t launch_vt(const SddmmArgs& a, hipStream_t s) {
  if (a.out_dtype == kF32)
    return a.col_i32 ? launch_typed<VT, float, int32_t>(a, s)
                     : launch_typed<VT, float, int16_t>(a, s);
  if constexpr (sizeof(VT) == 2)
    return a.col_i32 ? launch_typed<VT, VT, int32_t>(a, s) : launch_typed<VT, VT, int16_t>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

// K, leading dimensions or pointers that do not allow 16-byte vectors along K
// (the entry-list kernel needs them).
namespace {
template <typename OT>
// All of an entry's pieces (at most 16) and its position are requested
// together, then added in piece order.
__global__ __launch_bounds__(256) void sddmm_piece_sum_kernel(const float* part, int pieces,
                                                              int64_t count, const int32_t* pos,
                                                              int64_t start, OT* out) {
  constexpr int kMaxPieces = 16;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < count;
       j += (int64_t)gridDim.x * 256) {
    const int32_t q = pos[start + j];
    float p[kMaxPieces];
#pragma unroll
    for (int b = 0; b < kMaxPieces; ++b) p[b] = b < pieces ? part[(int64_t)b * count + j] : 0.f;
    float v = p[0];
#pragma unroll
    for (int b = 1; b < kMaxPieces; ++b)
      if (b < pieces) v += p[b];
    out[q] = from_f32<OT>(v);
  }
}
}  // namespace

hipError_t launch_sddmm_piece_sum(const float* part, int pieces, int64_t count,
                                  const int32_t* pos, int64_t start, void* out, int out_dtype,
                                  hipStream_t s) {
  if (count <= 0) return hipSuccess;
  if (pieces < 1 || pieces > 16) return hipErrorInvalidValue;
  const int64_t g = cdiv(count, 256);
  const dim3 grid((unsigned)(g < 2048 ? g : 2048));
  if (out_dtype == kF32)
    hipLaunchKernelGGL(sddmm_piece_sum_kernel<float>, grid, dim3(256), 0, s, part, pieces, count,
                       pos, start, (float*)out);
  else if (out_dtype == kF16)
    hipLaunchKernelGGL(sddmm_piece_sum_kernel<_Float16>, grid, dim3(256), 0, s, part, pieces,
                       count, pos, start, (_Float16*)out);
  else
    hipLaunchKernelGGL(sddmm_piece_sum_kernel<bf16_t>, grid, dim3(256), 0, s, part, pieces,
                       count, pos, start, (bf16_t*)out);
  return hipGetLastError();
}

hipError_t launch_sddmm_general(const SddmmArgs& a, hipStream_t s) {
  switch (a.dtype) {
    case kF32: return launch_vt<float>(a, s);
    case kF16: return launch_vt<_Float16>(a, s);
    case kBF16: return launch_vt<bf16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

// The list kernel needs 16-byte vectors along K (K, lda, ldbt multiples of
// the vector width, 16-byte aligned A and BT); the caller checks.
hipError_t launch_sddmm_list(const SddmmListArgs& a0, hipStream_t s) {
  SddmmListArgs a = a0;
  if (a.ksplit > 1) {
    // pieces of K: the kernel takes K = kpiece (a multiple of the vector)
    // and writes fp32 partial sums
    if (!a.part || a.kpiece <= 0 || a.ksplit * a.kpiece != a.K || a.ksplit > 16 ||
        (a.ksplit > 8 && a.ksplit % 8 != 0))
      return hipErrorInvalidValue;
    a.nb = a.ksplit;
    a.K = a.kpiece;
    a.out_dtype = kF32;
  } else if (a.nb < 1 || a.nb > kMaxBuckets) {
    return hipErrorInvalidValue;
  }
  switch (a.dtype) {
    case kF32: return launch_list_vt<float>(a, s);
    case kF16: return launch_list_vt<_Float16>(a, s);
    case kBF16: return launch_list_vt<bf16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spops

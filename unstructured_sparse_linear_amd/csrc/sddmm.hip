// sddmm.hip -- general SDDMM on gfx950 (spops README, section "Sampled
// Dense-Dense Matrix Multiplication (SDDMM)", the kernel for any pattern):
//     out[p] = sum_k A[r][k] * BT[c][k]   for each stored position p = (r, c).
//
// Work mapping.  Entries are independent, so each wavefront takes a fixed
// slice of E consecutive entries (balanced for any row-length mix, including
// rows with thousands of entries) and finds the first row of its slice with a
// wave-uniform binary search of the row offsets.  A wave is cut into groups
// of LPN lanes; a group owns a contiguous sub-slice and computes one entry's
// dot product with its lanes split along K: lane l holds 16-byte vectors
// v*LPN + l of the K axis, so the group's loads of a BT row are contiguous.
// The group's slice of A[r, :] stays in registers while consecutive entries
// share r.  Dots use v_dot2_f32_f16 / v_dot2_f32_bf16 (two products per lane
// per instruction, fp32 accumulation) or v_fma_f32; the LPN partial sums are
// combined with a fixed xor-shuffle tree.
//
// K split (optional).  When BT is larger than an XCD's 4 MB L2, K can be cut
// into ks slices; slice s runs on blocks s, s+ks, ... which the dispatcher
// places on the same XCD(s), so each L2 only holds its slice of BT.  Each slice
// writes its partial dot products to a workspace and a second kernel adds the
// ks partials of every entry in slice order (deterministic).
//
// The same kernel runs the remainder of the structure-aware backend, where
// entry j of a sub-matrix stands for mask position pos[j].
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

template <typename IT>
__device__ __forceinline__ int64_t mask_pos(const SddmmArgs& a, int64_t j) {
  return a.pos ? (int64_t)a.pos[j] : j;
}

// Entries per wavefront for a group width: each group takes 16 entries, or
// 32 for 64-lane groups, so the row search and the A-row loads of a wave are
// amortized over enough dot products.
template <int LPN>
constexpr int entries_per_wave() {
  return (kWave / LPN) * (LPN == kWave ? 32 : 16);
}

// Vectorised path.  KV = 16-byte vectors per lane per pass; K is covered in
// npass passes of LPN*KV vectors (npass == 1 keeps A in registers).
template <typename VT, typename OT, typename IT, int LPN, int KV>
__global__ __launch_bounds__(kBlock) void sddmm_vec_kernel(SddmmArgs a) {
  using TR = Traits<VT>;
  constexpr int VEC = TR::vec;
  constexpr int G = kWave / LPN;
  constexpr int E = entries_per_wave<LPN>();
  constexpr int U = 4;
  const int64_t slice = (int64_t)blockIdx.x % a.ks;
  const int64_t wave = ((int64_t)blockIdx.x / a.ks * kBlock + threadIdx.x) / kWave;
  const int lane = lane_id();
  const int grp = lane / LPN;
  const int gl = lane % LPN;
  const int64_t wb = wave * E;
  if (wb >= a.count) return;
  const int64_t we = (wb + E < a.count) ? wb + E : a.count;
  // this group's sub-slice
  const int64_t per = cdiv(we - wb, G);
  int64_t e = wb + grp * per;
  const int64_t e1 = (e + per < we) ? e + per : we;
  if (e > we) e = we;

  const int64_t m = a.m;
  const int32_t* ro = a.ro;
  int64_t r = wave_upper_row(ro, m, wb);
  while (r < m - 1 && (int64_t)ro[r + 1] <= e) ++r;

  // this slice's 16-byte vectors of the K axis: [kv0, kv1)
  const int64_t kvall = a.K / VEC;
  const int64_t kvper = cdiv(kvall, a.ks);
  const int64_t kv0 = slice * kvper;
  const int64_t kv1 = (kv0 + kvper < kvall) ? kv0 + kvper : kvall;
  const int64_t kvec = kv1 > kv0 ? kv1 - kv0 : 0;
  const int64_t npass = cdiv(kvec, (int64_t)LPN * KV);
  const VT* A = (const VT*)a.A + kv0 * VEC;
  const VT* BT = (const VT*)a.BT + kv0 * VEC;
  const IT* col = (const IT*)a.col;
  OT* out = (OT*)a.out;
  float* part = a.ks > 1 ? a.partial + slice * a.count : nullptr;
  const int64_t n = a.n;

  auto load_slice = [&](const VT* rowp, int64_t pass, uint4* dst) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int64_t kv = (pass * KV + v) * LPN + gl;
      dst[v] = kv < kvec ? *(const uint4*)(rowp + kv * VEC) : make_uint4(0, 0, 0, 0);
    }
  };

  uint4 areg[KV];
  if (e < e1) load_slice(A + r * a.lda, 0, areg);
  while (e < e1) {
    int64_t re = ro[r + 1];
    re = re < e1 ? re : e1;
    if (re <= e) re = e1;  // malformed offsets: never stall
    if (npass == 1) {
      for (; e + U <= re; e += U) {
        int64_t p[U];
        int c[U];
        uint4 b[U][KV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u] = mask_pos<IT>(a, e + u);
          c[u] = (int)col[p[u]];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int cc = ((unsigned)c[u] < (unsigned)n) ? c[u] : 0;
          load_slice(BT + (int64_t)cc * a.ldbt, 0, b[u]);
        }
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          s[u] = 0.f;
#pragma unroll
          for (int v = 0; v < KV; ++v) s[u] = TR::dot(areg[v], b[u][v], s[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = group_sum<LPN>(s[u]);
        if (gl == 0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float r = ((unsigned)c[u] < (unsigned)n) ? s[u] : 0.f;
            if (part)
              part[e + u] = r;
            else
              out[p[u]] = from_f32<OT>(r);
          }
        }
      }
    }
    for (; e < re; ++e) {
      const int64_t p = mask_pos<IT>(a, e);
      const int c = (int)col[p];
      const int cc = ((unsigned)c < (unsigned)n) ? c : 0;
      float s = 0.f;
      for (int64_t pass = 0; pass < npass; ++pass) {
        uint4 b[KV];
        if (npass > 1) load_slice(A + r * a.lda, pass, areg);
        load_slice(BT + (int64_t)cc * a.ldbt, pass, b);
#pragma unroll
        for (int v = 0; v < KV; ++v) s = TR::dot(areg[v], b[v], s);
      }
      s = group_sum<LPN>(s);
      if (gl == 0) {
        const float r = ((unsigned)c < (unsigned)n) ? s : 0.f;
        if (part)
          part[e] = r;
        else
          out[p] = from_f32<OT>(r);
      }
    }
    if (e >= e1) break;
    // next non-empty row
    while (r < m - 1 && (int64_t)ro[r + 1] <= e) ++r;
    load_slice(A + r * a.lda, 0, areg);
  }
}

// Scalar path for K, leading dims or pointers that do not allow 16-byte
// vectors: one wave per entry group of 64 lanes, lane l takes k = l, l+64, ...
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
    while (r < m - 1 && (int64_t)a.ro[r + 1] <= e) ++r;
    const int64_t p = mask_pos<IT>(a, e);
    const int c = (int)col[p];
    float s = 0.f;
    if ((unsigned)c < (unsigned)a.n) {
      for (int64_t k = lane; k < a.K; k += kWave)
        s = __builtin_fmaf(to_f32(A[r * a.lda + k]), to_f32(BT[(int64_t)c * a.ldbt + k]), s);
    }
    s = group_sum<kWave>(s);
    if (lane == 0) ((OT*)a.out)[p] = from_f32<OT>(s);
  }
}

// out[pos(j)] = sum over slices of partial[s * count + j], slices in order.
template <typename OT>
__global__ __launch_bounds__(kBlock) void sddmm_reduce_kernel(SddmmArgs a) {
  const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (j >= a.count) return;
  float t = 0.f;
  for (int64_t q = 0; q < a.ks; ++q) t += a.partial[q * a.count + j];
  ((OT*)a.out)[a.pos ? (int64_t)a.pos[j] : j] = from_f32<OT>(t);
}

template <typename VT, typename OT, typename IT, int LPN, int KV>
hipError_t launch_vec(const SddmmArgs& a, hipStream_t s) {
  constexpr int E = entries_per_wave<LPN>();
  const int64_t waves = cdiv(a.count, E);
  const dim3 grid((unsigned)(cdiv(waves * kWave, kBlock) * a.ks));
  hipLaunchKernelGGL((sddmm_vec_kernel<VT, OT, IT, LPN, KV>), grid, dim3(kBlock), 0, s, a);
  if (a.ks > 1)
    hipLaunchKernelGGL(sddmm_reduce_kernel<OT>, dim3((unsigned)cdiv(a.count, kBlock)),
                       dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <typename VT, typename OT, typename IT>
hipError_t launch_typed(SddmmArgs a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  constexpr int VEC = Traits<VT>::vec;
  const bool aligned = a.K > 0 && (a.K % VEC == 0) && (a.lda % VEC == 0) &&
                       (a.ldbt % VEC == 0) && ((uintptr_t)a.A % 16 == 0) &&
                       ((uintptr_t)a.BT % 16 == 0);
  if (!aligned) {
    a.ks = 1;
    const dim3 grid((unsigned)cdiv(cdiv(a.count, 8) * kWave, kBlock));
    hipLaunchKernelGGL((sddmm_scalar_kernel<VT, OT, IT>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
  }
  if (a.ks < 1 || !a.partial) a.ks = 1;
  const int64_t kvec = cdiv(a.K / VEC, a.ks);
  if (kvec <= 4) return launch_vec<VT, OT, IT, 4, 1>(a, s);
  if (kvec <= 8) return launch_vec<VT, OT, IT, 8, 1>(a, s);
  if (kvec <= 16) return launch_vec<VT, OT, IT, 16, 1>(a, s);
  if (kvec <= 32) return launch_vec<VT, OT, IT, 32, 1>(a, s);
  if (kvec <= 64) return launch_vec<VT, OT, IT, 64, 1>(a, s);
  if (kvec <= 128) return launch_vec<VT, OT, IT, 64, 2>(a, s);
  if (kvec <= 256) return launch_vec<VT, OT, IT, 64, 4>(a, s);
  return launch_vec<VT, OT, IT, 64, 8>(a, s);
}

// ---------------------------------------------------------- entry lists --

// Entry list (the structure-aware plan's remainder): entry j is mask position
// pos[j] in row rows[j]; rows ascend inside a bucket.  Bucket b = blockIdx % nb
// (its blocks share XCD b), so the BT rows gathered by one XCD come from one
// column range.  Groups of LPN lanes split K as in sddmm_vec_kernel; A's row
// slice is reloaded only when the row changes.
template <typename VT, typename OT, typename IT, int LPN, int KV>
__global__ __launch_bounds__(kBlock) void sddmm_list_kernel(SddmmListArgs a) {
  using TR = Traits<VT>;
  constexpr int VEC = TR::vec;
  constexpr int G = kWave / LPN;
  constexpr int E = entries_per_wave<LPN>();
  constexpr int U = 4;
  const int b = (int)(blockIdx.x % (unsigned)a.nb);
  const int64_t wave = (int64_t)(blockIdx.x / (unsigned)a.nb) * (kBlock / kWave) +
                       threadIdx.x / kWave;
  const int64_t bs = a.bstart[b], be = a.bstart[b + 1];
  const int64_t wb = bs + wave * E;
  if (wb >= be) return;
  const int64_t we = (wb + E < be) ? wb + E : be;
  const int lane = lane_id();
  const int grp = lane / LPN;
  const int gl = lane % LPN;
  const int64_t per = cdiv(we - wb, G);
  int64_t e = wb + grp * per;
  const int64_t e1 = (e + per < we) ? e + per : we;
  if (e > we) e = we;

  const int64_t kvec = a.K / VEC;
  const int64_t npass = cdiv(kvec, (int64_t)LPN * KV);
  const VT* A = (const VT*)a.A;
  const VT* BT = (const VT*)a.BT;
  const IT* col = (const IT*)a.col;
  OT* out = (OT*)a.out;
  const int64_t n = a.n;

  auto load_slice = [&](const VT* rowp, int64_t pass, uint4* dst) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int64_t kv = (pass * KV + v) * LPN + gl;
      dst[v] = kv < kvec ? *(const uint4*)(rowp + kv * VEC) : make_uint4(0, 0, 0, 0);
    }
  };

  int64_t rcur = -1;
  uint4 areg[KV];
  while (e < e1) {
    if (npass == 1 && e + U <= e1) {
      int64_t r[U], p[U];
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        r[u] = a.rows[e + u];
        p[u] = a.pos[e + u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = (int)col[p[u]];
      if (r[0] == r[U - 1]) {  // rows ascend, so the U entries share a row
        if (r[0] != rcur) {
          rcur = r[0];
          load_slice(A + rcur * a.lda, 0, areg);
        }
        uint4 bv[U][KV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int cc = ((unsigned)c[u] < (unsigned)n) ? c[u] : 0;
          load_slice(BT + (int64_t)cc * a.ldbt, 0, bv[u]);
        }
        float sacc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          sacc[u] = 0.f;
#pragma unroll
          for (int v = 0; v < KV; ++v) sacc[u] = TR::dot(areg[v], bv[u][v], sacc[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) sacc[u] = group_sum<LPN>(sacc[u]);
        if (gl == 0) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            out[p[u]] = from_f32<OT>(((unsigned)c[u] < (unsigned)n) ? sacc[u] : 0.f);
        }
        e += U;
        continue;
      }
    }
    const int64_t r = a.rows[e];
    const int64_t p = a.pos[e];
    const int c = (int)col[p];
    const int cc = ((unsigned)c < (unsigned)n) ? c : 0;
    float sacc = 0.f;
    for (int64_t pass = 0; pass < npass; ++pass) {
      if (npass > 1 || r != rcur) load_slice(A + r * a.lda, pass, areg);
      uint4 bv[KV];
      load_slice(BT + (int64_t)cc * a.ldbt, pass, bv);
#pragma unroll
      for (int v = 0; v < KV; ++v) sacc = TR::dot(areg[v], bv[v], sacc);
    }
    rcur = npass == 1 ? r : -1;
    sacc = group_sum<LPN>(sacc);
    if (gl == 0) out[p] = from_f32<OT>(((unsigned)c < (unsigned)n) ? sacc : 0.f);
    ++e;
  }
}

template <typename VT, typename OT, typename IT, int LPN, int KV>
hipError_t launch_list(const SddmmListArgs& a, hipStream_t s) {
  constexpr int E = entries_per_wave<LPN>();
  int64_t most = 0;
  for (int b = 0; b < a.nb; ++b) {
    const int64_t cnt = a.bstart[b + 1] - a.bstart[b];
    most = cnt > most ? cnt : most;
  }
  const int64_t blocks_per_bucket = cdiv(cdiv(most, E), kBlock / kWave);
  if (blocks_per_bucket == 0) return hipSuccess;
  hipLaunchKernelGGL((sddmm_list_kernel<VT, OT, IT, LPN, KV>),
                     dim3((unsigned)(blocks_per_bucket * a.nb)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
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

// Measured on MI355X, splitting K costs more (one reduction and one output
// write per slice and entry) than the L2 residency of the slices saves for
// the shapes benchmarked here, so the split is off unless SPOPS_SDDMM_KSPLIT
// asks for it (a cap on the number of slices, rounded down to a power of 2).
int64_t sddmm_k_slices(int64_t n, int64_t K, int dtype) {
  const char* env = getenv("SPOPS_SDDMM_KSPLIT");
  const int64_t cap = env ? atoll(env) : 1;
  const int64_t es = dtype == kF32 ? 4 : 2;
  const int64_t budget = 5 << 19;  // ~2.5 MB of BT per L2
  int64_t ks = 1;
  while (2 * ks <= cap && ks < 8 && n * K * es / ks > budget && K / (2 * ks) >= 128) ks *= 2;
  return ks;
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
hipError_t launch_sddmm_list(const SddmmListArgs& a, hipStream_t s) {
  if (a.nb < 1 || a.nb > kMaxBuckets) return hipErrorInvalidValue;
  switch (a.dtype) {
    case kF32: return launch_list_vt<float>(a, s);
    case kF16: return launch_list_vt<_Float16>(a, s);
    case kBF16: return launch_list_vt<bf16_t>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace spops

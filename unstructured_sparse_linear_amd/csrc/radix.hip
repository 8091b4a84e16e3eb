// radix.hip -- prefix sums and stable LSD radix sorting on gfx950, and the
// two operations built from them:
//   * csr_transpose (spops README, section "CSR Transpose"): a stable sort of
//     the stored entries by column; the output row offsets are the column
//     boundaries of the sorted keys;
//   * the row_idx order (section "Usage"): rows sorted by entry count, most
//     first, ties by ascending row -- a stable sort on (cols - count);
// and, for a pattern transposed once and its values many times, the
// transpose's permutation (the transpose of the entry indices, moved as
// 4-byte values) and a kernel that applies a permutation to values.
//
// Sorting is least-significant-digit radix with 8-bit digits, in three
// kernels per pass: per-tile digit counts, one exclusive scan over the
// digit-major count table, and a stable scatter.  Inside a tile the rank of
// each key among equal digits is found from a 64-lane match (the lanes of a
// wave holding the same digit, as a bit mask) plus per-wave digit counts in
// LDS, so no atomic's ordering decides any position and the output is
// deterministic.  No kernel waits on another
// block, so no launch order assumptions are made.
#include <stdlib.h>

#include <type_traits>

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
  const uint32_t x = wave_inclusive_sum(s);
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

// Whole exclusive scan in one workgroup of 1024 threads for n up to 65536.
// The array is read in 16 chunks of 4096 values; thread t takes values
// 4t..4t+3 of every chunk (one 16-byte load each, all issued before any
// arithmetic), so loads are coalesced and their latencies overlap.  Chunk
// and wave totals are combined through a 256-entry table in LDS.
constexpr int kSingleThreads = 1024;
constexpr int kSingleChunks = 16;
constexpr int64_t kSingleChunk = kSingleThreads * 4;
constexpr int64_t kSingleMax = kSingleChunk * kSingleChunks;

__global__ __launch_bounds__(kSingleThreads) void scan_single_kernel(const uint32_t* in,
                                                                     uint32_t* out, int64_t n,
                                                                     uint32_t* total) {
  constexpr int NW = kSingleThreads / kWave;
  __shared__ uint32_t wt[2][NW];  // wave totals of a chunk, double-buffered
  const int t = threadIdx.x, w = t / kWave, l = lane_id();
  uint4 v[kSingleChunks];
#pragma unroll
  for (int c = 0; c < kSingleChunks; ++c) {
    const int64_t b = c * kSingleChunk + (int64_t)t * 4;
    if (b + 3 < n) {
      v[c] = *(const uint4*)(in + b);
    } else {
      v[c].x = b < n ? in[b] : 0u;
      v[c].y = b + 1 < n ? in[b + 1] : 0u;
      v[c].z = b + 2 < n ? in[b + 2] : 0u;
      v[c].w = 0u;
    }
  }
  uint32_t carry = 0;  // total of the chunks before this one (same in every thread)
#pragma unroll
  for (int c = 0; c < kSingleChunks; ++c) {
    if (c * kSingleChunk >= n) break;
    const uint32_t s = v[c].x + v[c].y + v[c].z + v[c].w;
    const uint32_t x = wave_inclusive_sum(s);
    if (l == kWave - 1) wt[c & 1][w] = x;
    __syncthreads();
    uint32_t off = carry, tot = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const uint32_t q = wt[c & 1][ww];
      off += ww < w ? q : 0u;
      tot += q;
    }
    uint32_t run = off + x - s;
    const int64_t b = c * kSingleChunk + (int64_t)t * 4;
    uint4 o;
    o.x = run;
    run += v[c].x;
    o.y = run;
    run += v[c].y;
    o.z = run;
    run += v[c].z;
    o.w = run;
    if (b + 3 < n) {
      *(uint4*)(out + b) = o;
    } else {
      if (b < n) out[b] = o.x;
      if (b + 1 < n) out[b + 1] = o.y;
      if (b + 2 < n) out[b + 2] = o.z;
    }
    carry += tot;
  }
  if (t == 0 && total) *total = carry;
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

// Second payload of a scatter: none, or the raw bits of a 2- or 4-byte value.
struct NoPay {
  __device__ uint32_t operator()(int64_t) const { return 0u; }
};
template <int VB>
struct ValBits {  // VB == 0: no values (zero bits)
  const void* p;
  __device__ uint32_t operator()(int64_t i) const {
    if constexpr (VB == 4) return ((const uint32_t*)p)[i];
    else if constexpr (VB == 2) return (uint32_t)((const uint16_t*)p)[i];
    else return 0u;
  }
};

// Lanes of the wave whose (valid) digit equals this lane's, as a bit mask.
// Lanes holding lane 0's digit take it from one ballot; every other valid
// lane ORs its bit into its digit's 64-bit mask in LDS (`match`, this wave's
// row, all zero on entry and on return), reads the mask back and clears it
// -- one wave's LDS operations complete in issue order, so each read sees all
// of the call's ORs and each clear follows all of its reads.  Clustered keys
// (where LDS atomics on one address would serialize) mostly share lane 0's
// digit, so the LDS traffic is left to the scattered rest.
__device__ __forceinline__ uint64_t digit_peers(bool valid, uint32_t d, uint64_t* match,
                                                uint64_t lanebit) {
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)d);
  const bool first = valid && d == d0;
  const uint64_t same = __ballot(first);
  uint64_t peers = 0;
  if (valid && !first) {
    atomicOr((unsigned long long*)&match[d], (unsigned long long)lanebit);
    peers = match[d];
    match[d] = 0;
  }
  return first ? same : peers;
}

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

// Digit counts of tile b (workgroups b < ntiles) and, when row offsets `ro`
// of m rows are given (the transpose's first pass), the row owning every
// stored position of rows [b*rpb, (b+1)*rpb) (rows_of), so no separate launch
// expands the row offsets.  TM: counts stored tile-major,
// counts[tile * kRadix + d] (the layout radix_scatter_kernel reads when it
// derives its own offsets), else digit-major like radix_count_kernel.
template <class KS, bool TM>
__global__ __launch_bounds__(kThreads) void transpose_count_kernel(
    KS ks, int64_t n, int shift, uint32_t mask, uint32_t* counts, int64_t ntiles,
    const int32_t* __restrict__ ro, int64_t m, int64_t rpb, uint32_t* __restrict__ rows_of) {
  __shared__ uint32_t hist[kRadix];
  __shared__ int32_t rol[kThreads + 1];  // the block's row offsets
  const int t = threadIdx.x;
  const bool tile = blockIdx.x < ntiles;
  hist[t] = 0;
  const int64_t i0 = (int64_t)blockIdx.x * kTile + (int64_t)t * kItems;
  uint32_t key[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) key[q] = tile && i0 + q < n ? ks(i0 + q) : 0u;
  // rpb <= kThreads: the rpb + 1 offsets are read in one round (rpb <=
  // kExpandRows as launched)
  const int64_t r0 = (int64_t)blockIdx.x * rpb;
  const int nr = (int)(r0 >= m ? 0 : (m - r0 < rpb ? m - r0 : rpb));
  if (nr > 0 && t <= nr) rol[t] = ro[r0 + t];  // (nr == 0: no offset is read)
  if (t == 0 && nr == kThreads) rol[kThreads] = ro[r0 + kThreads];
  __syncthreads();
  // one wave per row (loop bounds are wave-uniform)
  const int w = t / kWave, lane = lane_id();
  for (int j = w; j < nr; j += kThreads / kWave) {
    int64_t p0 = rol[j], p1 = rol[j + 1];
    p0 = p0 < 0 ? 0 : p0;
    p1 = p1 > n ? n : p1;
    for (int64_t p = p0 + lane; p < p1; p += kWave) rows_of[p] = (uint32_t)(r0 + j);
  }
  __syncthreads();
  if (!tile) return;
  // lanes sharing lane 0's digit add once through their lowest lane (keys
  // of a tile are often clustered, and LDS atomics on one address serialize)
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const bool v = i0 + q < n;
    const uint32_t d = (key[q] >> shift) & mask;
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)d);
    const uint64_t same = __ballot(v && d == d0);
    if (v && d == d0 && (same & lt) == 0) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    if (v && d != d0) atomicAdd(&hist[d], 1u);
  }
  __syncthreads();
  counts[TM ? (int64_t)blockIdx.x * kRadix + t : (int64_t)t * ntiles + blockIdx.x] = hist[t];
}

// Stable scatter.  Keys of a tile are taken in rounds of kThreads (round-major,
// then thread order == index order).  In a round each wave finds the lanes
// holding the same digit (digit_peers); the lowest such lane publishes the
// count; digit offsets per wave then follow from the running per-digit base.
// RB != 0: a second payload VS2 too, and each entry goes out as one record
// at kout (an array of n records), one store per entry: RB = 16, {key, pay,
// pay2, 0}; RB = 8, {pay << shift | key's bits below shift, pay2} (pay below
// 2^(32 - shift)).
//
// SELF (single pass, ntiles <= kSelfMaxTiles): `offs` holds the raw digit
// counts, tile-major, and every workgroup derives its own offsets from the
// whole table: base of digit d in tile b = (entries of all digits below d) +
// (entries of digit d in tiles below b).  Workgroup 0 also stores the digit
// starts to bstart[0..kRadix) (if given), which replaces the scan launch.
constexpr int64_t kSelfMaxTiles = 128;
constexpr int64_t kExpandRows = 32;  // most rows one count workgroup expands

template <class KS, class VS, class VS2, int RB, bool SELF = false>
__global__ __launch_bounds__(kThreads) void radix_scatter_kernel(
    KS ks, VS vs, int64_t n, int shift, int nbits, const uint32_t* offs, int64_t ntiles,
    uint32_t* kout, uint32_t* vout, VS2 vs2, uint32_t* bstart = nullptr) {
  constexpr bool kTwo = RB != 0;
  __shared__ uint32_t base_d[kRadix];
  __shared__ uint32_t wcnt[kThreads / kWave][kRadix];
  // per wave and digit: the lanes of the current round holding it
  __shared__ uint64_t match[kThreads / kWave][kRadix];
  const int t = threadIdx.x;
  const int w = t / kWave;
  const uint32_t mask = (1u << nbits) - 1u;
  if constexpr (!SELF) base_d[t] = offs[(int64_t)t * ntiles + blockIdx.x];
#pragma unroll
  for (int ww = 0; ww < kThreads / kWave; ++ww) match[ww][t] = 0;
  const int64_t tbase = (int64_t)blockIdx.x * kTile;
  const uint64_t lt = lanemask_lt();
  const uint64_t lanebit = lt + 1;
  // all keys and payloads of the tile are loaded before the first round
  uint32_t keys[kItems], pay[kItems], pay2[kTwo ? kItems : 1];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int64_t i = tbase + r * kThreads + t;
    keys[r] = i < n ? ks(i) : 0u;
    pay[r] = i < n ? vs(i) : 0u;
    if constexpr (kTwo) pay2[r] = i < n ? vs2(i) : 0u;
  }
  if constexpr (SELF) {
    // thread t sums digits 4*(t % 64) .. +3 over tiles t/64, t/64 + 4, ...
    // (16-byte loads, up to 32 per thread, all in flight together), split
    // into tiles below this one and all tiles; the four phases meet in LDS.
    __shared__ uint4 part[2 * 4 * kWave];  // [pre, all][phase][lane]
    const int q = t % kWave, ph = t / kWave;
    constexpr int kLoads = (int)(kSelfMaxTiles / 4);
    uint4 c[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int64_t tl = ph + 4 * j;
      c[j] = tl < ntiles ? ((const uint4*)offs)[tl * (kRadix / 4) + q] : make_uint4(0, 0, 0, 0);
    }
    uint4 pre = make_uint4(0, 0, 0, 0), tot = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      tot.x += c[j].x;
      tot.y += c[j].y;
      tot.z += c[j].z;
      tot.w += c[j].w;
      if (ph + 4 * j < (int64_t)blockIdx.x) {
        pre.x += c[j].x;
        pre.y += c[j].y;
        pre.z += c[j].z;
        pre.w += c[j].w;
      }
    }
    part[ph * kWave + q] = pre;
    part[(4 + ph) * kWave + q] = tot;
    __syncthreads();
    // thread t now owns digit t
    const uint32_t* pw = (const uint32_t*)part;
    uint32_t dpre = 0, dtot = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      dpre += pw[(p * kWave + t / 4) * 4 + t % 4];
      dtot += pw[((4 + p) * kWave + t / 4) * 4 + t % 4];
    }
    const uint32_t inc = wave_inclusive_sum(dtot);
    if (lane_id() == kWave - 1) wcnt[0][w] = inc;
    __syncthreads();
    uint32_t below = inc - dtot;
    for (int ww = 0; ww < w; ++ww) below += wcnt[0][ww];
    base_d[t] = below + dpre;
    if (blockIdx.x == 0 && bstart) bstart[t] = below;
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
#pragma unroll
    for (int ww = 0; ww < kThreads / kWave; ++ww) wcnt[ww][t] = 0;
    __syncthreads();
    const int64_t i = tbase + r * kThreads + t;
    const bool valid = i < n;
    const uint32_t key = keys[r];
    const uint32_t d = (key >> shift) & mask;
    const uint64_t peers = digit_peers(valid, d, match[w], lanebit);
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
      if constexpr (RB == 16) {
        ((uint4*)kout)[dst] = make_uint4(key, pay[r], pay2[r], 0u);
      } else if constexpr (RB == 8) {
        ((uint2*)kout)[dst] =
            make_uint2((pay[r] << shift) | (key & ((1u << shift) - 1u)), pay2[r]);
      } else {
        kout[dst] = key;
        vout[dst] = pay[r];
      }
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
// payload iota.  Returns the buffer index holding the result.  Up to
// kSelfMaxTiles tiles a pass is two launches (count, then a scatter that
// derives its own offsets), else three (count, scan, scatter).
template <class KS0>
hipError_t radix_sort_iota(KS0 ks0, int64_t n, int bits, const RadixWs& R, int* result,
                           hipStream_t s) {
  const int64_t ntiles = cdiv(n, kTile);
  if (bits < 1) bits = 1;
  int cur = -1;  // -1: source functor; else buffer index holding current keys
  int dst = 0;
  const bool self = ntiles <= kSelfMaxTiles;
  for (int shift = 0; shift < bits; shift += kRadixBits) {
    const int nb = (bits - shift) < kRadixBits ? (bits - shift) : kRadixBits;
    const uint32_t mask = (1u << nb) - 1u;
    if (self) {
      // count (clustered lanes added once) and a scatter that derives its
      // own offsets: two launches per pass
      if (cur < 0) {
        hipLaunchKernelGGL((transpose_count_kernel<KS0, true>), dim3(ntiles), dim3(kThreads), 0,
                           s, ks0, n, shift, mask, R.counts, ntiles, nullptr, 0, 0, nullptr);
        hipLaunchKernelGGL((radix_scatter_kernel<KS0, ValIota, NoPay, 0, true>), dim3(ntiles),
                           dim3(kThreads), 0, s, ks0, ValIota{}, n, shift, nb, R.counts, ntiles,
                           R.keys[dst], R.vals[dst], NoPay{}, nullptr);
      } else {
        const KeyFromU32 kc{R.keys[cur]};
        hipLaunchKernelGGL((transpose_count_kernel<KeyFromU32, true>), dim3(ntiles),
                           dim3(kThreads), 0, s, kc, n, shift, mask, R.counts, ntiles, nullptr, 0,
                           0, nullptr);
        hipLaunchKernelGGL((radix_scatter_kernel<KeyFromU32, ValFromU32, NoPay, 0, true>),
                           dim3(ntiles), dim3(kThreads), 0, s, kc, ValFromU32{R.vals[cur]}, n,
                           shift, nb, R.counts, ntiles, R.keys[dst], R.vals[dst], NoPay{},
                           nullptr);
      }
      cur = dst;
      dst ^= 1;
      continue;
    }
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
      hipLaunchKernelGGL((radix_scatter_kernel<KS0, ValIota, NoPay, 0>), dim3(ntiles),
                         dim3(kThreads), 0, s, ks0, ValIota{}, n, shift, nb, R.counts, ntiles,
                         R.keys[dst], R.vals[dst], NoPay{});
    } else {
      hipLaunchKernelGGL((radix_scatter_kernel<KeyFromU32, ValFromU32, NoPay, 0>), dim3(ntiles),
                         dim3(kThreads), 0, s, KeyFromU32{R.keys[cur]}, ValFromU32{R.vals[cur]},
                         n, shift, nb, R.counts, ntiles, R.keys[dst], R.vals[dst], NoPay{});
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

// Second stage of the two-level transpose.  The entries were stably grouped
// by coarse column digit c >> SH (one radix pass); workgroup d now orders
// bucket d by the fine digit c & (F - 1), F = 2^SH <= 512, stably; bucket d
// starts at bstart[d * bstride] and ends where bucket d + 1 starts.  The
// bucket is cut into one contiguous slice per wave.  Each wave counts the
// fine digits of its slice (its own row of an LDS table); one pass over the
// table gives, per digit, the count in earlier slices, and a scan over the
// digit totals gives the bucket's output row offsets.  Then every wave walks
// its slice in rounds of 64 entries with no further barrier: an entry's rank
// among equal digits of the round comes from digit_peers, its destination
// is digit base + earlier slices + the wave's running count, and the first
// lane of each digit advances that count.  The first pass wrote each
// entry's column, row and value bits as one 16-byte record, so the slice is
// read sequentially, four rounds ahead of their use.
constexpr int kFinishThreads = 1024;
constexpr int kFinishWaves = kFinishThreads / kWave;
constexpr int kMaxFine = 512;

// Records as the first pass wrote them (RB = 8 or 16 bytes, see
// radix_scatter_kernel): fine digit, row and value bits of each entry.
template <int RB>
struct Rec;
template <>
struct Rec<16> {
  uint4 r;
  __device__ uint32_t fine(uint32_t fmask, int) const { return r.x & fmask; }
  __device__ uint32_t row(int) const { return r.y; }
  __device__ uint32_t bits() const { return r.z; }
};
template <>
struct Rec<8> {
  uint2 r;
  __device__ uint32_t fine(uint32_t fmask, int) const { return r.x & fmask; }
  __device__ uint32_t row(int sh) const { return r.x >> sh; }
  __device__ uint32_t bits() const { return r.y; }
};

template <typename OI, int VB, int RB, int SUB>
__global__ __launch_bounds__(kFinishThreads) void transpose_bucket_kernel(
    const Rec<RB>* rec, const uint32_t* bstart, int64_t bstride, int64_t nnz, int64_t n, int sh,
    uint8_t* out_val, int32_t* out_ro, OI* out_col) {
  __shared__ uint32_t base_f[kMaxFine];
  __shared__ uint32_t wcnt[kFinishWaves][kMaxFine];
  __shared__ uint32_t wsum[kMaxFine / kWave];
  // per wave and fine digit: the lanes of the current round holding it
  __shared__ uint64_t match[kFinishWaves][kMaxFine];
  const int t = threadIdx.x, w = t / kWave, lane = lane_id();
  const int d = blockIdx.x;
  const int F = 1 << sh;
  const uint32_t fmask = (uint32_t)F - 1u;
  const int64_t bs = bstart[(int64_t)d * bstride];
  const int64_t be = d + 1 < kRadix ? (int64_t)bstart[(int64_t)(d + 1) * bstride] : nnz;
  const uint64_t lt = lanemask_lt();
  const uint64_t lanebit = lt + 1;
  for (int k = t; k < kFinishWaves * F; k += kFinishThreads) {
    wcnt[k / F][k % F] = 0;
    match[k / F][k % F] = 0;
  }
  __syncthreads();
  // this wave's slice [s0, s1) of the bucket
  const int64_t len = be - bs;
  const int64_t L = cdiv(len, (int64_t)kFinishWaves);
  const int64_t s0 = bs + (w * L < len ? w * L : len);
  const int64_t s1 = bs + ((w + 1) * L < len ? (w + 1) * L : len);
  // per-slice digit counts, eight key loads in flight per lane
  for (int64_t q = s0 + lane; q < s1; q += 8 * kWave) {
    uint32_t kk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t qi = q + (int64_t)i * kWave;
      kk[i] = rec[qi < s1 ? qi : s1 - 1].r.x;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (q + (int64_t)i * kWave < s1) atomicAdd(&wcnt[w][kk[i] & fmask], 1u);
  }
  __syncthreads();
  // per digit: counts of earlier slices; digit totals scanned over digits
  const int fpad = F < kWave ? kWave : F;
  uint32_t cnt = 0, inc = 0;
  if (t < fpad) {
    if (t < F) {
      uint32_t run = 0;
#pragma unroll
      for (int ww = 0; ww < kFinishWaves; ++ww) {
        const uint32_t c = wcnt[ww][t];
        wcnt[ww][t] = run;
        run += c;
      }
      cnt = run;
    }
    inc = wave_inclusive_sum(cnt);
    if (lane == kWave - 1) wsum[w] = inc;
  }
  __syncthreads();
  if (t < F) {
    uint32_t off = 0;
    for (int ww = 0; ww < w; ++ww) off += wsum[ww];
    base_f[t] = off + inc - cnt;
    const int64_t c = ((int64_t)d << sh) + t;
    if (c < n) out_ro[c] = (int32_t)(bs + off + inc - cnt);
  }
  if (d == 0 && t == 0) out_ro[n] = (int32_t)nnz;
  __syncthreads();
  if (s0 >= s1) return;
  // rounds of 64 entries, taken SUB at a time: the records of the next SUB
  // rounds are requested before the current SUB are ranked and written
  constexpr int kSub = SUB;
  auto clampq = [&](int64_t q) { return q < s1 ? q : s0; };
  Rec<RB> cur[kSub];
#pragma unroll
  for (int j = 0; j < kSub; ++j) cur[j] = rec[clampq(s0 + j * kWave + lane)];
  for (int64_t qb = s0; qb < s1; qb += kSub * kWave) {
    Rec<RB> nxt[kSub];
#pragma unroll
    for (int j = 0; j < kSub; ++j) nxt[j] = rec[clampq(qb + (kSub + j) * kWave + lane)];
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const bool valid = qb + j * kWave + lane < s1;
      const uint32_t f = valid ? cur[j].fine(fmask, sh) : 0u;
      const uint64_t peers = digit_peers(valid, f, match[w], lanebit);
      const uint32_t rank = (uint32_t)__popcll(peers & lt);
      const uint32_t before = wcnt[w][f];
      if (valid) {
        const int64_t dst = bs + base_f[f] + before + rank;
        out_col[dst] = (OI)cur[j].row(sh);
        if constexpr (VB == 4) {
          ((uint32_t*)out_val)[dst] = cur[j].bits();
        } else if constexpr (VB == 2) {
          ((uint16_t*)out_val)[dst] = (uint16_t)cur[j].bits();
        }
        if (rank == 0) wcnt[w][f] = before + (uint32_t)__popcll(peers);
      }
    }
#pragma unroll
    for (int j = 0; j < kSub; ++j) cur[j] = nxt[j];
  }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void iota_i32_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = (int32_t)i;
}

// out[j] = in[src[j]], T a 2- or 4-byte word moved as is; src[j] outside
// [0, n_in) gives zero.  Four outputs per thread and round, their loads
// issued together.
template <typename T>
__global__ __launch_bounds__(256) void permute_values_kernel(const T* in, int64_t n_in,
                                                             const int32_t* src, int64_t n,
                                                             T* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t j0 = (int64_t)blockIdx.x * 256 + threadIdx.x; j0 < n; j0 += 4 * stride) {
    int32_t q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = j0 + u * stride;
      q[u] = j < n ? src[j] : -1;
    }
    T v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (q[u] >= 0 && q[u] < n_in) ? in[q[u]] : T(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = j0 + u * stride;
      if (j < n) out[j] = v[u];
    }
  }
}

template <typename OI, int RB>
hipError_t launch_bucket_finish(const void* rec, const uint32_t* bstart, int64_t bstride,
                                int64_t nnz, int64_t n, int sh, int vb, void* out_val,
                                int32_t* out_ro, void* out_col, hipStream_t s) {
  const int64_t nb = cdiv(n, (int64_t)1 << sh);
  const dim3 grid((unsigned)nb);
  const dim3 blk(kFinishThreads);
  const Rec<RB>* r = (const Rec<RB>*)rec;
  // records requested eight rounds ahead when the average wave slice holds
  // more than four rounds (3.1 M entries in 242 buckets: transpose 95.5 ->
  // 92.7 us), else four (168 K entries in 256 buckets, about one round per
  // wave: eight ahead cost 28.3 -> 29.9 us)
  const bool deep = nnz > nb * kFinishWaves * 4 * kWave;
  auto go = [&](auto vbc, auto subc) {
    constexpr int VB = decltype(vbc)::value;
    constexpr int SUB = decltype(subc)::value;
    hipLaunchKernelGGL((transpose_bucket_kernel<OI, VB, RB, SUB>), grid, blk, 0, s, r, bstart,
                       bstride, nnz, n, sh, (uint8_t*)out_val, out_ro, (OI*)out_col);
  };
  auto pick = [&](auto vbc) {
    if (deep) go(vbc, std::integral_constant<int, 8>{});
    else go(vbc, std::integral_constant<int, 4>{});
  };
  if (vb == 4) pick(std::integral_constant<int, 4>{});
  else if (vb == 2) pick(std::integral_constant<int, 2>{});
  else pick(std::integral_constant<int, 0>{});
  return hipGetLastError();
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

// Row order of up to kBlockSortMax rows in one workgroup of 1024 threads.
//
// Usual case, a small spread of row lengths (max - min < 4096): a one-pass
// stable counting sort on k = max - count.  Wave w owns a contiguous run of
// rows; it histograms its rows into column w of a [k][wave] table (LDS,
// 16-bit), the table is scanned in k-major order, and wave w then places its
// rows in order: a row's slot is its (k, w) base plus the number of earlier
// lanes of the step with the same k (wave ballots), so equal keys keep row
// order.  Otherwise: LSD radix sort of 16-bit keys (cols - count) packed above
// 16-bit row ids, two 8-bit passes through LDS, same ballot ranking.
constexpr int kBlockSortThreads = 1024;
constexpr int kBlockSortWaves = kBlockSortThreads / kWave;
constexpr int64_t kBlockSortMax = 16384;
constexpr int kCountSortRange = 4096;
// LDS: the counting table (kCountSortRange x 16 x 2 bytes) or the radix
// buffers (2 x kBlockSortMax + 16 x 256 words); the larger decides.
constexpr int kBlockSortLdsWords = 2 * (int)kBlockSortMax + kBlockSortWaves * kRadix;

__device__ __forceinline__ int row_len(const int32_t* ro, int64_t i, int32_t cols) {
  int64_t c = (int64_t)ro[i + 1] - (int64_t)ro[i];
  return (int)(c < 0 ? 0 : (c > cols ? cols : c));
}

template <typename OI>
__global__ __launch_bounds__(kBlockSortThreads) void sort_rows_block_kernel(const int32_t* ro,
                                                                           int64_t m,
                                                                           int32_t cols,
                                                                           OI* out) {
  __shared__ uint32_t lds[kBlockSortLdsWords];
  __shared__ uint32_t base_d[kRadix];
  __shared__ uint32_t wsum[kBlockSortThreads / kWave];
  __shared__ int red[2][kBlockSortWaves];
  const int t = threadIdx.x, w = t / kWave, l = lane_id();
  const uint64_t lt = lanemask_lt();

  // Wave w owns rows [r0, r1); lane l keeps the lengths of rows r0 + 64j + l
  // in registers, so row_offsets is read once.
  constexpr int RPL = (int)(kBlockSortMax / kBlockSortThreads);  // rows per lane
  const int64_t chunk = cdiv(cdiv(m, kBlockSortWaves), kWave) * kWave;
  const int64_t r0 = (int64_t)w * chunk;
  const int64_t r1 = r0 + chunk < m ? r0 + chunk : m;
  int len[RPL];
  int lo = cols, hi = 0;
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    const int64_t i = r0 + (int64_t)j * kWave + l;
    len[j] = i < r1 ? row_len(ro, i, cols) : -1;
    if (len[j] >= 0) {
      lo = len[j] < lo ? len[j] : lo;
      hi = len[j] > hi ? len[j] : hi;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const int lo2 = __shfl_xor(lo, o, 64), hi2 = __shfl_xor(hi, o, 64);
    lo = lo2 < lo ? lo2 : lo;
    hi = hi2 > hi ? hi2 : hi;
  }
  if (l == 0) {
    red[0][w] = lo;
    red[1][w] = hi;
  }
  __syncthreads();
  lo = red[0][0];
  hi = red[1][0];
  for (int ww = 1; ww < kBlockSortWaves; ++ww) {
    lo = red[0][ww] < lo ? red[0][ww] : lo;
    hi = red[1][ww] > hi ? red[1][ww] : hi;
  }
  const int range = hi - lo + 1;

  if (range <= kCountSortRange) {
    uint16_t* tab = (uint16_t*)lds;  // [k][wave]
    int bits = 0;
    while ((1 << bits) < range) ++bits;
    for (int q = t; q < range * kBlockSortWaves; q += kBlockSortThreads) tab[q] = 0;
    __syncthreads();
    // per-wave histograms (leaders of equal-key lane groups add the group size)
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      if (r0 + (int64_t)j * kWave >= r1) break;
      const bool valid = len[j] >= 0;
      const uint32_t k = valid ? (uint32_t)(hi - len[j]) : 0u;
      uint64_t peers = __ballot(valid);
      for (int x = 0; x < bits; ++x) {
        const bool bit = (k >> x) & 1u;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      if (valid && (peers & lt) == 0)
        tab[k * kBlockSortWaves + w] += (uint16_t)__popcll(peers);
    }
    __syncthreads();
    // exclusive scan of the table in k-major order: wave w owns a contiguous
    // segment and walks it 64 entries at a time (lane l reads entry j*64 + l,
    // so the lanes hit consecutive LDS addresses); the first walk only sums.
    const int total = range * kBlockSortWaves;
    const int seg = (int)cdiv(cdiv(total, kBlockSortWaves), kWave) * kWave;
    const int e0 = w * seg;
    const int e1 = e0 + seg < total ? e0 + seg : total;
    uint32_t s = 0;
    for (int e = e0 + l; e < e1; e += kWave) s += tab[e];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (l == 0) wsum[w] = s;
    __syncthreads();
    uint32_t carry = 0;
    for (int ww = 0; ww < w; ++ww) carry += wsum[ww];
    for (int b = e0; b < e1; b += kWave) {
      const int e = b + l;
      const uint32_t c = e < e1 ? tab[e] : 0u;
      const uint32_t inc = wave_inclusive_sum(c);
      if (e < e1) tab[e] = (uint16_t)(carry + inc - c);
      carry += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
    }
    __syncthreads();
    // placement, in row order inside each wave's run
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      if (r0 + (int64_t)j * kWave >= r1) break;
      const int64_t i = r0 + (int64_t)j * kWave + l;
      const bool valid = len[j] >= 0;
      const uint32_t k = valid ? (uint32_t)(hi - len[j]) : 0u;
      uint64_t peers = __ballot(valid);
      for (int x = 0; x < bits; ++x) {
        const bool bit = (k >> x) & 1u;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      const uint32_t rank = (uint32_t)__popcll(peers & lt);
      uint32_t base = 0;
      if (valid) base = tab[k * kBlockSortWaves + w];
      if (valid) out[base + rank] = (OI)i;
      if (valid && rank == 0) tab[k * kBlockSortWaves + w] = (uint16_t)(base + __popcll(peers));
    }
    return;
  }

  // wide spread: two 8-bit LSD passes on 16-bit keys
  uint32_t* const buf0 = lds;
  uint32_t* const buf1 = lds + kBlockSortMax;
  uint32_t* const cntf = lds + 2 * kBlockSortMax;  // [wave][digit]
  for (int64_t i = t; i < m; i += kBlockSortThreads)
    buf0[i] = ((uint32_t)(cols - row_len(ro, i, cols)) << 16) | (uint32_t)i;
  int cur = 0;
  for (int shift = 16; shift < 32; shift += 8) {
    if (t < kRadix) base_d[t] = 0;
    __syncthreads();
    for (int64_t i = t; i < m; i += kBlockSortThreads)
      atomicAdd(&base_d[((cur ? buf1 : buf0)[i] >> shift) & 0xffu], 1u);
    __syncthreads();
    // exclusive scan of the 256 digit counts by the first four waves
    if (t < kRadix) {
      const uint32_t c = base_d[t];
      const uint32_t inc2 = wave_inclusive_sum(c);
      if (l == kWave - 1) wsum[w] = inc2;
      base_d[t] = inc2 - c;
    }
    __syncthreads();
    if (t < kRadix) {
      uint32_t off = 0;
      for (int ww = 0; ww < w; ++ww) off += wsum[ww];
      base_d[t] += off;
    }
    __syncthreads();
    for (int64_t q0 = 0; q0 < m; q0 += kBlockSortThreads) {
      for (int q = t; q < kBlockSortWaves * kRadix; q += kBlockSortThreads) cntf[q] = 0;
      __syncthreads();
      const int64_t i = q0 + t;
      const bool valid = i < m;
      const uint32_t item = valid ? (cur ? buf1 : buf0)[i] : 0u;
      const uint32_t d = (item >> shift) & 0xffu;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
      }
      const uint32_t rank = (uint32_t)__popcll(peers & lt);
      if (valid && rank == 0) cntf[w * kRadix + d] = (uint32_t)__popcll(peers);
      __syncthreads();
      if (t < kRadix) {
        uint32_t run = base_d[t];
        for (int ww = 0; ww < kBlockSortWaves; ++ww) {
          const uint32_t c = cntf[ww * kRadix + t];
          cntf[ww * kRadix + t] = run;
          run += c;
        }
        base_d[t] = run;
      }
      __syncthreads();
      if (valid) (cur ? buf0 : buf1)[cntf[w * kRadix + d] + rank] = item;
      __syncthreads();
    }
    cur ^= 1;
  }
  for (int64_t i = t; i < m; i += kBlockSortThreads)
    out[i] = (OI)((cur ? buf1 : buf0)[i] & 0xffffu);
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
  if (n <= kSingleMax && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 16 == 0) {
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

hipError_t radix_sort_u32_iota_ptrs(const uint32_t* keys, int64_t n, int bits, void* ws,
                                    const uint32_t** sorted_keys, const uint32_t** sorted_vals,
                                    hipStream_t s) {
  RadixWs R = carve_radix_ws(ws, n);
  int res = 0;
  hipError_t e = n > 0 ? radix_sort_iota(KeyFromU32{keys}, n, bits, R, &res, s) : hipSuccess;
  *sorted_keys = R.keys[res < 0 ? 0 : res];
  *sorted_vals = R.vals[res < 0 ? 0 : res];
  return e;
}

// Stable two-level sort of n entries by key (< nkeys <= 2^17): one radix
// pass on the top 8 key bits, then one workgroup per coarse bucket orders it
// by the remaining <= 9 bits (transpose_bucket_kernel), which writes the
// entries' payloads to out_col (and value bits to out_val) in key order and
// the key boundaries to out_ro[0..nkeys].  Payload: the row of each stored
// position (rows_of, expanded from the row offsets `ro` of `rows` rows by
// the count launch) or, with ro == nullptr, the entry's own index.  Up to
// kSelfMaxTiles tiles the scatter derives its own offsets from the count
// table (three launches); beyond that an exclusive scan of the table runs
// between count and scatter.  Workspace: radix buffers (records), rows_of,
// bucket starts.
template <class KS>
hipError_t two_level_sort(KS ks, int64_t n, int64_t nkeys, const int32_t* ro, int64_t rows,
                          const void* val, int vb, void* out_val, int32_t* out_ro,
                          void* out_col, int out_col_i32, void* ws, hipStream_t s) {
  RadixWs R = carve_radix_ws(ws, n);
  uint32_t* rows_of = (uint32_t*)((char*)ws + radix_ws_bytes_for(n));
  uint32_t* bstart = rows_of + align256((size_t)n * 4) / 4;
  const int bits = nkeys > 1 ? bit_length((uint64_t)(nkeys - 1)) : 1;
  const int sh = bits > kRadixBits ? bits - kRadixBits : 0;
  const int64_t ntiles = cdiv(n, kTile);
  const int64_t erows = ro ? rows : 0;  // rows to expand
  const int64_t pay_max = ro ? rows : n;  // payloads are below this
  // the count launch also expands row offsets, at most kExpandRows rows per
  // workgroup (eight per wave), extra workgroups beyond the tiles only expand
  const int64_t cgrid =
      ntiles > cdiv(erows, kExpandRows) ? ntiles : cdiv(erows, kExpandRows);
  const int64_t rpb = cdiv(erows, cgrid);
  // (the kOptTransposeForceScan switch forces the scan path, for its test)
  const bool self = ntiles <= kSelfMaxTiles && option(kOptTransposeForceScan) == 0;
  // first pass: keys with their payloads and value bits, one record per
  // entry over the key and payload buffers of the workspace (which lie back
  // to back and hold at least 16 bytes per entry): 8 bytes while the
  // payloads fit above the fine digit, else 16
  uint32_t* rec = R.keys[0];
  // (the kOptTransposeWideRecords switch selects 16, for its test)
  const bool rec8 =
      pay_max <= ((int64_t)1 << (32 - sh)) && option(kOptTransposeWideRecords) == 0;
  auto scatter = [&](auto vs, auto rb, auto sf) -> hipError_t {
    using VS = decltype(vs);
    constexpr int RB = decltype(rb)::value;
    constexpr bool SELF = decltype(sf)::value;
    hipLaunchKernelGGL((transpose_count_kernel<KS, SELF>), dim3((unsigned)cgrid), dim3(kThreads),
                       0, s, ks, n, sh, 0xffu, R.counts, ntiles, ro, erows, rpb, rows_of);
    if constexpr (!SELF) {
      hipError_t e =
          exclusive_scan_u32(R.counts, R.counts, ntiles * kRadix, nullptr, R.scan_ws, s);
      if (e != hipSuccess) return e;
    }
    if (vb == 4)
      hipLaunchKernelGGL((radix_scatter_kernel<KS, VS, ValBits<4>, RB, SELF>),
                         dim3((unsigned)ntiles), dim3(kThreads), 0, s, ks, vs, n, sh,
                         kRadixBits, R.counts, ntiles, rec, nullptr, ValBits<4>{val}, bstart);
    else if (vb == 2)
      hipLaunchKernelGGL((radix_scatter_kernel<KS, VS, ValBits<2>, RB, SELF>),
                         dim3((unsigned)ntiles), dim3(kThreads), 0, s, ks, vs, n, sh,
                         kRadixBits, R.counts, ntiles, rec, nullptr, ValBits<2>{val}, bstart);
    else
      hipLaunchKernelGGL((radix_scatter_kernel<KS, VS, ValBits<0>, RB, SELF>),
                         dim3((unsigned)ntiles), dim3(kThreads), 0, s, ks, vs, n, sh,
                         kRadixBits, R.counts, ntiles, rec, nullptr, ValBits<0>{nullptr},
                         bstart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t* bs = SELF ? bstart : R.counts;
    const int64_t bstride = SELF ? 1 : ntiles;
    if (out_col_i32)
      return launch_bucket_finish<int32_t, RB>(rec, bs, bstride, n, nkeys, sh, vb, out_val,
                                               out_ro, out_col, s);
    return launch_bucket_finish<int16_t, RB>(rec, bs, bstride, n, nkeys, sh, vb, out_val,
                                             out_ro, out_col, s);
  };
  auto pick = [&](auto vs) -> hipError_t {
    using R8 = std::integral_constant<int, 8>;
    using R16 = std::integral_constant<int, 16>;
    using Y = std::true_type;
    using N = std::false_type;
    if (self) return rec8 ? scatter(vs, R8{}, Y{}) : scatter(vs, R16{}, Y{});
    return rec8 ? scatter(vs, R8{}, N{}) : scatter(vs, R16{}, N{});
  };
  if (ro) return pick(ValFromU32{rows_of});
  return pick(ValIota{});
}

size_t transpose_workspace_bytes(int64_t rows, int64_t cols, int64_t nnz) {
  (void)rows;
  (void)cols;
  // radix buffers, rows_of, and the coarse bucket starts of the single-pass
  // first stage
  return radix_ws_bytes_for(nnz) + align256((size_t)nnz * 4) + align256(kRadix * 4);
}

// Transpose for up to 2^17 columns: the two-level sort of the stored entries
// by column, payload the entry's row.
hipError_t transpose_two_level(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                               const void* col, int col_i32, const void* val, int vb,
                               void* out_val, int32_t* out_ro, void* out_col, int out_col_i32,
                               void* ws, hipStream_t s) {
  if (col_i32)
    return two_level_sort(KeyFromIndex<int32_t>{(const int32_t*)col, (int32_t)(cols - 1)}, nnz,
                          cols, ro, rows, val, vb, out_val, out_ro, out_col, out_col_i32, ws, s);
  return two_level_sort(KeyFromIndex<int16_t>{(const int16_t*)col, (int32_t)(cols - 1)}, nnz,
                        cols, ro, rows, val, vb, out_val, out_ro, out_col, out_col_i32, ws, s);
}

hipError_t launch_csr_transpose(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                                const void* col, int col_i32, const void* val, int val_bytes,
                                void* out_val, int32_t* out_ro, void* out_col, int out_col_i32,
                                void* ws, hipStream_t s) {
  const int vb0 = val ? val_bytes : 0;
  if (nnz == 0) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)cdiv(cols + 1, 256)), dim3(256), 0, s,
                       out_ro, cols + 1, 0);
    return hipGetLastError();
  }
  if (cols <= ((int64_t)1 << (kRadixBits + 9)))
    return transpose_two_level(rows, cols, nnz, ro, col, col_i32, val, vb0, out_val, out_ro,
                               out_col, out_col_i32, ws, s);
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

hipError_t launch_csr_transpose_perm(int64_t rows, int64_t cols, int64_t nnz, const int32_t* ro,
                                     const void* col, int col_i32, int32_t* out_src,
                                     int32_t* out_ro, void* out_col, int out_col_i32, void* ws,
                                     int32_t* iota, hipStream_t s) {
  if (nnz > 0) {
    hipLaunchKernelGGL(iota_i32_kernel, dim3((unsigned)cdiv(nnz, 256)), dim3(256), 0, s, iota,
                       nnz);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the entry indices are 4-byte words that the transpose moves bit for bit
  return launch_csr_transpose(rows, cols, nnz, ro, col, col_i32, iota, 4, out_src, out_ro,
                              out_col, out_col_i32, ws, s);
}

hipError_t launch_permute_values(const void* in, int64_t n_in, int elem_bytes,
                                 const int32_t* src, int64_t n, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = cdiv(n, 4 * 256);
  const dim3 grid((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20)));
  if (elem_bytes == 4)
    hipLaunchKernelGGL(permute_values_kernel<uint32_t>, grid, dim3(256), 0, s,
                       (const uint32_t*)in, n_in, src, n, (uint32_t*)out);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(permute_values_kernel<uint16_t>, grid, dim3(256), 0, s,
                       (const uint16_t*)in, n_in, src, n, (uint16_t*)out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

size_t sort_rows_workspace_bytes(int64_t rows, int64_t cols) {
  (void)cols;
  return radix_ws_bytes_for(rows);
}

hipError_t launch_sort_rows(const int32_t* ro, int64_t rows, int64_t cols, void* row_idx,
                            int row_idx_i32, void* ws, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows <= kBlockSortMax && cols <= 65535) {
    if (row_idx_i32)
      hipLaunchKernelGGL(sort_rows_block_kernel<int32_t>, dim3(1), dim3(kBlockSortThreads), 0, s,
                         ro, rows, (int32_t)cols, (int32_t*)row_idx);
    else
      hipLaunchKernelGGL(sort_rows_block_kernel<int16_t>, dim3(1), dim3(kBlockSortThreads), 0, s,
                         ro, rows, (int32_t)cols, (int16_t*)row_idx);
    return hipGetLastError();
  }
  // LSD passes over the key cols - count (not the two-level sort: the keys
  // crowd just below cols, which would put every row in one coarse bucket)
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

// sddmm_dense.hip -- structure-aware SDDMM on gfx950 (spops README, section
// "Sampled Dense-Dense Matrix Multiplication (SDDMM)", the kernel for masks
// whose entries cluster in a small subset of rows and columns).
//
// Plan (integer work, once per mask, on the device):
//   * a row is dense when it holds at least tau*n entries;
//   * over the remaining rows, a column is dense when it holds at least
//     tau*(remaining rows) entries;
//   * region A = dense rows x all columns, region B = remaining rows x dense
//     columns; both are cut into TM x TN tiles of gathered rows / columns;
//   * every entry gets a tile key (or a sentinel for "neither"), and a stable
//     radix sort groups the entries tile by tile, keeping the remainder in
//     CSR order; the remainder becomes a sub-CSR for the general kernel.
//
// Execute: one workgroup per non-empty tile computes the dense TM x TN block
// A[rows] * BT[cols]^T with v_mfma_f32_32x32x16_{f16,bf16} (fp32 accumulate),
// staging 64-wide K slices of the gathered rows through two LDS stages, then
// writes only the tile's mask positions from an LDS copy of the block.  Every mask entry
// belongs to exactly one tile or to the remainder, so each output is written
// once.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int TM = 128;       // tile rows
constexpr int TN = 128;       // tile columns
constexpr int TK = 64;        // K slice staged per step
constexpr int LDK = TK + 8;   // padded LDS row (16-bit elements)
constexpr int LDC = TN + 4;   // padded LDS row of the fp32 result block
constexpr int kThreads = 256;
constexpr int kStage = (TM + TN) * LDK;  // 16-bit elements per LDS stage (A, then BT)
constexpr int kChunks = TM * TK / 8 / kThreads;  // 16-byte chunks per thread per operand
static_assert(TM == TN, "A and BT tiles share the staging map");
static_assert(TM * LDC * 4 <= 2 * kStage * 2, "the fp32 block reuses the LDS stages");


typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf168v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

struct TileArgs {
  int64_t K, lda, ldbt, n;
  const uint16_t* A;
  const uint16_t* BT;
  const int32_t* hot_rows;
  const int32_t* cold_rows;
  const int32_t* hot_cols;
  int64_t n_rows_hot, n_rows_cold, n_cols_hot;
  int64_t tiles_a, tiles_a_cols, tiles_b_cols;
  const int32_t* tile_start;
  const int32_t* ent_pos;
  const int32_t* ent_rc;
  void* out;
};

template <bool BF16>
__device__ __forceinline__ float16v mfma32(const uint4& a, const uint4& b, float16v c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf168v, a),
                                                   __builtin_bit_cast(bf168v, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8v, a),
                                                  __builtin_bit_cast(half8v, b), c, 0, 0, 0);
  }
}

// One workgroup (4 waves) per tile; wave (wr, wc) computes the 64 x 64
// quarter (wr, wc) as 2 x 2 MFMA 32x32x16 blocks.  K runs in slices of TK = 64
// through two LDS stages: while the waves multiply out of one stage, the next
// slice's gathered rows are already in registers and are stored into the
// other stage afterwards, so each slice costs one barrier.  After the K loop
// the fp32 block goes to LDS and only the tile's mask positions are written.
template <bool BF16, typename OT>
__global__ __launch_bounds__(kThreads, 2) void sddmm_tile_kernel(TileArgs t) {
  const int64_t tile = blockIdx.x;
  const int32_t e0 = t.tile_start[tile], e1 = t.tile_start[tile + 1];
  if (e1 <= e0) return;  // no mask entry in this tile

  // region and gathered row/column lists
  const int32_t* rlist;
  const int32_t* clist;
  int64_t rcount, ccount, tr, tc;
  if (tile < t.tiles_a) {
    tr = tile / t.tiles_a_cols;
    tc = tile % t.tiles_a_cols;
    rlist = t.hot_rows;
    rcount = t.n_rows_hot;
    clist = nullptr;  // identity over all columns
    ccount = t.n;
  } else {
    const int64_t b = tile - t.tiles_a;
    tr = b / t.tiles_b_cols;
    tc = b % t.tiles_b_cols;
    rlist = t.cold_rows;
    rcount = t.n_rows_cold;
    clist = t.hot_cols;
    ccount = t.n_cols_hot;
  }

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
  float* Cs = (float*)smem;  // [TM][LDC] after the K loop

  const int tid = threadIdx.x;
  // chunk q = tid + 256*h: tile row q / 8, K offset (q % 8) * 8
  const uint16_t* ap[kChunks];
  const uint16_t* bp[kChunks];
  const int skc = (tid & 7) * 8;
#pragma unroll
  for (int h = 0; h < kChunks; ++h) {
    const int row = (tid >> 3) + h * (kThreads / 8);
    const int64_t ri = tr * TM + row;
    const int64_t ci = tc * TN + row;
    ap[h] = ri < rcount ? t.A + (int64_t)rlist[ri] * t.lda : nullptr;
    bp[h] = ci < ccount ? t.BT + (int64_t)(clist ? clist[ci] : ci) * t.ldbt : nullptr;
  }
  uint4 ra[kChunks], rb[kChunks];
  auto fetch = [&](int64_t k0) {
    const int64_t k = k0 + skc;
    const bool ok = k < t.K;  // K is a multiple of 8: a chunk is all in or all out
#pragma unroll
    for (int h = 0; h < kChunks; ++h) {
      ra[h] = (ap[h] && ok) ? *(const uint4*)(ap[h] + k) : make_uint4(0, 0, 0, 0);
      rb[h] = (bp[h] && ok) ? *(const uint4*)(bp[h] + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int stage) {
    uint16_t* As = smem + stage * kStage;
    uint16_t* Bs = As + TM * LDK;
#pragma unroll
    for (int h = 0; h < kChunks; ++h) {
      const int row = (tid >> 3) + h * (kThreads / 8);
      *(uint4*)(As + row * LDK + skc) = ra[h];
      *(uint4*)(Bs + row * LDK + skc) = rb[h];
    }
  };

  const int w = tid / kWave, l = lane_id();
  const int wr = w >> 1, wc = w & 1;
  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int64_t nst = cdiv(t.K, TK);
  fetch(0);
  stash(0);
  __syncthreads();
  for (int64_t st = 0; st < nst; ++st) {
    const int stage = (int)(st & 1);
    if (st + 1 < nst) fetch((st + 1) * TK);
    const uint16_t* As = smem + stage * kStage;
    const uint16_t* Bs = As + TM * LDK;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int kk = ks * 16 + (l >> 5) * 8;
      uint4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *(const uint4*)(As + (wr * 64 + i * 32 + (l & 31)) * LDK + kk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *(const uint4*)(Bs + (wc * 64 + j * 32 + (l & 31)) * LDK + kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<BF16>(fa[i], fb[j], acc[i][j]);
    }
    if (st + 1 < nst) stash(stage ^ 1);
    __syncthreads();
  }
  // 32x32 fp32 result layout: lane l holds column l%32; value v sits at row
  // (v/4)*8 + (l/32)*4 + v%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wr * 64 + i * 32 + (v >> 2) * 8 + (l >> 5) * 4 + (v & 3);
        const int col = wc * 64 + j * 32 + (l & 31);
        Cs[row * LDC + col] = acc[i][j][v];
      }
  __syncthreads();
  OT* out = (OT*)t.out;
  for (int32_t e = e0 + tid; e < e1; e += kThreads) {
    const int32_t rc = t.ent_rc[e];
    out[t.ent_pos[e]] = from_f32<OT>(Cs[(rc >> 16) * LDC + (rc & 0xffff)]);
  }
}

// ----------------------------------------------------------------- plan --

__global__ void row_flags_kernel(const int32_t* ro, int64_t m, int64_t nnz, int64_t thr,
                                 uint32_t* hot) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= m) return;
  int64_t p0 = ro[r], p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > nnz ? nnz : p1);
  const int64_t len = p1 - p0;
  hot[r] = (len > 0 && len >= thr) ? 1u : 0u;
}

__global__ void compact_rows_kernel(const uint32_t* hot, const uint32_t* rank, int64_t m,
                                    int32_t* hot_rows, int32_t* cold_rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= m) return;
  if (hot[r])
    hot_rows[rank[r]] = (int32_t)r;
  else
    cold_rows[r - rank[r]] = (int32_t)r;
}

// 16 lanes per row.
template <typename IT>
__global__ void col_count_kernel(const int32_t* ro, const IT* col, int64_t m, int64_t n,
                                 int64_t nnz, const uint32_t* hot, uint32_t* cnt) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  if (r >= m || hot[r]) return;
  int64_t p0 = ro[r], p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > nnz ? nnz : p1);
  for (int64_t p = p0 + sub; p < p1; p += 16) {
    const int c = (int)col[p];
    if ((unsigned)c < (unsigned)n) atomicAdd(&cnt[c], 1u);
  }
}

__global__ void col_flags_kernel(const uint32_t* cnt, int64_t n, int64_t thr, uint32_t* flag) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  flag[c] = (cnt[c] > 0 && (int64_t)cnt[c] >= thr) ? 1u : 0u;
}

__global__ void compact_cols_kernel(const uint32_t* flag, const uint32_t* rank, int64_t n,
                                    int32_t* hot_cols, int32_t* col_map) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  if (flag[c]) {
    hot_cols[rank[c]] = (int32_t)c;
    col_map[c] = (int32_t)rank[c];
  } else {
    col_map[c] = -1;
  }
}

struct ClassifyArgs {
  const int32_t* ro;
  const void* col;
  int64_t m, n, nnz;
  const uint32_t* hot;       // row flags
  const uint32_t* row_rank;  // exclusive rank among dense rows
  const int32_t* col_map;    // dense-column index or -1
  int64_t tiles_a, tiles_a_cols, tiles_b_cols, tiles;
  int nb;                    // column buckets of the remainder
  uint32_t* key;             // [nnz]
  uint32_t* rc;              // [nnz] in-tile coordinates, or the row (remainder)
  uint32_t* rest_total;      // number of remainder entries (accumulated)
};

// 16 lanes per row: tile key and in-tile coordinates of every entry; an
// entry of neither region gets key tiles + (its column bucket) and keeps its
// row in rc.
template <typename IT>
__global__ void classify_kernel(ClassifyArgs a) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  if (r >= a.m) return;
  const IT* col = (const IT*)a.col;
  int64_t p0 = a.ro[r], p1 = a.ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > a.nnz ? a.nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > a.nnz ? a.nnz : p1);
  const bool hot = a.hot[r] != 0;
  const int64_t hr = a.row_rank[r];        // rank among dense rows
  const int64_t cr = r - hr;               // rank among the other rows
  uint32_t rest = 0;
  for (int64_t p = p0 + sub; p < p1; p += 16) {
    int c = (int)col[p];
    c = (unsigned)c < (unsigned)a.n ? c : 0;
    uint32_t key, rc = 0;
    if (hot) {
      key = (uint32_t)((hr / TM) * a.tiles_a_cols + c / TN);
      rc = ((uint32_t)(hr % TM) << 16) | (uint32_t)(c % TN);
    } else if (a.col_map[c] >= 0) {
      const int64_t hc = a.col_map[c];
      key = (uint32_t)(a.tiles_a + (cr / TM) * a.tiles_b_cols + hc / TN);
      rc = ((uint32_t)(cr % TM) << 16) | (uint32_t)(hc % TN);
    } else {
      key = (uint32_t)(a.tiles + ((int64_t)c * a.nb) / a.n);
      rc = (uint32_t)r;
      ++rest;
    }
    a.key[p] = key;
    a.rc[p] = rc;
  }
  for (int o = 8; o > 0; o >>= 1) rest += __shfl_xor(rest, o, 16);
  if (sub == 0 && rest) atomicAdd(a.rest_total, rest);
}

// All remainder entries into one bucket (keys tiles+b -> tiles).
__global__ void merge_buckets_kernel(uint32_t* key, int64_t nnz, uint32_t tiles) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p < nnz && key[p] > tiles) key[p] = tiles;
}

// Key boundaries (tile_start[t] = first sorted entry with key >= t, for
// t in [0, nkeys]: tiles, then the remainder buckets) and the gathered
// in-tile coordinates / remainder rows.
__global__ void tile_bounds_kernel(const uint32_t* skey, const uint32_t* src, const uint32_t* rc,
                                   int64_t nnz, int64_t nkeys, int32_t* tile_start,
                                   int32_t* ent_pos, int32_t* ent_rc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q > nnz) return;
  const int64_t kprev = q == 0 ? -1 : (int64_t)skey[q - 1];
  const int64_t kcur = q == nnz ? nkeys : (int64_t)skey[q];
  for (int64_t k = kprev + 1; k <= kcur; ++k) tile_start[k] = (int32_t)q;
  if (q == nnz) return;
  const uint32_t p = src[q];
  ent_pos[q] = (int32_t)p;
  ent_rc[q] = (int32_t)rc[p];
}

int bit_length(uint64_t v) {
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

template <typename OT>
hipError_t launch_tiles_typed(const SddmmPlanDev& p, const TileArgs& ta, int dtype,
                              hipStream_t s) {
  if (dtype == kBF16)
    hipLaunchKernelGGL((sddmm_tile_kernel<true, OT>), dim3((unsigned)p.tiles), dim3(kThreads), 0,
                       s, ta);
  else
    hipLaunchKernelGGL((sddmm_tile_kernel<false, OT>), dim3((unsigned)p.tiles), dim3(kThreads),
                       0, s, ta);
  return hipGetLastError();
}

}  // namespace

hipError_t build_sddmm_plan(int64_t m, int64_t n, int64_t nnz, const int32_t* ro,
                            const void* col, int col_i32, double tau, SddmmPlanDev* out,
                            hipStream_t s) {
  *out = SddmmPlanDev{};
  out->m = m;
  out->n = n;
  out->nnz = nnz;
  out->tau = tau;
  out->mask_ro = ro;
  out->mask_col = col;
  const size_t mb = align256((size_t)(m + 1) * 4), nb = align256((size_t)(n + 1) * 4);
  const size_t zb = align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  const size_t sws = scan_workspace_bytes(m > n ? m + 1 : n + 1);
  const size_t rws = radix_pairs_workspace_bytes(nnz);
  char* tmp = nullptr;
  hipError_t e = hipMalloc(&tmp, 3 * mb + 3 * nb + 4 * zb + sws + rws + 256);
  if (e != hipSuccess) return e;
  uint32_t* hot = (uint32_t*)tmp;
  uint32_t* rrank = (uint32_t*)(tmp + mb);
  uint32_t* ccnt = (uint32_t*)(tmp + 3 * mb);
  uint32_t* cflag = (uint32_t*)(tmp + 3 * mb + nb);
  uint32_t* crank = (uint32_t*)(tmp + 3 * mb + 2 * nb);
  uint32_t* key = (uint32_t*)(tmp + 3 * mb + 3 * nb);
  uint32_t* rc = (uint32_t*)(tmp + 3 * mb + 3 * nb + zb);
  uint32_t* skey = (uint32_t*)(tmp + 3 * mb + 3 * nb + 2 * zb);
  uint32_t* src = (uint32_t*)(tmp + 3 * mb + 3 * nb + 3 * zb);
  uint32_t* dtot = (uint32_t*)(tmp + 3 * mb + 3 * nb + 4 * zb);  // 4 counters
  void* scan_ws = tmp + 3 * mb + 3 * nb + 4 * zb + 256;
  void* radix_ws = (char*)scan_ws + sws;
  uint32_t htot[4] = {0, 0, 0, 0};
  const unsigned gm = (unsigned)cdiv(m > 0 ? m : 1, 256), gn = (unsigned)cdiv(n > 0 ? n : 1, 256);
  const unsigned gm16 = (unsigned)cdiv((m > 0 ? m : 1) * 16, 256);
  do {
    const int64_t thr_r = (int64_t)ceil(tau * (double)n);
    if (m > 0) {
      hipLaunchKernelGGL(row_flags_kernel, dim3(gm), dim3(256), 0, s, ro, m, nnz, thr_r, hot);
      if ((e = exclusive_scan_u32(hot, rrank, m, dtot, scan_ws, s)) != hipSuccess) break;
    }
    if ((e = hipMemcpyAsync(htot, dtot, 4, hipMemcpyDeviceToHost, s)) != hipSuccess) break;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
    const int64_t H = m > 0 ? htot[0] : 0;
    const int64_t mc = m - H;
    // column counts over the remaining rows
    if ((e = hipMemsetAsync(ccnt, 0, (size_t)(n + 1) * 4, s)) != hipSuccess) break;
    if (m > 0) {
      if (col_i32)
        hipLaunchKernelGGL(col_count_kernel<int32_t>, dim3(gm16), dim3(256), 0, s, ro,
                           (const int32_t*)col, m, n, nnz, hot, ccnt);
      else
        hipLaunchKernelGGL(col_count_kernel<int16_t>, dim3(gm16), dim3(256), 0, s, ro,
                           (const int16_t*)col, m, n, nnz, hot, ccnt);
    }
    const int64_t thr_c = (int64_t)ceil(tau * (double)mc);
    int64_t Hc = 0;
    if (n > 0) {
      hipLaunchKernelGGL(col_flags_kernel, dim3(gn), dim3(256), 0, s, ccnt, n, thr_c, cflag);
      if ((e = exclusive_scan_u32(cflag, crank, n, dtot + 1, scan_ws, s)) != hipSuccess) break;
      if ((e = hipMemcpyAsync(htot + 1, dtot + 1, 4, hipMemcpyDeviceToHost, s)) != hipSuccess)
        break;
      if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
      Hc = htot[1];
    }
    if (mc == 0) Hc = 0;
    out->n_rows_hot = H;
    out->n_rows_cold = mc;
    out->n_cols_hot = Hc;
    out->tiles_a_cols = cdiv(n, TN);
    out->tiles_a = H > 0 ? cdiv(H, TM) * out->tiles_a_cols : 0;
    out->tiles_b_cols = Hc > 0 ? cdiv(Hc, TN) : 0;
    const int64_t tiles_b = (Hc > 0 && mc > 0) ? cdiv(mc, TM) * out->tiles_b_cols : 0;
    out->tiles = out->tiles_a + tiles_b;
    // remainder column buckets, one per XCD when there are enough columns
    // (revisited below once the remainder is counted)
    out->nb = n >= 1024 ? kMaxBuckets : 1;
    int forced = 0;
    if (const char* env = getenv("SPOPS_SDDMM_BUCKETS")) {
      const int v = atoi(env);
      out->nb = v < 1 ? 1 : (v > kMaxBuckets ? kMaxBuckets : v);
      forced = 1;
    }
    // plan memory
    const size_t b_hot = align256((size_t)(H + 1) * 4), b_cold = align256((size_t)(mc + 1) * 4);
    const size_t b_hc = align256((size_t)(Hc + 1) * 4), b_cm = nb;
    const size_t b_ts = align256((size_t)(out->tiles + kMaxBuckets + 1) * 4);
    char* mem = nullptr;
    if ((e = hipMalloc(&mem, b_hot + b_cold + b_hc + b_cm + b_ts + 2 * zb)) != hipSuccess)
      break;
    out->mem = mem;
    out->hot_rows = (int32_t*)mem;
    out->cold_rows = (int32_t*)(mem + b_hot);
    out->hot_cols = (int32_t*)(mem + b_hot + b_cold);
    int32_t* col_map = (int32_t*)(mem + b_hot + b_cold + b_hc);
    out->tile_start = (int32_t*)(mem + b_hot + b_cold + b_hc + b_cm);
    out->ent_pos = (int32_t*)(mem + b_hot + b_cold + b_hc + b_cm + b_ts);
    out->ent_rc = (int32_t*)(mem + b_hot + b_cold + b_hc + b_cm + b_ts + zb);
    if (m > 0)
      hipLaunchKernelGGL(compact_rows_kernel, dim3(gm), dim3(256), 0, s, hot, rrank, m,
                         out->hot_rows, out->cold_rows);
    if (n > 0) {
      if (mc > 0) {
        hipLaunchKernelGGL(compact_cols_kernel, dim3(gn), dim3(256), 0, s, cflag, crank, n,
                           out->hot_cols, col_map);
      } else {
        if ((e = hipMemsetAsync(col_map, 0xff, (size_t)n * 4, s)) != hipSuccess) break;
      }
    }
    if ((e = hipGetLastError()) != hipSuccess) break;
    if (m > 0) {
      if ((e = hipMemsetAsync(dtot + 2, 0, 4, s)) != hipSuccess) break;
      ClassifyArgs ca{ro,   col,       m,     n,    nnz,      hot, rrank, col_map,
                      out->tiles_a, out->tiles_a_cols, out->tiles_b_cols, out->tiles,
                      out->nb, key,  rc, dtot + 2};
      if (col_i32)
        hipLaunchKernelGGL(classify_kernel<int32_t>, dim3(gm16), dim3(256), 0, s, ca);
      else
        hipLaunchKernelGGL(classify_kernel<int16_t>, dim3(gm16), dim3(256), 0, s, ca);
      if ((e = hipGetLastError()) != hipSuccess) break;
      if ((e = hipMemcpyAsync(htot + 2, dtot + 2, 4, hipMemcpyDeviceToHost, s)) != hipSuccess)
        break;
      if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
      // Buckets pay when each remaining row keeps several entries per bucket
      // (A's row is reloaded once per row and bucket): at least 32 remainder
      // entries per remaining row on average, else one bucket.
      if (!forced && out->nb > 1 && (int64_t)htot[2] < 32 * (mc > 0 ? mc : 1)) {
        out->nb = 1;
        hipLaunchKernelGGL(merge_buckets_kernel, dim3((unsigned)cdiv(nnz, 256)), dim3(256), 0, s,
                           key, nnz, (uint32_t)out->tiles);
        if ((e = hipGetLastError()) != hipSuccess) break;
      }
    }
    const int64_t nkeys = out->tiles + out->nb;
    if (nnz > 0) {
      if ((e = radix_sort_u32_iota(key, nnz, bit_length((uint64_t)(nkeys - 1)), skey, src,
                                   radix_ws, s)) != hipSuccess)
        break;
    }
    hipLaunchKernelGGL(tile_bounds_kernel, dim3((unsigned)cdiv(nnz + 1, 256)), dim3(256), 0, s,
                       skey, src, rc, nnz, nkeys, out->tile_start, out->ent_pos, out->ent_rc);
    if ((e = hipGetLastError()) != hipSuccess) break;
    int32_t bounds[kMaxBuckets + 1] = {};
    if ((e = hipMemcpyAsync(bounds, out->tile_start + out->tiles, (size_t)(out->nb + 1) * 4,
                            hipMemcpyDeviceToHost, s)) != hipSuccess)
      break;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) break;
    const int32_t tiled = bounds[0];
    out->tiled_nnz = tiled;
    out->rest_nnz = nnz - tiled;
    for (int b = 0; b <= out->nb; ++b) out->bucket_start[b] = bounds[b] - tiled;
    out->rest_pos = out->ent_pos + tiled;
    out->rest_row = out->ent_rc + tiled;
  } while (0);
  hipFree(tmp);
  if (e != hipSuccess) free_sddmm_plan(out);
  return e;
}

void free_sddmm_plan(SddmmPlanDev* p) {
  if (p->mem) hipFree(p->mem);
  *p = SddmmPlanDev{};
}

hipError_t launch_sddmm_tiles(const SddmmPlanDev& p, int64_t K, const void* A, int64_t lda,
                              const void* BT, int64_t ldbt, int dtype, void* out, int out_dtype,
                              hipStream_t s) {
  if (p.tiles == 0 || p.tiled_nnz == 0) return hipSuccess;
  TileArgs ta{K,          lda,          ldbt,          p.n,           (const uint16_t*)A,
              (const uint16_t*)BT,      p.hot_rows,    p.cold_rows,   p.hot_cols,
              p.n_rows_hot, p.n_rows_cold, p.n_cols_hot, p.tiles_a,    p.tiles_a_cols,
              p.tiles_b_cols, p.tile_start, p.ent_pos,  p.ent_rc,      out};
  if (out_dtype == kF32) return launch_tiles_typed<float>(p, ta, dtype, s);
  if (dtype == kBF16) return launch_tiles_typed<bf16_t>(p, ta, dtype, s);
  return launch_tiles_typed<_Float16>(p, ta, dtype, s);
}

}  // namespace spops

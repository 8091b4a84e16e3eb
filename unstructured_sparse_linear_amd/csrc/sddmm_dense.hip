// sddmm_dense.hip -- structure-aware SDDMM on gfx950 (spops README, section
// "Sampled Dense-Dense Matrix Multiplication (SDDMM)", the kernel for masks
// whose entries cluster in a small subset of rows and columns).
//
// Plan (integer work, once per mask, entirely on the device: no host
// round trip, so it can also be built inside an execute call from the
// caller's workspace):
//   * a row is dense when it holds at least tau*n entries;
//   * over the remaining rows, a column is dense when it holds at least
//     tau*(remaining rows) entries;
//   * region A = dense rows x all columns, region B = remaining rows x dense
//     columns; both are cut into TM x TN tiles of gathered rows / columns;
//   * every entry gets a key: its tile for a tile entry, rest_key +
//     (column bucket) for the remainder; a stable
//     radix sort groups the entries by key (the remainder of each bucket
//     stays in CSR order), and key_start[k] is the first sorted entry with
//     key >= k.  Counts (dense rows, tiles, ...) stay in device memory; the
//     key space is sized by bounds the host knows from (m, n, nnz).
//
// Execute: a workgroup (8 waves) takes one (tile, K split) item and computes
// the dense TM x TN block A[rows] * BT[cols]^T over its share of K with
// v_mfma_f32_32x32x16_{f16,bf16} (fp32 accumulate), then writes the tile's
// mask positions from an LDS copy of the block.
// The (tile, K slice) units are spread evenly over the compute units; a
// tile computed in one piece writes the output, a tile cut into several
// pieces writes fp32 partial sums and a second kernel adds them in order
// (deterministic).  Every mask entry belongs to exactly
// one tile or to the remainder, so each output is written once.
#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int TM = kSddmmTM;           // tile rows
constexpr int TN = kSddmmTN;           // tile columns
constexpr int TK = 64;                 // K slice staged per step
constexpr int LDK = TK + 8;            // padded LDS row (16-bit elements)
constexpr int kThreads = 512;          // 8 waves, 2 x 4 over the tile
constexpr int kTileWgPerCu = 2;        // workgroups resident per compute unit
constexpr int kTileWavesPerSimd = kTileWgPerCu * kThreads / kWave / 4;  // launch bound
constexpr int WM = TM / 2, WN = TN / 4;  // wave tile
constexpr int BM = WM / 32, BN = WN / 32;  // 32 x 32 MFMA blocks per wave
constexpr int kStaged = TM + TN;       // rows staged per slice (A rows, then BT rows)
constexpr int kChunks = kStaged * (TK / 8) / kThreads;  // 16-byte chunks per thread and slice
constexpr int kChunksA = TM * (TK / 8) / kThreads;      // the first ones are A rows
constexpr int kStage = kStaged * LDK;  // 16-bit elements per LDS stage
constexpr int LDR = TM + 4;            // padded fp32 column of the block in LDS
constexpr int kEpi = 8;                // entries per thread per round of the split sum
constexpr int kTileEpi = 2;            // entries per thread per epilogue round
static_assert(kChunks * kThreads * 8 == kStaged * TK, "chunks cover the staged slice");
static_assert(TN * LDR * 4 <= 2 * kStage * 2, "the fp32 block reuses the LDS stages");
static_assert(LDR % 4 == 0, "16-byte column segments");
static_assert(TM < 65536 && TN < 65536, "tile coordinates pack into 16 bits");

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf168v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

struct TileArgs {
  int64_t K, lda, ldbt, n;
  const uint16_t* A;
  const uint16_t* BT;
  uint32_t a_bytes, bt_bytes;  // extents of A and BT (each below 2 GiB)
  const int32_t* rows;       // dense rows, then the other rows
  const int32_t* hot_cols;
  const SddmmPlanScalars* sc;
  int64_t tiles_a_cols;
  const int32_t* key_start;
  const int32_t* ent_pos;
  const int32_t* ent_rc;
  int splits;                // K splits per tile; item i = (tile i / splits, split i % splits)
  float* part;               // [splits][tiled] partial sums when splits > 1
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

// A workgroup computes items: the K slices [s0, s0 + nst) of one tile (the
// whole tile, or one of its `splits` fixed splits).
// Eight waves in a 2 x 4 grid: wave (wr, wc) owns the WM x WN block (wr, wc)
// of the tile as BM x BN MFMA 32x32x16 blocks (fp32 accumulators), two
// waves per SIMD per workgroup and two workgroups per compute unit.  K runs
// in slices of TK through two LDS stages; each thread gathers its 16-byte
// chunks of the next slice into registers while the current slice is
// multiplied, so a load has one slice of MFMA work to land, and each slice
// costs one barrier.  A segment that covers its whole tile writes the
// output; segment j of a tile split into several writes partial sums to
// part[j].  The epilogue's entry metadata (in-tile coordinates, positions)
// for the first kTileEpi entries per thread is requested before the K loop
// so that its latency hides behind the MFMA work.
//
// MFMA 32x32x16 operand layout: lane l supplies row (l mod 32) of the A
// block and column (l mod 32) of the B block, K elements 8*(l/32)..+8; it
// receives column (l mod 32) of the result, value v at row
// 8*(v/4) + 4*(l/32) + (v mod 4).
template <bool BF16, typename OT>
__global__ __launch_bounds__(kThreads, kTileWavesPerSimd) void sddmm_tile_kernel(TileArgs t) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStage];
  const int tid = threadIdx.x;
  const int w = tid / kWave, l = lane_id();
  const int wr = w >> 2, wc = w & 3;
  const int64_t H = t.sc->H, mc = t.sc->mc, Hc = t.sc->Hc;
  const int64_t tiles_a = t.sc->tiles_a, tiles_b_cols = t.sc->tiles_b_cols;
  const int64_t tiled = t.sc->tiled;
  const int64_t tiles = t.sc->tiles;
  const int64_t nsl = cdiv(t.K, TK);
  const int64_t per = cdiv(nsl, t.splits);
  const int kc = (tid & 7) * 8;  // K offset of this thread's chunks in a slice
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(t.A, t.a_bytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(t.BT, t.bt_bytes);
  // XCD-aware order: workgroup b runs on XCD b mod 8, so with a grid that is
  // a multiple of 8 the logical index (b mod 8) * (grid / 8) + b / 8 gives
  // each XCD a run of consecutive items; items are ordered so that tiles
  // sharing gathered rows are neighbours (region A column-major over its
  // tile rows, which share BT's columns; region B row-major, whose tiles of
  // one row share A's rows), so those rows are fetched once per L2.
  const int64_t nb8 = gridDim.x / 8;
  const int64_t lb = (gridDim.x % 8 == 0) ? (blockIdx.x % 8) * nb8 + blockIdx.x / 8 : blockIdx.x;
  const int64_t ra = tiles_a > 0 ? tiles_a / t.tiles_a_cols : 0;  // tile rows of region A
  for (int64_t item = lb; item < tiles * t.splits; item += gridDim.x) {
    const int64_t ord = item / t.splits;
    const int64_t tile = ord < tiles_a ? (ord % ra) * t.tiles_a_cols + ord / ra : ord;
    const int seg = (int)(item % t.splits);
    const int64_t s0 = (int64_t)seg * per;
    const int64_t nst = s0 < nsl ? (s0 + per < nsl ? per : nsl - s0) : 0;
    const bool direct = t.splits == 1;
    // gathered rows (region A: dense rows x all columns; region B: other
    // rows x dense columns), requested before the tile's entry range is
    // known so that the two loads overlap
    int64_t tr, tcol, rcount, ccount;
    const int32_t* rlist;
    const int32_t* clist;
    if (tile < tiles_a) {
      tr = tile / t.tiles_a_cols;
      tcol = tile % t.tiles_a_cols;
      rlist = t.rows;
      rcount = H;
      clist = nullptr;  // identity over all columns
      ccount = t.n;
    } else {
      const int64_t b = tile - tiles_a;
      tr = b / tiles_b_cols;
      tcol = b % tiles_b_cols;
      rlist = t.rows + H;
      rcount = mc;
      clist = t.hot_cols;
      ccount = Hc;
    }
    // chunk h covers staged row (tid / 8) + (kThreads / 8) h: A rows first,
    // then BT rows; roff = byte offset of its row, or kOob for padding rows
    // (their buffer loads return zeros without a memory access)
    uint32_t roff[kChunks];
#pragma unroll
    for (int h = 0; h < kChunks; ++h) {
      const int row = (tid >> 3) + h * (kThreads / 8);
      if (h < kChunksA) {
        const int64_t i = tr * TM + row;
        roff[h] = i < rcount ? (uint32_t)rlist[i] * (uint32_t)(t.lda * 2) : kOob;
      } else {
        const int64_t j = tcol * TN + (row - TM);
        roff[h] = j < ccount ? (uint32_t)(clist ? clist[j] : (int32_t)j) * (uint32_t)(t.ldbt * 2)
                             : kOob;
      }
    }
    const int32_t e0 = t.key_start[tile], e1 = t.key_start[tile + 1];
    if (e1 <= e0) continue;  // no mask entry in this tile

    // in-tile coordinates and output positions of the first epilogue round,
    // requested now so that they arrive during the K loop
    int32_t pre_rc[kTileEpi], pre_pos[kTileEpi];
#pragma unroll
    for (int u = 0; u < kTileEpi; ++u) {
      const int32_t q = e0 + tid + u * kThreads;
      pre_rc[u] = q < e1 ? t.ent_rc[q] : 0;
      pre_pos[u] = (q < e1 && direct) ? t.ent_pos[q] : 0;
    }

    // always issued (a slice past the segment loads from kOob: zeros, no
    // memory access), so the compiler can count the loads in flight and wait
    // only for the older buffer
    auto fetch = [&](uint4 (&rb)[kChunks], int64_t slice, bool live) {
      const int64_t k = slice * TK + kc;
      const bool ok = live && k < t.K;  // K is a multiple of 8: a chunk is all in or out
      const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
      for (int h = 0; h < kChunks; ++h) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(h < kChunksA ? rsA : rsB,
                                                             ok ? roff[h] + kb : kOob, 0, 0);
        rb[h] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    };
    auto stash = [&](int stage, const uint4 (&rb)[kChunks]) {
      uint16_t* S = smem + stage * kStage;
#pragma unroll
      for (int h = 0; h < kChunks; ++h) {
        const int row = (tid >> 3) + h * (kThreads / 8);
        *(uint4*)(S + row * LDK + kc) = rb[h];
      }
    };

    float16v acc[BM][BN];
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
      for (int j = 0; j < BN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    auto compute = [&](int stage) {
      const uint16_t* As = smem + stage * kStage;
      const uint16_t* Bs = As + TM * LDK;
#pragma unroll
      for (int ks = 0; ks < TK / 16; ++ks) {
        const int kk = ks * 16 + (l >> 5) * 8;
        uint4 fa[BM], fb[BN];
#pragma unroll
        for (int i = 0; i < BM; ++i)
          fa[i] = *(const uint4*)(As + (wr * WM + i * 32 + (l & 31)) * LDK + kk);
#pragma unroll
        for (int j = 0; j < BN; ++j)
          fb[j] = *(const uint4*)(Bs + (wc * WN + j * 32 + (l & 31)) * LDK + kk);
#pragma unroll
        for (int i = 0; i < BM; ++i)
#pragma unroll
          for (int j = 0; j < BN; ++j) acc[i][j] = mfma32<BF16>(fa[i], fb[j], acc[i][j]);
      }
    };

    // slices [s0, s0 + nst) of K: slice st is computed from LDS stage st & 1
    // while slice st + 1 is in flight into the register buffer
    uint4 rb[kChunks];
    fetch(rb, s0, nst > 0);
    stash(0, rb);
    fetch(rb, s0 + 1, nst > 1);
    __syncthreads();
    for (int64_t st = 0; st < nst; ++st) {
      compute((int)(st & 1));
      if (st + 1 < nst) stash((int)((st + 1) & 1), rb);
      __syncthreads();
      fetch(rb, s0 + st + 2, st + 2 < nst);
    }

    // epilogue: the whole fp32 block goes to LDS (column-major, in the
    // stages' space), then every thread writes entries of the tile, kTileEpi per
    // round with all their loads issued together
    float* Cs = (float*)smem;
    auto write_round = [&](const int32_t (&rc)[kTileEpi], const int32_t (&pos)[kTileEpi], int32_t e) {
#pragma unroll
      for (int u = 0; u < kTileEpi; ++u) {
        const int32_t q = e + u * kThreads;
        if (q < e1) {
          const float v = Cs[(rc[u] & 0xffff) * LDR + (rc[u] >> 16)];
          if (direct)
            ((OT*)t.out)[pos[u]] = from_f32<OT>(v);
          else
            t.part[(int64_t)seg * tiled + q] = v;
        }
      }
    };
    {
      // a lane's values v = 4q..4q+3 are 4 consecutive rows of one column:
      // one 16-byte store each, all at immediate offsets from one address
      float* cb = Cs + (wc * WN + (l & 31)) * LDR + wr * WM + (l >> 5) * 4;
#pragma unroll
      for (int i = 0; i < BM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(float4*)(cb + j * 32 * LDR + i * 32 + q * 8) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
    }
    __syncthreads();
    write_round(pre_rc, pre_pos, e0 + tid);
    for (int32_t e = e0 + tid + kTileEpi * kThreads; e < e1; e += kTileEpi * kThreads) {
      int32_t rc[kTileEpi], pos[kTileEpi];
#pragma unroll
      for (int u = 0; u < kTileEpi; ++u) {
        const int32_t q = e + u * kThreads;
        rc[u] = q < e1 ? t.ent_rc[q] : 0;
        pos[u] = (q < e1 && direct) ? t.ent_pos[q] : 0;
      }
      write_round(rc, pos, e);
    }
    __syncthreads();
  }
}

// Tiles computed in several splits: out[ent_pos[e]] = sum over the tile's
// splits j (in order) of part[j][e].  Workgroup (x, y) takes tile
// x's entries [y * kSumChunk, (y + 1) * kSumChunk), kEpi per thread with all
// loads of a round issued together.
constexpr int kSumChunk = kEpi * 256;
template <typename OT>
__global__ __launch_bounds__(256) void sddmm_split_sum_kernel(TileArgs t) {
  const int64_t tile = blockIdx.x;
  if (tile >= t.sc->tiles) return;
  const int nseg = t.splits;
  if (nseg <= 1) return;
  const int64_t tiled = t.sc->tiled;
  const int32_t e1 = t.key_start[tile + 1];
  for (int32_t e = t.key_start[tile] + (int32_t)(blockIdx.y * kSumChunk + threadIdx.x);
       e < e1; e += (int32_t)(gridDim.y * kSumChunk)) {
    float v[kEpi];
    int32_t pos[kEpi];
#pragma unroll
    for (int u = 0; u < kEpi; ++u) {
      const int32_t q = e + u * 256;
      v[u] = q < e1 ? t.part[q] : 0.f;
      pos[u] = q < e1 ? t.ent_pos[q] : 0;
    }
    for (int j = 1; j < nseg; ++j) {
#pragma unroll
      for (int u = 0; u < kEpi; ++u) {
        const int32_t q = e + u * 256;
        if (q < e1) v[u] += t.part[(int64_t)j * tiled + q];
      }
    }
#pragma unroll
    for (int u = 0; u < kEpi; ++u)
      if (e + u * 256 < e1) ((OT*)t.out)[pos[u]] = from_f32<OT>(v[u]);
  }
}

// ----------------------------------------------------------------- plan --

__global__ void plan_init_kernel(SddmmPlanScalars* sc) {
  if (threadIdx.x == 0) *sc = SddmmPlanScalars{};
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// Row offsets clamped into [0, nnz] and nondecreasing within a row.
__device__ __forceinline__ void clamped_row(const int32_t* ro, int64_t r, int64_t nnz,
                                            int64_t& p0, int64_t& p1) {
  p0 = ro[r];
  p1 = ro[r + 1];
  p0 = p0 < 0 ? 0 : (p0 > nnz ? nnz : p0);
  p1 = p1 < p0 ? p0 : (p1 > nnz ? nnz : p1);
}

__global__ void row_flags_kernel(const int32_t* ro, int64_t m, int64_t nnz, int64_t thr,
                                 uint32_t* hot) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= m) return;
  int64_t p0, p1;
  clamped_row(ro, r, nnz, p0, p1);
  const int64_t len = p1 - p0;
  hot[r] = (len > 0 && len >= thr) ? 1u : 0u;
}

// 16 lanes per row: column counts over the rows that are not dense.
template <typename IT>
__global__ void col_count_kernel(const int32_t* ro, const IT* col, int64_t m, int64_t n,
                                 int64_t nnz, const uint32_t* hot, uint32_t* cnt) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  if (r >= m || hot[r]) return;
  int64_t p0, p1;
  clamped_row(ro, r, nnz, p0, p1);
  for (int64_t p = p0 + sub; p < p1; p += 16) {
    const int c = (int)col[p];
    if ((unsigned)c < (unsigned)n) atomicAdd(&cnt[c], 1u);
  }
}

// A column is dense when, over the mc = m - H other rows, it holds at least
// max(ceil(tau * mc), min_count) entries (and at least one).
__global__ void col_flags_kernel(const uint32_t* cnt, int64_t n, int64_t m, double tau,
                                 int64_t min_count, const SddmmPlanScalars* sc,
                                 uint32_t* flag) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  const int64_t mc = m - sc->H;
  int64_t thr = (int64_t)ceil(tau * (double)mc);
  if (thr < min_count) thr = min_count;
  flag[c] = (mc > 0 && cnt[c] > 0 && (int64_t)cnt[c] >= thr) ? 1u : 0u;
}

// rows[0, H) = dense rows ascending, rows[H, m) = the others ascending.
__global__ void compact_rows_kernel(const uint32_t* hot, const uint32_t* rank, int64_t m,
                                    const SddmmPlanScalars* sc, int32_t* rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= m) return;
  if (hot[r])
    rows[rank[r]] = (int32_t)r;
  else
    rows[sc->H + (r - rank[r])] = (int32_t)r;
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

// Tile counts from the dense row and column counts.
__global__ void derive_tiles_kernel(int64_t m, int64_t tiles_a_cols, SddmmPlanScalars* sc) {
  if (threadIdx.x != 0) return;
  const int64_t H = sc->H;
  const int64_t mc = m - H;
  const int64_t Hc = mc > 0 ? sc->Hc : 0;
  const int64_t tiles_a = H > 0 ? cdiv(H, TM) * tiles_a_cols : 0;
  const int64_t tbc = Hc > 0 ? cdiv(Hc, TN) : 0;
  sc->mc = (int32_t)mc;
  sc->Hc = (int32_t)Hc;
  sc->tiles_a = (int32_t)tiles_a;
  sc->tiles_b_cols = (int32_t)tbc;
  sc->tiles = (int32_t)(tiles_a + (tbc > 0 ? cdiv(mc, TM) * tbc : 0));
  sc->rest_count = 0;
}

struct ClassifyArgs {
  const int32_t* ro;
  const void* col;
  int64_t m, n, nnz;
  const uint32_t* hot;       // row flags
  const uint32_t* row_rank;  // exclusive rank among dense rows
  const int32_t* col_map;    // dense-column index or -1
  SddmmPlanScalars* sc;
  int64_t tiles_a_cols;
  int64_t rest_key;
  int nb;                    // column buckets of the remainder
  uint32_t* key;             // [nnz]
  uint32_t* rc;              // [nnz] in-tile coordinates, or the row (remainder)
};

// 16 lanes per row: the key and in-tile coordinates of every entry; an entry
// of neither region gets rest_key + (its column bucket) and keeps its row in
// rc.
template <typename IT>
__global__ void classify_kernel(ClassifyArgs a) {
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  if (r >= a.m) return;
  const IT* col = (const IT*)a.col;
  int64_t p0, p1;
  clamped_row(a.ro, r, a.nnz, p0, p1);
  const bool hot = a.hot[r] != 0;
  const int64_t hr = a.row_rank[r];  // rank among dense rows
  const int64_t cr = r - hr;         // rank among the other rows
  const int64_t tiles_a = a.sc->tiles_a, tbc = a.sc->tiles_b_cols;
  uint32_t rest = 0;
  for (int64_t p = p0 + sub; p < p1; p += 16) {
    int c = (int)col[p];
    c = (unsigned)c < (unsigned)a.n ? c : 0;
    uint32_t key, rc;
    if (hot) {
      const int64_t tile = (hr / TM) * a.tiles_a_cols + c / TN;
      key = (uint32_t)tile;
      rc = ((uint32_t)(hr % TM) << 16) | (uint32_t)(c % TN);
    } else if (a.col_map[c] >= 0) {
      const int64_t hc = a.col_map[c];
      const int64_t tile = tiles_a + (cr / TM) * tbc + hc / TN;
      key = (uint32_t)tile;
      rc = ((uint32_t)(cr % TM) << 16) | (uint32_t)(hc % TN);
    } else {
      key = (uint32_t)(a.rest_key + ((int64_t)c * a.nb) / a.n);
      rc = (uint32_t)r;
      ++rest;
    }
    a.key[p] = key;
    a.rc[p] = rc;
  }
  for (int o = 8; o > 0; o >>= 1) rest += __shfl_xor(rest, o, 16);
  if (sub == 0 && rest) atomicAdd(&a.sc->rest_count, rest);
}

// Buckets pay while each remaining row keeps several remainder entries per
// bucket (a row's A slice is reloaded once per row and bucket): the most
// buckets (a power of two up to nb_max) with at least 4 remainder entries
// per remaining row and bucket on average; adjacent buckets are merged into
// one (contiguous column ranges).  Thread 0 records the bucket count.
__global__ void merge_buckets_kernel(uint32_t* key, int64_t nnz, uint32_t rest_key, int nb_max,
                                     int forced, SddmmPlanScalars* sc) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t mc = sc->mc > 0 ? sc->mc : 1;
  int nb = nb_max;
  if (!forced)
    while (nb > 1 && (int64_t)sc->rest_count < 4 * (int64_t)nb * mc) nb /= 2;
  if (p == 0) sc->nb = nb;
  if (nb < nb_max && p < nnz && key[p] >= rest_key)
    key[p] = rest_key + (key[p] - rest_key) * (uint32_t)nb / (uint32_t)nb_max;
}

// Thread q < nnz: the sort key of sorted entry q for the remainder's row
// order (its row; m for a tile entry, which sorts them behind).
__global__ void rest_row_key_kernel(const int32_t* ent_rc, int64_t nnz, int64_t m,
                                    const SddmmPlanScalars* sc, uint32_t* key) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nnz) return;
  const int64_t r = ent_rc[q];
  key[q] = (uint32_t)((q >= sc->tiled && r >= 0 && r < m) ? r : m);
}

// The remainder in row order: entry i is sorted entry src[i].
__global__ void rest_gather_kernel(const uint32_t* src, int64_t nnz, const int32_t* ent_pos,
                                   const int32_t* ent_rc, const int32_t* ent_col, int32_t* pos,
                                   int32_t* rc, int32_t* col) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nnz) return;
  const uint32_t q = src[i];
  pos[i] = ent_pos[q];
  rc[i] = ent_rc[q];
  col[i] = ent_col[q];
}

// Thread t < nkeys + 1: key_start[t] = first sorted entry with key >= t (a
// binary search over the sorted keys).  Thread t < nnz: the gathered
// position, in-tile coordinates / row and column of sorted entry t.
template <typename IT>
__global__ void key_bounds_kernel(const uint32_t* skey, const uint32_t* src, const uint32_t* rc,
                                  const IT* col, int64_t nnz, int64_t nkeys,
                                  int32_t* key_start, int32_t* ent_pos, int32_t* ent_rc,
                                  int32_t* ent_col) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t <= nkeys) {
    int64_t lo = 0, hi = nnz;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if ((int64_t)skey[mid] < t) lo = mid + 1;
      else hi = mid;
    }
    key_start[t] = (int32_t)lo;
  }
  if (t < nnz) {
    const uint32_t p = src[t];
    ent_pos[t] = (int32_t)p;
    ent_rc[t] = (int32_t)rc[p];
    ent_col[t] = (int32_t)col[p];
  }
}

__global__ void plan_finish_kernel(const int32_t* key_start, int64_t nnz,
                                   SddmmPlanScalars* sc) {
  if (threadIdx.x != 0) return;
  const int32_t tiled = key_start[sc->tiles];
  sc->tiled = tiled;
  sc->rest = (int32_t)(nnz - tiled);
}

int bit_length(uint64_t v) {
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

int64_t max_tiles_for(int64_t m, int64_t n) { return (cdiv(m, TM) + 1) * cdiv(n, TN); }

int planned_buckets(int64_t n, int* forced) {
  const int64_t opt = option(kOptSddmmBuckets);
  *forced = opt > 0;
  if (opt > 0) return (int)(opt > kMaxBuckets ? kMaxBuckets : opt);
  return n >= 1024 ? kMaxBuckets : 1;
}

struct PlanLayout {
  size_t sc, rows, hot_cols, key_start, ent_pos, ent_rc, ent_col, row_pos, row_rc, row_col,
      total;
};
PlanLayout plan_layout(int64_t m, int64_t n, int64_t nnz) {
  PlanLayout L{};
  const int64_t nkeys = max_tiles_for(m, n) + kMaxBuckets;
  size_t o = 0;
  L.sc = o;
  o += align256(sizeof(SddmmPlanScalars));
  L.rows = o;
  o += align256((size_t)(m > 0 ? m : 1) * 4);
  L.hot_cols = o;
  o += align256((size_t)(n > 0 ? n : 1) * 4);
  L.key_start = o;
  o += align256((size_t)(nkeys + 1) * 4);
  L.ent_pos = o;
  o += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  L.ent_rc = o;
  o += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  L.ent_col = o;
  o += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  L.row_pos = o;
  o += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  L.row_rc = o;
  o += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  L.row_col = o;
  o += align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  L.total = o;
  return L;
}

struct ScratchLayout {
  size_t hot, rrank, ccnt, cflag, crank, col_map, key, rc, scan, radix, total;
};
ScratchLayout scratch_layout(int64_t m, int64_t n, int64_t nnz) {
  ScratchLayout L{};
  const size_t mb = align256((size_t)(m > 0 ? m : 1) * 4);
  const size_t nb = align256((size_t)(n > 0 ? n : 1) * 4);
  const size_t zb = align256((size_t)(nnz > 0 ? nnz : 1) * 4);
  size_t o = 0;
  L.hot = o;
  o += mb;
  L.rrank = o;
  o += mb;
  L.ccnt = o;
  o += nb;
  L.cflag = o;
  o += nb;
  L.crank = o;
  o += nb;
  L.col_map = o;
  o += nb;
  L.key = o;
  o += zb;
  L.rc = o;
  o += zb;
  L.scan = o;
  o += align256(scan_workspace_bytes(m > n ? m : n));
  L.radix = o;
  o += align256(radix_pairs_workspace_bytes(nnz > 0 ? nnz : 1));
  L.total = o;
  return L;
}

template <typename OT>
hipError_t launch_tiles_typed(const TileArgs& ta, unsigned grid, int dtype, hipStream_t s) {
  if (dtype == kBF16)
    hipLaunchKernelGGL((sddmm_tile_kernel<true, OT>), dim3(grid), dim3(kThreads), 0, s, ta);
  else
    hipLaunchKernelGGL((sddmm_tile_kernel<false, OT>), dim3(grid), dim3(kThreads), 0, s, ta);
  return hipGetLastError();
}

template <typename OT>
hipError_t launch_split_sum(const TileArgs& ta, int64_t tiles, int64_t most, hipStream_t s) {
  const int64_t chunks = cdiv(most > 0 ? most : 1, kSumChunk);
  hipLaunchKernelGGL(sddmm_split_sum_kernel<OT>, dim3((unsigned)tiles, (unsigned)chunks),
                     dim3(256), 0, s, ta);
  return hipGetLastError();
}

}  // namespace

size_t sddmm_plan_bytes(int64_t m, int64_t n, int64_t nnz) {
  return plan_layout(m, n, nnz).total;
}

size_t sddmm_plan_scratch_bytes(int64_t m, int64_t n, int64_t nnz) {
  return scratch_layout(m, n, nnz).total;
}

hipError_t enqueue_sddmm_plan(int64_t m, int64_t n, int64_t nnz, const int32_t* ro,
                              const void* col, int col_i32, double tau, int64_t min_count,
                              void* mem, void* scratch, SddmmPlanDev* out, hipStream_t s) {
  *out = SddmmPlanDev{};
  out->m = m;
  out->n = n;
  out->nnz = nnz;
  out->tau = tau;
  out->mask_ro = ro;
  out->mask_col = col;
  out->tiles_a_cols = cdiv(n, TN);
  out->max_tiles = max_tiles_for(m, n);
  out->rest_key = out->max_tiles;
  int forced = 0;
  out->nb_max = planned_buckets(n, &forced);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0)
    out->cus = cus;
  const PlanLayout P = plan_layout(m, n, nnz);
  const ScratchLayout W = scratch_layout(m, n, nnz);
  char* pm = (char*)mem;
  char* ws = (char*)scratch;
  SddmmPlanScalars* sc = (SddmmPlanScalars*)(pm + P.sc);
  out->sc = sc;
  out->rows = (int32_t*)(pm + P.rows);
  out->hot_cols = (int32_t*)(pm + P.hot_cols);
  out->key_start = (int32_t*)(pm + P.key_start);
  out->ent_pos = (int32_t*)(pm + P.ent_pos);
  out->ent_rc = (int32_t*)(pm + P.ent_rc);
  out->ent_col = (int32_t*)(pm + P.ent_col);
  out->row_pos = (int32_t*)(pm + P.row_pos);
  out->row_rc = (int32_t*)(pm + P.row_rc);
  out->row_col = (int32_t*)(pm + P.row_col);
  uint32_t* hot = (uint32_t*)(ws + W.hot);
  uint32_t* rrank = (uint32_t*)(ws + W.rrank);
  uint32_t* ccnt = (uint32_t*)(ws + W.ccnt);
  uint32_t* cflag = (uint32_t*)(ws + W.cflag);
  uint32_t* crank = (uint32_t*)(ws + W.crank);
  int32_t* col_map = (int32_t*)(ws + W.col_map);
  uint32_t* key = (uint32_t*)(ws + W.key);
  uint32_t* rc = (uint32_t*)(ws + W.rc);
  void* scan_ws = ws + W.scan;
  void* radix_ws = ws + W.radix;

  const unsigned gm = (unsigned)cdiv(m > 0 ? m : 1, 256), gn = (unsigned)cdiv(n > 0 ? n : 1, 256);
  const unsigned gm16 = (unsigned)cdiv((m > 0 ? m : 1) * 16, 256);
  const int64_t nkeys = out->rest_key + out->nb_max;
  hipError_t e;
  hipLaunchKernelGGL(plan_init_kernel, dim3(1), dim3(64), 0, s, sc);
  if (m > 0) {
    int64_t thr_r = (int64_t)ceil(tau * (double)n);
    if (thr_r < min_count) thr_r = min_count;
    hipLaunchKernelGGL(row_flags_kernel, dim3(gm), dim3(256), 0, s, ro, m, nnz, thr_r, hot);
    if ((e = exclusive_scan_u32(hot, rrank, m, (uint32_t*)&sc->H, scan_ws, s)) != hipSuccess)
      return e;
  }
  if (n > 0) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(gn), dim3(256), 0, s, ccnt, n, 0u);
    if (m > 0) {
      if (col_i32)
        hipLaunchKernelGGL(col_count_kernel<int32_t>, dim3(gm16), dim3(256), 0, s, ro,
                           (const int32_t*)col, m, n, nnz, hot, ccnt);
      else
        hipLaunchKernelGGL(col_count_kernel<int16_t>, dim3(gm16), dim3(256), 0, s, ro,
                           (const int16_t*)col, m, n, nnz, hot, ccnt);
    }
    hipLaunchKernelGGL(col_flags_kernel, dim3(gn), dim3(256), 0, s, ccnt, n, m, tau, min_count,
                       sc, cflag);
    if ((e = exclusive_scan_u32(cflag, crank, n, (uint32_t*)&sc->Hc, scan_ws, s)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(compact_cols_kernel, dim3(gn), dim3(256), 0, s, cflag, crank, n,
                       out->hot_cols, col_map);
  }
  if (m > 0)
    hipLaunchKernelGGL(compact_rows_kernel, dim3(gm), dim3(256), 0, s, hot, rrank, m, sc,
                       out->rows);
  hipLaunchKernelGGL(derive_tiles_kernel, dim3(1), dim3(64), 0, s, m, out->tiles_a_cols, sc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nnz > 0) {
    ClassifyArgs ca{ro,  col,  m,       n,   nnz, hot, rrank, col_map, sc, out->tiles_a_cols,
                    out->rest_key, out->nb_max, key, rc};
    if (col_i32)
      hipLaunchKernelGGL(classify_kernel<int32_t>, dim3(gm16), dim3(256), 0, s, ca);
    else
      hipLaunchKernelGGL(classify_kernel<int16_t>, dim3(gm16), dim3(256), 0, s, ca);
  }
  hipLaunchKernelGGL(merge_buckets_kernel, dim3((unsigned)cdiv(nnz > 0 ? nnz : 1, 256)),
                     dim3(256), 0, s, key, nnz, (uint32_t)out->rest_key, out->nb_max, forced,
                     sc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const uint32_t* skey = key;
  const uint32_t* src = key;
  if (nnz > 0) {
    if ((e = radix_sort_u32_iota_ptrs(key, nnz, bit_length((uint64_t)(nkeys - 1)), radix_ws,
                                      &skey, &src, s)) != hipSuccess)
      return e;
  }
  const unsigned gkb = (unsigned)cdiv((nnz > nkeys ? nnz : nkeys) + 1, 256);
  if (col_i32)
    hipLaunchKernelGGL(key_bounds_kernel<int32_t>, dim3(gkb), dim3(256), 0, s, skey, src, rc,
                       (const int32_t*)col, nnz, nkeys, out->key_start, out->ent_pos,
                       out->ent_rc, out->ent_col);
  else
    hipLaunchKernelGGL(key_bounds_kernel<int16_t>, dim3(gkb), dim3(256), 0, s, skey, src, rc,
                       (const int16_t*)col, nnz, nkeys, out->key_start, out->ent_pos,
                       out->ent_rc, out->ent_col);
  hipLaunchKernelGGL(plan_finish_kernel, dim3(1), dim3(64), 0, s, out->key_start, nnz, sc);
  if (nnz > 0) {
    // the remainder once more in row order (tile entries behind it), for
    // calls that cut K into pieces: the key array and the sort's workspace
    // are free again
    const unsigned gz = (unsigned)cdiv(nnz, 256);
    hipLaunchKernelGGL(rest_row_key_kernel, dim3(gz), dim3(256), 0, s, out->ent_rc, nnz, m, sc,
                       key);
    const uint32_t* skey2 = key;
    const uint32_t* src2 = key;
    if ((e = radix_sort_u32_iota_ptrs(key, nnz, bit_length((uint64_t)m), radix_ws, &skey2, &src2,
                                      s)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(rest_gather_kernel, dim3(gz), dim3(256), 0, s, src2, nnz, out->ent_pos,
                       out->ent_rc, out->ent_col, out->row_pos, out->row_rc, out->row_col);
  }
  return hipGetLastError();
}

hipError_t fetch_sddmm_plan_counts(SddmmPlanDev* p, hipStream_t s) {
  int32_t ks[kMaxBuckets + 1] = {};
  hipError_t e = hipMemcpyAsync(&p->h, p->sc, sizeof(SddmmPlanScalars), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(ks, p->key_start + p->rest_key, (size_t)(p->nb_max + 1) * 4,
                       hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  for (int b = 0; b <= kMaxBuckets; ++b) p->bucket_start[b] = ks[b <= p->h.nb ? b : p->h.nb];
  // most entries in one tile (sizes the grid of the partial-sum kernel)
  p->max_tile_nnz = 0;
  if (p->h.tiles > 0) {
    int32_t* kst = (int32_t*)malloc((size_t)(p->h.tiles + 1) * 4);
    if (!kst) return hipErrorOutOfMemory;
    e = hipMemcpyAsync(kst, p->key_start, (size_t)(p->h.tiles + 1) * 4,
                       hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess)
      for (int64_t t = 0; t < p->h.tiles; ++t) {
        const int64_t c = kst[t + 1] - kst[t];
        p->max_tile_nnz = c > p->max_tile_nnz ? c : p->max_tile_nnz;
      }
    free(kst);
    if (e != hipSuccess) return e;
  }
  p->host_ok = true;
  return hipSuccess;
}

// K splits of the dense tiles for this plan and K.  With the tile count on
// the host (plans made by spops_sddmm_plan_create): kOptSddmmSplits when set,
// else, when there are fewer tiles than compute units, the count S (at most
// the number of K slices, and at most 16) that minimizes rounds * (slices
// per item + 2), where a round is one item per resident workgroup slot and
// 2 slices stand for an item's fixed cost (gathering its rows, pipeline
// start, epilogue); ties go to fewer splits.  Otherwise, and without host
// counts: 1.
SddmmTileSched sddmm_tile_schedule(const SddmmPlanDev& p, int64_t K) {
  SddmmTileSched sc{};
  sc.splits = 1;
  if (!p.host_ok || p.h.tiles <= 0 || K <= 0) return sc;
  const int64_t nsl = cdiv(K, TK);
  const int64_t smax = nsl < 16 ? nsl : 16;
  const int64_t opt = option(kOptSddmmSplits);
  if (opt > 0) {
    sc.splits = (int)(opt < smax ? opt : smax);
    return sc;
  }
  // a full round of tiles already keeps every compute unit busy; splitting
  // then only adds items and the partial-sum pass (measured slower)
  if (p.h.tiles >= p.cus) return sc;
  int64_t best_cost = INT64_MAX;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t cost = cdiv(p.h.tiles * S, (int64_t)p.cus * kTileWgPerCu) * (cdiv(nsl, S) + 2);
    if (cost < best_cost) {
      best_cost = cost;
      sc.splits = (int)S;
    }
  }
  return sc;
}

size_t sddmm_split_bytes(const SddmmPlanDev& p, const SddmmTileSched& sc) {
  if (sc.splits <= 1 || !p.host_ok) return 0;
  return align256((size_t)sc.splits * (size_t)(p.h.tiled > 0 ? p.h.tiled : 1) * 4);
}

hipError_t launch_sddmm_tiles(const SddmmPlanDev& p, int64_t K, const void* A, int64_t lda,
                              const void* BT, int64_t ldbt, int dtype, void* out, int out_dtype,
                              const SddmmTileSched& sched, float* part, hipStream_t s) {
  if (p.host_ok && (p.h.tiles == 0 || p.h.tiled == 0)) return hipSuccess;
  // buffer offsets are 32-bit: each operand under 2 GiB
  if (p.m * lda * 2 >= ((int64_t)1 << 31) || p.n * ldbt * 2 >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  SddmmTileSched sc = sched;
  if (!p.host_ok || (sc.splits > 1 && !part)) sc.splits = 1;
  TileArgs ta{K,           lda,        ldbt,         p.n,          (const uint16_t*)A,
              (const uint16_t*)BT,     (uint32_t)(p.m * lda * 2),  (uint32_t)(p.n * ldbt * 2),
              p.rows,       p.hot_cols,   p.sc,
              p.tiles_a_cols,          p.key_start,  p.ent_pos,    p.ent_rc,
              sc.splits,   part,       out};
  // one workgroup per item when the tile count is known on the host, else a
  // grid of at most two rounds over the compute units looping over the
  // items; a multiple of 8 (the kernel's XCD-aware order needs it)
  int64_t grid = p.host_ok ? p.h.tiles * (int64_t)sc.splits : p.max_tiles;
  if (!p.host_ok && grid > 2 * kTileWgPerCu * p.cus) grid = 2 * kTileWgPerCu * p.cus;
  grid = (grid + 7) & ~(int64_t)7;
  hipError_t e;
  if (out_dtype == kF32)
    e = launch_tiles_typed<float>(ta, (unsigned)grid, dtype, s);
  else if (dtype == kBF16)
    e = launch_tiles_typed<bf16_t>(ta, (unsigned)grid, dtype, s);
  else
    e = launch_tiles_typed<_Float16>(ta, (unsigned)grid, dtype, s);
  if (e != hipSuccess || sc.splits <= 1) return e;
  const int64_t most = p.max_tile_nnz;
  if (out_dtype == kF32) return launch_split_sum<float>(ta, p.h.tiles, most, s);
  if (dtype == kBF16) return launch_split_sum<bf16_t>(ta, p.h.tiles, most, s);
  return launch_split_sum<_Float16>(ta, p.h.tiles, most, s);
}

}  // namespace spops

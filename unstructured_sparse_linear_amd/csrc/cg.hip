// cg.hip -- conjugate gradients on gfx950.
//
// The torchsparsegradutils README lists a CG solver among its built-in
// iterative solvers ("Built-in Iterative Solvers") and calls a sparse solve
// with it and a tolerance ("Generic solve").  The page gives no steps; the
// method is that of Hestenes and Stiefel (1952):
//   r = b - A x, p = r;  per iteration  q = A p,  alpha = r.r / p.q,
//   x += alpha p,  r -= alpha q,  beta = r'.r' / r.r,  p = r' + beta p,
// stopping once r.r <= rtol^2 b.b or after max_iter iterations.
//
// Iteration k is laid out as
//   begin:   r.r from the partials of the previous update; record it, stop
//            when it is small enough; beta = r.r / (r.r of iteration k-1)
//            (0 for k = 0)
//   product: p = r + beta p_prev and q = A p, with the partials of p.q
//   update:  alpha = r.r / p.q, x += alpha p, r -= alpha q, partials of r.r
// so that the whole iteration is two launches when the SpMV can run as
// entry-range blocks (balanced rows with a plan): the direction is formed on the
// fly where the SpMV gathers it (every workgroup computes beta itself from
// the same partials) and each workgroup writes p and q for its own rows and
// the p.q partial of its rows.  p and r are stored interleaved, (p, r) pairs
// of floats, so forming a direction entry takes one 8-byte gather; two such
// arrays alternate between iterations (iteration k reads pairs (p_prev, r)
// from one and leaves (p, r_new) in the other), so no workgroup overwrites a
// value another one still gathers.  Otherwise the iteration is the library's
// SpMV (reading p with a leading dimension of 2) between a direction kernel
// and a p.q kernel.  Vectors are f32; dot products, alpha and beta are
// float64.  Every dot product is summed per workgroup in a fixed order into a
// partial, and every workgroup that needs the total adds all partials in the
// same fixed order, so all see the same bits and a run is deterministic.
//
// The solver state (r.r of the last two iterations, b.b, the threshold, the
// iteration count and a done flag) stays in device memory; the host enqueues
// iterations with their index k as an argument and reads the state only at
// its convergence checks.  Once the done flag is set every later solver
// kernel returns at once, so iterations enqueued past convergence change
// nothing.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
static_assert(kBlock == kStreamBlock, "row blocks use the vector kernels' block size");

// Sum of v over the workgroup, the same value returned to every thread.
// Lane 0 of each wave holds its wave's butterfly sum; wave sums are added in
// wave order.
__device__ double block_sum(double v, double* lds) {
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = lds[0];
    for (int w = 1; w < kWaves; ++w) t += lds[w];
    lds[kWaves] = t;
  }
  __syncthreads();
  return lds[kWaves];
}

// Sum of the n per-workgroup partials, in a fixed order: thread t adds
// partials t, t + kBlock, ... (up to eight of them requested together),
// then the workgroup sum.
__device__ double sum_partials(const double* part, int n, double* lds) {
  constexpr int kTogether = 8;
  double s = 0.0;
  for (int i0 = threadIdx.x; i0 < n; i0 += kBlock * kTogether) {
    double v[kTogether];
#pragma unroll
    for (int u = 0; u < kTogether; ++u) {
      const int i = i0 + u * kBlock;
      v[u] = i < n ? part[i] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kTogether; ++u)
      if (i0 + u * kBlock < n) s += v[u];
  }
  return block_sum(s, lds);
}

// The done flag as one value for the whole workgroup: workgroup 0 of the
// same launch may set it while others start, and every thread of a
// workgroup must take the same branch (the sums hold barriers).
__device__ bool stopped(const CgState* st, int* flag) {
  if (threadIdx.x == 0) *flag = *(const volatile int32_t*)&st->done;
  __syncthreads();
  return *flag != 0;
}

// Start of iteration k, after stopped(): r.r of the current residual from
// the partials of the previous update (or of the set-up), recorded by
// workgroup 0 together with the count of finished iterations; false (and
// done set) when it is at most the threshold.  beta for the new direction
// goes to *beta.
__device__ bool begin_iteration(int64_t k, int nparts, const double* part_rr, CgState* st,
                                double* lds, double* beta) {
  const double rr = sum_partials(part_rr, nparts, lds);
  const bool go = rr > st->thr;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st->rr[k & 1] = rr;
    st->iters = k;
    if (!go) st->done = 1;
  }
  *beta = k == 0 ? 0.0 : rr / st->rr[(k - 1) & 1];
  return go;
}

// p = r + beta p_prev from a (p_prev, r) pair.
__device__ __forceinline__ float direction(double beta, float2 pr) {
  return (float)__builtin_fma(beta, (double)pr.x, (double)pr.y);
}

__device__ __forceinline__ int64_t first() { return (int64_t)blockIdx.x * kBlock + threadIdx.x; }
__device__ __forceinline__ int64_t stride() { return (int64_t)gridDim.x * kBlock; }

// r = b - q (q = A x0); pairs (0, r), so the first direction is r; partial
// sums of r.r and b.b.
__global__ __launch_bounds__(kBlock) void cg_init_kernel(int64_t m, const float* b,
                                                         const float* q, float2* pr,
                                                         double* part_rr, double* part_bb) {
  __shared__ double lds[kWaves + 1];
  double srr = 0.0, sbb = 0.0;
  for (int64_t i = first(); i < m; i += stride()) {
    const float bi = b[i];
    const float ri = bi - q[i];
    pr[i] = make_float2(0.f, ri);
    srr += (double)ri * (double)ri;
    sbb += (double)bi * (double)bi;
  }
  srr = block_sum(srr, lds);
  sbb = block_sum(sbb, lds);
  if (threadIdx.x == 0) {
    part_rr[blockIdx.x] = srr;
    part_bb[blockIdx.x] = sbb;
  }
}

__global__ __launch_bounds__(kBlock) void cg_init_state_kernel(int nparts, const double* part_bb,
                                                               double rtol, CgState* st) {
  __shared__ double lds[kWaves + 1];
  const double bb = sum_partials(part_bb, nparts, lds);
  if (threadIdx.x == 0) {
    st->rr[0] = st->rr[1] = 0.0;
    st->bb = bb;
    st->thr = rtol * rtol * bb;
    st->iters = 0;
    st->done = 0;
  }
}

// Records the state of iteration k (at the host's convergence checks).
__global__ __launch_bounds__(kBlock) void cg_record_kernel(int64_t k, int nparts,
                                                           const double* part_rr, CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  double beta;
  if (stopped(st, &flag)) return;
  begin_iteration(k, nparts, part_rr, st, lds, &beta);
}

// Direction for the library's SpMV: p = r + beta p_prev into the p slots of
// the next pair array.
__global__ __launch_bounds__(kBlock) void cg_direction_kernel(int64_t m, int64_t k, int nparts,
                                                              const double* part_rr,
                                                              const float2* pr, float2* pr_next,
                                                              CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  double beta;
  if (stopped(st, &flag)) return;
  if (!begin_iteration(k, nparts, part_rr, st, lds, &beta)) return;
  for (int64_t i = first(); i < m; i += stride()) pr_next[i].x = direction(beta, pr[i]);
}

// partial sums of p.q (after the library's SpMV)
__global__ __launch_bounds__(kBlock) void cg_dot_kernel(int64_t m, const float2* pr_next,
                                                        const float* q, double* part,
                                                        const CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  if (stopped(st, &flag)) return;
  double s = 0.0;
  for (int64_t i = first(); i < m; i += stride()) s += (double)pr_next[i].x * (double)q[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// alpha = r.r / p.q; x += alpha p; r_new = r - alpha q (r from the pairs
// read this iteration, p and r_new in the next pairs); partial sums of
// r_new.r_new.  A step that is not positive and finite (p.q <= 0: A is not
// positive definite, or the iteration has broken down) stops the solver
// (done = 2) before anything is written.  Each thread takes kUpdateElems
// elements per round, strided by the grid; the first round's loads are
// issued before the p.q sum so that their latency overlaps it.
constexpr int kUpdateElems = 2;

__global__ __launch_bounds__(kBlock) void cg_update_kernel(
    int64_t m, int64_t k, int nparts, const double* __restrict__ part_pq, float* __restrict__ x,
    const float2* __restrict__ pr, float2* __restrict__ pr_next, const float* __restrict__ q,
    double* __restrict__ part_rr, CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  if (stopped(st, &flag)) return;
  constexpr int E = kUpdateElems;
  const int64_t step = stride() * E;
  int64_t i0 = first();
  float xv[E], pv[E], rv[E], qv[E];
  auto load = [&](int64_t base) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i = base + e * stride();
      const int64_t j = i < m ? i : m - 1;
      xv[e] = x[j];
      pv[e] = pr_next[j].x;
      rv[e] = pr[j].y;
      qv[e] = q[j];
    }
  };
  load(i0);
  const double pq = sum_partials(part_pq, nparts, lds);
  const double alpha = st->rr[k & 1] / pq;
  if (!(pq > 0.0) || !(alpha < INFINITY)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) st->done = 2;
    return;
  }
  double s = 0.0;
  for (; i0 < m; i0 += step) {
    if (i0 != first()) load(i0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t i = i0 + e * stride();
      if (i < m) {
        const float xi = (float)__builtin_fma(alpha, (double)pv[e], (double)xv[e]);
        const float ri = (float)__builtin_fma(-alpha, (double)qv[e], (double)rv[e]);
        x[i] = xi;
        pr_next[i] = make_float2(pv[e], ri);
        s += (double)ri * (double)ri;
      }
    }
  }
  s = block_sum(s, lds);
  if (threadIdx.x == 0) part_rr[blockIdx.x] = s;
}

// Begin + product of iteration k in one launch, as the entry-range blocks of
// the SpMV (spmv_flat_kernel): workgroup b loads the entries [b*E, (b+1)*E)
// and the T after them in 4-entry groups, puts their products in LDS and
// writes q, p and the p.q partial of the rows that start in its range
// (blk_row), one thread per row adding its products in stored order.  The
// gathered operand is the new direction, formed from a (p_prev, r) pair
// where it is read.  The col/val loads are issued before the r.r sum, so
// that their latency overlaps it.  Offsets that do not match the plan send
// the block's rows to a wave per row.
template <typename IT, int U, bool QUAD>
__global__ __launch_bounds__(kBlock) void cg_spmv_kernel(CgSpmvArgs a) {
  extern __shared__ __align__(16) float prod[];  // E + T + 8 floats
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  if (stopped(a.st, &flag)) return;
  const IT* col = (const IT*)a.col;
  const float* val = a.val;
  const float2* pr = a.pr;
  // entry positions fit in 32 bits with room for E + T past the last one
  const int m = (int)a.m, nnz = (int)a.nnz;
  const int E = a.E, T = a.T;
  const int nblk = (nnz + E - 1) / E;
  const int b = (int)row_block(blockIdx.x, gridDim.x, 1);  // 0 for workgroup 0
  const int t = threadIdx.x;
  const bool live = b < nblk;
  const int e0 = live ? b * E : 0;
  const int e1 = live ? min(e0 + E, nnz) : 0;
  const int eL = live ? min(e1 + T, nnz) : 0;
  const int gbeg = e0 >> 2;
  const int gend = QUAD && live ? min(nnz >> 2, (eL + 3) >> 2) : gbeg;
  IT c[U][4];
  float v[U][4];
  if (gend > gbeg) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gq = min(gbeg + t + u * kBlock, gend - 1);
      load_quad(col + 4 * gq, c[u]);
      load_quad(val + 4 * gq, v[u]);
    }
  }
  double beta;
  if (!begin_iteration(a.k, a.nparts_rr, a.part_rr, a.st, lds, &beta)) return;
  if (!live) {
    if (t == 0) a.part_pq[blockIdx.x] = 0.0;
    return;
  }
  const int rb = min(max(a.blk_row[b], 0), m);
  const int re = min(max(a.blk_row[b + 1], rb), m);
  const int lo = a.ro[rb], hi = a.ro[re];
  const int r = rb + t;
  const int rl = min(r < re ? r : rb, m - 1);
  const int o0 = a.ro[rl], o1 = a.ro[rl + 1];
  float* p_next = (float*)a.pr_next;  // p of row i at p_next[2 i]
  double s = 0.0;
  int p_done = e0;
  if (gend > gbeg) {
    p_done = max(e0, 4 * gend);
    float xv[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ci = (int)c[u][q];
        const bool ok = (unsigned)ci < (unsigned)m;
        const float pv = direction(beta, pr[ok ? ci : 0]);
        xv[u][q] = ok ? pv : 0.f;
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = gbeg + t + u * kBlock;
      if (gu < gend) {
        float4 pq4;
        pq4.x = v[u][0] * xv[u][0];
        pq4.y = v[u][1] * xv[u][1];
        pq4.z = v[u][2] * xv[u][2];
        pq4.w = v[u][3] * xv[u][3];
        *reinterpret_cast<float4*>(prod + (4 * gu - e0)) = pq4;
      }
    }
  }
  for (int e = p_done + t; e < eL; e += kBlock) {
    const int ci = (int)col[e];
    const bool ok = (unsigned)ci < (unsigned)m;
    const float pv = direction(beta, pr[ok ? ci : 0]);
    prod[e - e0] = ok ? val[e] * pv : 0.f;
  }
  __syncthreads();
  if (lo >= e0 && hi <= eL) {
    for (int rr = r; rr < re; rr += kBlock) {
      const int a0 = rr == r ? o0 : a.ro[rr];
      const int a1 = rr == r ? o1 : a.ro[rr + 1];
      const int q0 = a0 < e0 ? e0 : (a0 > eL ? eL : a0);
      const int q1 = a1 < q0 ? q0 : (a1 > eL ? eL : a1);
      float y = 0.f;
#pragma unroll 4
      for (int i = q0; i < q1; ++i) y += prod[i - e0];
      const float pn = direction(beta, pr[rr]);
      a.q[rr] = y;
      p_next[2 * (int64_t)rr] = pn;
      s += (double)pn * (double)y;
    }
  } else {
    // offsets that do not match the plan: a wave per owned row
    const int w = t / kWave, l = lane_id();
    for (int rr = rb + w; rr < re; rr += kWaves) {
      const int64_t lo2 = a.ro[rr], hi2 = a.ro[rr + 1];
      const int64_t p0 = lo2 < 0 ? 0 : (lo2 > nnz ? nnz : lo2);
      const int64_t p1 = hi2 < p0 ? p0 : (hi2 > nnz ? nnz : hi2);
      float y = 0.f;
      for (int64_t p = p0 + l; p < p1; p += kWave) {
        const int ci = (int)col[p];
        if ((unsigned)ci < (unsigned)m) y = __builtin_fmaf(val[p], direction(beta, pr[ci]), y);
      }
      y = group_sum<kWave>(y);
      if (l == 0) {
        const float pn = direction(beta, pr[rr]);
        a.q[rr] = y;
        p_next[2 * (int64_t)rr] = pn;
        s += (double)pn * (double)y;
      }
    }
  }
  s = block_sum(s, lds);
  if (t == 0) a.part_pq[blockIdx.x] = s;
}

}  // namespace

int cg_parts(int64_t m) {
  // kUpdateElems elements per thread: few partials for every workgroup to add
  const int64_t nb = cdiv(m, kUpdateElems * kBlock);
  return (int)(nb < 1 ? 1 : (nb > kCgMaxParts ? kCgMaxParts : nb));
}

size_t cg_workspace_bytes(int64_t m, int64_t npq, size_t spmm_ws) {
  const int64_t np = std::max<int64_t>(npq, kCgMaxParts);
  return 2 * align256((size_t)m * sizeof(float2)) + align256((size_t)m * sizeof(float)) +
         align256((size_t)np * sizeof(double)) + align256(kCgMaxParts * sizeof(double)) +
         align256(sizeof(CgState)) + align256(spmm_ws);
}

CgBuffers carve_cg_workspace(void* ws, int64_t m, int64_t npq) {
  char* c = (char*)ws;
  CgBuffers w;
  const size_t pb = align256((size_t)m * sizeof(float2));
  const size_t qb = align256((size_t)m * sizeof(float));
  const size_t pqb = align256((size_t)std::max<int64_t>(npq, kCgMaxParts) * sizeof(double));
  const size_t rrb = align256(kCgMaxParts * sizeof(double));
  w.pr[0] = (float2*)c;
  w.pr[1] = (float2*)(c + pb);
  w.q = (float*)(c + 2 * pb);
  w.part_pq = (double*)(c + 2 * pb + qb);
  w.part_rr = (double*)(c + 2 * pb + qb + pqb);
  w.st = (CgState*)(c + 2 * pb + qb + pqb + rrb);
  w.spmm_ws = c + 2 * pb + qb + pqb + rrb + align256(sizeof(CgState));
  return w;
}

hipError_t launch_cg_init(int64_t m, const float* b, const CgBuffers& w, double rtol,
                          hipStream_t s) {
  const int nb = cg_parts(m);
  // b.b partials borrow the p.q partials (free until the first product)
  hipLaunchKernelGGL(cg_init_kernel, dim3(nb), dim3(kBlock), 0, s, m, b, (const float*)w.q,
                     w.pr[0], w.part_rr, w.part_pq);
  hipLaunchKernelGGL(cg_init_state_kernel, dim3(1), dim3(kBlock), 0, s, nb,
                     (const double*)w.part_pq, rtol, w.st);
  return hipGetLastError();
}

hipError_t launch_cg_record(int64_t m, int64_t k, const CgBuffers& w, hipStream_t s) {
  hipLaunchKernelGGL(cg_record_kernel, dim3(1), dim3(kBlock), 0, s, k, cg_parts(m),
                     (const double*)w.part_rr, w.st);
  return hipGetLastError();
}

hipError_t launch_cg_direction(int64_t m, int64_t k, const CgBuffers& w, hipStream_t s) {
  const int nb = cg_parts(m);
  hipLaunchKernelGGL(cg_direction_kernel, dim3(nb), dim3(kBlock), 0, s, m, k, nb,
                     (const double*)w.part_rr, (const float2*)w.pr[k & 1], w.pr[(k + 1) & 1],
                     w.st);
  return hipGetLastError();
}

hipError_t launch_cg_dot_update(int64_t m, int64_t k, float* x, const CgBuffers& w,
                                hipStream_t s) {
  const int nb = cg_parts(m);
  hipLaunchKernelGGL(cg_dot_kernel, dim3(nb), dim3(kBlock), 0, s, m,
                     (const float2*)w.pr[(k + 1) & 1], (const float*)w.q, w.part_pq,
                     (const CgState*)w.st);
  hipLaunchKernelGGL(cg_update_kernel, dim3(nb), dim3(kBlock), 0, s, m, k, nb,
                     (const double*)w.part_pq, x, (const float2*)w.pr[k & 1], w.pr[(k + 1) & 1],
                     (const float*)w.q, w.part_rr, w.st);
  return hipGetLastError();
}

hipError_t launch_cg_fused(const CgSpmvArgs& a0, float* x, const CgBuffers& w, hipStream_t s) {
  CgSpmvArgs a = a0;
  const int64_t m = a.m, k = a.k;
  if (a.U <= 0 || a.E <= 0 || a.E + a.T > a.U * 4 * kBlock || a.nnz + a.E + a.T >= INT32_MAX)
    return hipErrorInvalidValue;
  a.pr = w.pr[k & 1];
  a.pr_next = w.pr[(k + 1) & 1];
  a.q = w.q;
  a.part_pq = w.part_pq;
  a.part_rr = w.part_rr;
  a.nparts_rr = cg_parts(m);
  a.st = w.st;
  const bool quad = ((uintptr_t)a.col % (4 * (a.col_i32 ? 4 : 2)) == 0) &&
                    ((uintptr_t)a.val % 16 == 0);
  const int64_t grid = cg_fused_grid(a.nnz, a.E);
  const size_t lds = (size_t)(a.E + a.T + 8) * sizeof(float);
#define CGK(IT, U, Q) \
  hipLaunchKernelGGL((cg_spmv_kernel<IT, U, Q>), dim3((unsigned)grid), dim3(kBlock), lds, s, a)
#define CGU(IT, U)     \
  if (quad)            \
    CGK(IT, U, true);  \
  else                 \
    CGK(IT, U, false)
  switch (a.U) {
    case 1: if (a.col_i32) { CGU(int32_t, 1); } else { CGU(int16_t, 1); } break;
    case 2: if (a.col_i32) { CGU(int32_t, 2); } else { CGU(int16_t, 2); } break;
    case 4: if (a.col_i32) { CGU(int32_t, 4); } else { CGU(int16_t, 4); } break;
    default: return hipErrorInvalidValue;
  }
#undef CGU
#undef CGK
  hipLaunchKernelGGL(cg_update_kernel, dim3(cg_parts(m)), dim3(kBlock), 0, s, m, k, (int)grid,
                     (const double*)w.part_pq, x, (const float2*)a.pr, a.pr_next,
                     (const float*)w.q, w.part_rr, w.st);
  return hipGetLastError();
}

int64_t cg_fused_grid(int64_t nnz, int32_t E) {
  if (E <= 0 || nnz <= 0) return 0;
  return (cdiv(nnz, (int64_t)E) + 7) & ~(int64_t)7;
}

}  // namespace spops

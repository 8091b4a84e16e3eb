// cg.hip -- the vector kernels of conjugate gradients on gfx950.
//
// The torchsparsegradutils README lists a CG solver among its built-in
// iterative solvers ("Built-in Iterative Solvers") and calls a sparse solve
// with it and a tolerance ("Generic solve").  The page gives no steps; the
// method is that of Hestenes and Stiefel (1952):
//   r = b - A x, p = r;  per iteration  q = A p,  alpha = r.r / p.q,
//   x += alpha p,  r -= alpha q,  beta = r'.r' / r.r,  p = r' + beta p,
// stopping once r.r <= rtol^2 b.b or after max_iter iterations.
//
// The product q = A p is the library's SpMV (launch_spmm with N = 1); this
// file holds the rest.  Vectors are f32; dot products, alpha and beta are
// float64.  Each dot product is summed per workgroup in a fixed order into a
// partial, and every workgroup that needs the total adds all partials in the
// same fixed order, so every workgroup sees the same bits and a run is
// deterministic.  The solver state (r.r of the last two iterations, b.b, the
// threshold, the iteration count and a done flag) lives in device memory:
// the host enqueues iterations with their index k as an argument and reads
// the state only at its convergence checks.  Once the done flag is set every
// later kernel of the solver returns at once, so iterations enqueued past
// convergence leave x as it was at convergence.
#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

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

// Sum of the n per-workgroup partials, in a fixed order.
__device__ double sum_partials(const double* part, int n, double* lds) {
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kBlock) s += part[i];
  return block_sum(s, lds);
}

// The done flag as one value for the whole workgroup: workgroup 0 of the
// same launch may set it while others start, and every thread of a
// workgroup must take the same branch (the sums below hold barriers).
__device__ bool stopped(const CgState* st, int* flag) {
  if (threadIdx.x == 0) *flag = *(const volatile int32_t*)&st->done;
  __syncthreads();
  return *flag != 0;
}

__device__ __forceinline__ int64_t first() { return (int64_t)blockIdx.x * kBlock + threadIdx.x; }
__device__ __forceinline__ int64_t stride() { return (int64_t)gridDim.x * kBlock; }

// r = b - q (q = A x0), p = r; partial sums of r.r and b.b.
__global__ __launch_bounds__(kBlock) void cg_init_kernel(int64_t m, const float* b,
                                                         const float* q, float* r, float* p,
                                                         double* part_rr, double* part_bb) {
  __shared__ double lds[kWaves + 1];
  double srr = 0.0, sbb = 0.0;
  for (int64_t i = first(); i < m; i += stride()) {
    const float bi = b[i];
    const float ri = bi - q[i];
    r[i] = ri;
    p[i] = ri;
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

__global__ __launch_bounds__(kBlock) void cg_init_state_kernel(int nparts, const double* part_rr,
                                                               const double* part_bb, double rtol,
                                                               CgState* st) {
  __shared__ double lds[kWaves + 1];
  const double rr = sum_partials(part_rr, nparts, lds);
  const double bb = sum_partials(part_bb, nparts, lds);
  if (threadIdx.x == 0) {
    st->rr[0] = rr;
    st->rr[1] = 0.0;
    st->bb = bb;
    st->thr = rtol * rtol * bb;
    st->iters = 0;
    st->done = rr > st->thr ? 0 : 1;
  }
}

// partial sums of p.q
__global__ __launch_bounds__(kBlock) void cg_dot_kernel(int64_t m, const float* p, const float* q,
                                                        double* part, const CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  if (stopped(st, &flag)) return;
  double s = 0.0;
  for (int64_t i = first(); i < m; i += stride()) s += (double)p[i] * (double)q[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// alpha = r.r / p.q; x += alpha p; r -= alpha q; partial sums of the new r.r.
// A step that is not positive and finite (p.q <= 0: A is not positive
// definite, or the iteration has broken down) stops the solver (done = 2)
// before anything is written.
__global__ __launch_bounds__(kBlock) void cg_update_kernel(int64_t m, int64_t k, int nparts,
                                                           const double* part_pq, float* x,
                                                           const float* p, float* r,
                                                           const float* q, double* part_rr,
                                                           CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  if (stopped(st, &flag)) return;
  const double pq = sum_partials(part_pq, nparts, lds);
  const double alpha = st->rr[k & 1] / pq;
  if (!(pq > 0.0) || !(alpha < INFINITY)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) st->done = 2;
    return;
  }
  double s = 0.0;
  for (int64_t i = first(); i < m; i += stride()) {
    const float xi = (float)__builtin_fma(alpha, (double)p[i], (double)x[i]);
    const float ri = (float)__builtin_fma(-alpha, (double)q[i], (double)r[i]);
    x[i] = xi;
    r[i] = ri;
    s += (double)ri * (double)ri;
  }
  s = block_sum(s, lds);
  if (threadIdx.x == 0) part_rr[blockIdx.x] = s;
}

// beta = r'.r' / r.r; p = r' + beta p; workgroup 0 records the iteration.
__global__ __launch_bounds__(kBlock) void cg_direction_kernel(int64_t m, int64_t k, int nparts,
                                                              const double* part_rr,
                                                              const float* r, float* p,
                                                              CgState* st) {
  __shared__ double lds[kWaves + 1];
  __shared__ int flag;
  if (stopped(st, &flag)) return;
  const double rr1 = sum_partials(part_rr, nparts, lds);
  const double beta = rr1 / st->rr[k & 1];
  for (int64_t i = first(); i < m; i += stride())
    p[i] = (float)__builtin_fma(beta, (double)p[i], (double)r[i]);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st->rr[(k + 1) & 1] = rr1;
    st->iters = k + 1;
    if (!(rr1 > st->thr)) st->done = 1;
  }
}

}  // namespace

size_t cg_workspace_bytes(int64_t m, size_t spmm_ws) {
  return 3 * align256((size_t)m * sizeof(float)) + 2 * align256(kCgMaxParts * sizeof(double)) +
         align256(sizeof(CgState)) + align256(spmm_ws);
}

CgBuffers carve_cg_workspace(void* ws, int64_t m) {
  char* c = (char*)ws;
  CgBuffers w;
  const size_t vb = align256((size_t)m * sizeof(float));
  const size_t pb = align256(kCgMaxParts * sizeof(double));
  w.r = (float*)c;
  w.p = (float*)(c + vb);
  w.q = (float*)(c + 2 * vb);
  w.part0 = (double*)(c + 3 * vb);
  w.part1 = (double*)(c + 3 * vb + pb);
  w.st = (CgState*)(c + 3 * vb + 2 * pb);
  w.spmm_ws = c + 3 * vb + 2 * pb + align256(sizeof(CgState));
  return w;
}

int cg_parts(int64_t m) {
  const int64_t nb = cdiv(m, kBlock);
  return (int)(nb < 1 ? 1 : (nb > kCgMaxParts ? kCgMaxParts : nb));
}

hipError_t launch_cg_init(int64_t m, const float* b, const float* q, const CgBuffers& w,
                          double rtol, hipStream_t s) {
  const int nb = cg_parts(m);
  hipLaunchKernelGGL(cg_init_kernel, dim3(nb), dim3(kBlock), 0, s, m, b, q, w.r, w.p, w.part0,
                     w.part1);
  hipLaunchKernelGGL(cg_init_state_kernel, dim3(1), dim3(kBlock), 0, s, nb, w.part0, w.part1,
                     rtol, w.st);
  return hipGetLastError();
}

hipError_t launch_cg_after_product(int64_t m, int64_t k, float* x, const CgBuffers& w,
                                   hipStream_t s) {
  const int nb = cg_parts(m);
  hipLaunchKernelGGL(cg_dot_kernel, dim3(nb), dim3(kBlock), 0, s, m, w.p, w.q, w.part0, w.st);
  hipLaunchKernelGGL(cg_update_kernel, dim3(nb), dim3(kBlock), 0, s, m, k, nb, w.part0, x, w.p,
                     w.r, w.q, w.part1, w.st);
  hipLaunchKernelGGL(cg_direction_kernel, dim3(nb), dim3(kBlock), 0, s, m, k, nb, w.part1, w.r,
                     w.p, w.st);
  return hipGetLastError();
}

}  // namespace spops

// adam.hip -- masked Adam step over a value vector on gfx950.
//
// The SparseAdam page (tensorplay.optim.sparse_adam) describes a masked
// Adam: only positions whose gradient is materialized update their moments
// and their parameter; all other positions are left untouched, and a
// materialized zero still counts.  The step is Adam's (Kingma and Ba, 2015,
// Algorithm 1, in the efficient form of the end of their Section 2):
//   m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
//   theta -= alpha_t m / (sqrt(v) + eps),
//   alpha_t = lr sqrt(1 - beta2^t) / (1 - beta1^t)  (computed on the host).
// One thread per materialized entry: consecutive threads take consecutive
// gradient entries, so the gradient (and, without a position list, the
// value and the moments) streams coalesced.  fp32 arithmetic, moments in
// fp32; the new value is rounded once to the value format.  Positions
// outside [0, nnz) are skipped.
#include "common.h"
#include "kernels.h"

namespace spops {
namespace {

constexpr int kBlock = 256;

template <typename VT>
__global__ __launch_bounds__(kBlock) void masked_adam_kernel(AdamArgs a) {
  const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (j >= a.ngrad) return;
  const int64_t i = a.positions ? (int64_t)a.positions[j] : j;
  if (i < 0 || i >= a.nnz) return;
  VT* val = (VT*)a.values;
  float g = to_f32(((const VT*)a.grad)[j]);
  if (a.maximize) g = -g;
  const float m = __builtin_fmaf(a.beta1, a.exp_avg[i], a.one_minus_beta1 * g);
  const float v = __builtin_fmaf(a.beta2, a.exp_avg_sq[i], a.one_minus_beta2 * (g * g));
  const float th = to_f32(val[i]) - a.alpha_t * (m / (__builtin_sqrtf(v) + a.eps));
  a.exp_avg[i] = m;
  a.exp_avg_sq[i] = v;
  val[i] = from_f32<VT>(th);
}

}  // namespace

hipError_t launch_masked_adam(const AdamArgs& a, int dtype, hipStream_t s) {
  if (a.ngrad <= 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(a.ngrad, kBlock));
  switch (dtype) {
    case kF32: hipLaunchKernelGGL(masked_adam_kernel<float>, grid, dim3(kBlock), 0, s, a); break;
    case kF16:
      hipLaunchKernelGGL(masked_adam_kernel<_Float16>, grid, dim3(kBlock), 0, s, a);
      break;
    case kBF16: hipLaunchKernelGGL(masked_adam_kernel<bf16_t>, grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace spops

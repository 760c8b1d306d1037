// Expert-bias update of "LongCat-Flash Technical Report" section 2.1.1,
// Eq.(2): for FFN expert i,
//   delta b_i = mu * ( K_e/K * 1/N  -  T_i / (K * T_all) ),
// and zero for the zero-computation experts (their share follows once every
// FFN expert sits at its target).  Binary64 arithmetic with exactly the
// operations below and no fused multiply-add, then one rounding to the fp32
// master bias, so the result is bitwise reproducible by any IEEE
// implementation of the same steps.
#include "zc_common.h"

#pragma clang fp contract(off)

namespace zc {
namespace {

__global__ void pid_kernel(int N, int K, const int32_t* __restrict__ counts, int64_t T_all,
                           double mu, double K_e, float* __restrict__ bias) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const double tgt = K_e / (static_cast<double>(K) * static_cast<double>(N));
  const double obs = static_cast<double>(counts[i]) / (static_cast<double>(K) * static_cast<double>(T_all));
  bias[i] = static_cast<float>(static_cast<double>(bias[i]) + mu * (tgt - obs));
}

}  // namespace

hipError_t launch_pid(int N, int K, const int32_t* counts, int64_t T_all, double mu, double K_e,
                      float* bias, hipStream_t s) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(pid_kernel, dim3((N + 255) / 256), dim3(256), 0, s, N, K, counts, T_all, mu,
                     K_e, bias);
  return hipGetLastError();
}

}  // namespace zc

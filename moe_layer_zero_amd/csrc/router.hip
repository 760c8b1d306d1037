// Router: routing keys, biased top-K and gates (one wavefront per token).
//
// "LongCat-Flash Technical Report", section 2.1, Eq.(1): the K experts of a
// token are the TopK of R(x_t)_i + b_i over all N+Z experts, and the gate of
// a picked expert is R(x_t)_i, the unbiased softmax.  Because a float value
// here decides an integer (the picked set), the keys are computed in
// binary64 by a fixed sequence of IEEE operations, so that any
// implementation of the same sequence picks the same experts bit for bit:
//   m    = max_j l_j                        (exact)
//   e_j  = exp(l_j - m)                     (key_exp below)
//   S    = sum of e_j: lane L of the wave sums e_j for j = L, L+64, ...
//          ascending from 0.0, then six rounds v = v + v[lane ^ o] for
//          o = 32, 16, 8, 4, 2, 1
//   key_j = e_j / S + (double)b_j
//   K rounds of "largest key, ties to the lower index"; slot r = round r.
//   gate_r = (float)(e_{s_r} / sum_{q<K} e_{s_q})  (renormalised, q ascending)
//          or (float)(e_{s_r} / S)                 (Eq.(1) as printed)
// This file is compiled with -ffp-contract=off and the pragma below, so no
// multiply-add is fused except the explicit fma calls.
#include "zc_common.h"

#pragma clang fp contract(off)

namespace zc {
namespace {

// ln 2 split for Cody-Waite reduction (W. J. Cody and W. Waite, "Software
// Manual for the Elementary Functions", 1980): head = ln 2 rounded to 32
// significant bits (2977044472 / 2^32), tail = ln 2 - head rounded to
// binary64; inv = 1/ln 2 rounded to binary64.
constexpr double kLn2Head = 0x1.62e42ff000000p-1;
constexpr double kLn2Tail = -0x1.718432a1b0e26p-35;
constexpr double kInvLn2 = 0x1.71547652b82fep+0;

// e^z for z <= 0: 0 below -700; otherwise z = k ln2 + r, e^r by its Taylor
// series to degree 13 (Horner, fused multiply-adds), times 2^k.
__device__ __forceinline__ double key_exp(double z) {
  if (z < -700.0) return 0.0;
  const double k = __builtin_rint(z * kInvLn2);
  const double r = (z - k * kLn2Head) - k * kLn2Tail;
  double p = 1.0 / 6227020800.0;                // 1/13!
  p = __builtin_fma(p, r, 1.0 / 479001600.0);   // 1/12!
  p = __builtin_fma(p, r, 1.0 / 39916800.0);    // 1/11!
  p = __builtin_fma(p, r, 1.0 / 3628800.0);     // 1/10!
  p = __builtin_fma(p, r, 1.0 / 362880.0);      // 1/9!
  p = __builtin_fma(p, r, 1.0 / 40320.0);       // 1/8!
  p = __builtin_fma(p, r, 1.0 / 5040.0);        // 1/7!
  p = __builtin_fma(p, r, 1.0 / 720.0);         // 1/6!
  p = __builtin_fma(p, r, 1.0 / 120.0);         // 1/5!
  p = __builtin_fma(p, r, 1.0 / 24.0);          // 1/4!
  p = __builtin_fma(p, r, 1.0 / 6.0);           // 1/3!
  p = __builtin_fma(p, r, 1.0 / 2.0);           // 1/2!
  p = __builtin_fma(p, r, 1.0);                 // 1/1!
  p = __builtin_fma(p, r, 1.0);                 // 1/0!
  return __builtin_ldexp(p, static_cast<int>(k));
}

// Is candidate (ka, ja) ahead of (kb, jb)?  Larger key first, then lower index.
__device__ __forceinline__ bool ahead(double ka, int ja, double kb, int jb) {
  return ka > kb || (ka == kb && ja < jb);
}

constexpr int kWavesPerBlock = 4;

// One wavefront per token; NPER = register slots per lane (E <= 64*NPER).
template <int NPER>
__global__ __launch_bounds__(64 * kWavesPerBlock) void topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int Tn, int E, int K,
    int gate_norm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const float* l = logits + static_cast<int64_t>(t) * E;

  double ev[NPER], kv[NPER];
  float lv[NPER];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int j = lane + 64 * i;
    lv[i] = j < E ? l[j] : -INFINITY;
    m = fmaxf(m, lv[i]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const double md = static_cast<double>(m);

  double part = 0.0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int j = lane + 64 * i;
    ev[i] = j < E ? key_exp(static_cast<double>(lv[i]) - md) : 0.0;
    if (j < E) part = part + ev[i];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part = part + __shfl_xor(part, o);
  const double S = part;

#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int j = lane + 64 * i;
    kv[i] = j < E ? ev[i] / S + static_cast<double>(bias[j]) : -INFINITY;
  }

  uint32_t taken = 0;
  int my_j = 0;
  double my_e = 0.0, den = 0.0;
  for (int r = 0; r < K; ++r) {
    double bk = -INFINITY, be = 0.0;
    int bj = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int j = lane + 64 * i;
      if (j < E && !((taken >> i) & 1u) && ahead(kv[i], j, bk, bj)) {
        bk = kv[i];
        bj = j;
        be = ev[i];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ok = __shfl_xor(bk, o);
      const int oj = __shfl_xor(bj, o);
      const double oe = __shfl_xor(be, o);
      if (ahead(ok, oj, bk, bj)) {
        bk = ok;
        bj = oj;
        be = oe;
      }
    }
    if ((bj & 63) == lane) taken |= 1u << (bj >> 6);
    den = den + be;
    if (lane == r) {
      my_j = bj;
      my_e = be;
    }
  }
  if (lane < K) {
    const double g = gate_norm ? my_e / den : my_e / S;
    const int64_t o = static_cast<int64_t>(t) * K + lane;
    topk_idx[o] = my_j;
    topk_gate[o] = static_cast<float>(g);
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, const float* bias, int Tn, int E, int K,
                       int gate_norm, int32_t* topk_idx, float* topk_gate, hipStream_t s) {
  if (Tn == 0) return hipSuccess;
  const dim3 grid((Tn + kWavesPerBlock - 1) / kWavesPerBlock), block(64 * kWavesPerBlock);
  const int nper = (E + 63) / 64;
#define ZC_TOPK(NP)                                                                      \
  hipLaunchKernelGGL((topk_kernel<NP>), grid, block, 0, s, logits, bias, Tn, E, K,      \
                     gate_norm, topk_idx, topk_gate)
  if (nper <= 1) ZC_TOPK(1);
  else if (nper <= 2) ZC_TOPK(2);
  else if (nper <= 4) ZC_TOPK(4);
  else if (nper <= 8) ZC_TOPK(8);
  else if (nper <= 12) ZC_TOPK(12);
  else ZC_TOPK(16);
#undef ZC_TOPK
  return hipGetLastError();
}

}  // namespace zc

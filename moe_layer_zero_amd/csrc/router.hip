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
//   key_j = e_j / S + (double)b_j, a NaN key taken as -infinity
//   K rounds of "largest key, ties to the lower index"; slot r = round r.
// A NaN score (or an infinite one, through inf - inf) makes every key of its
// token NaN; ordering NaN as -infinity keeps the selection total, so such a
// token picks experts 0..K-1 (valid indices) and gets NaN gates, which carry
// the NaN into its outputs and gradients.
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
  if (z != z) return z;  // NaN in, NaN out (no conversion of NaN to int below)
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

// Is candidate (ka, ja) ahead of (kb, jb)?  Larger key first, then lower
// index; evaluated without short-circuit branches.
__device__ __forceinline__ bool ahead_nb(double ka, int ja, double kb, int jb) {
  return static_cast<bool>(static_cast<int>(ka > kb) | (static_cast<int>(ka == kb) & static_cast<int>(ja < jb)));
}

constexpr int kWavesPerBlock = 4;

// The routing exponentials of one token for one wavefront: lane L holds
// e_j = key_exp(l_j - m) for j = L + 64 i (0 past E), and every lane gets S.
template <int NPER>
__device__ __forceinline__ void token_exps(const float* __restrict__ l, int E, int lane,
                                           double (&ev)[NPER], double& S) {
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
  S = part;
}

// One step of a wave-wide arg-max over (key, index) pairs: lane L compares
// its pair with the pair of the lane that the DPP control CTRL routes to it
// and keeps the one ahead.  The winner of a set of pairs is the same in
// whatever order they are compared (the order of ahead_nb is total), so the
// reduction can take the cheapest lane routes: in-row DPP moves, no LDS.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(double& bk, int& bj) {
  const uint64_t u = __builtin_bit_cast(uint64_t, bk);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF, false);
  const int oj = __builtin_amdgcn_update_dpp(0, bj, CTRL, 0xF, 0xF, false);
  const double ok = __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
  const bool take = ahead_nb(ok, oj, bk, bj);
  bk = take ? ok : bk;
  bj = take ? oj : bj;
}

// The same across the two 16-lane rows of each 32-lane half (swizzle, lane
// xor 16).
__device__ __forceinline__ void argmax_xor16(double& bk, int& bj) {
  constexpr int kPat = 0x1F | (0x10 << 10);  // bit mode: and 0x1F, or 0, xor 0x10
  const uint64_t u = __builtin_bit_cast(uint64_t, bk);
  const uint32_t lo = __builtin_amdgcn_ds_swizzle(static_cast<int>(u), kPat);
  const uint32_t hi = __builtin_amdgcn_ds_swizzle(static_cast<int>(u >> 32), kPat);
  const int oj = __builtin_amdgcn_ds_swizzle(bj, kPat);
  const double ok = __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
  const bool take = ahead_nb(ok, oj, bk, bj);
  bk = take ? ok : bk;
  bj = take ? oj : bj;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), l);
  return __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// One wavefront per token; NPER = register slots per lane (E <= 64*NPER).
// Each of the K rounds finds the untaken expert whose key is ahead of all
// others (larger key, then lower index): a lane's best over its slots, then
// the wave's best by DPP moves inside 16-lane rows (quad xor 1, quad xor 2,
// half-row mirror, row mirror), a swizzle across rows and the two halves
// read as scalars; the winner's e_j is then read from its lane.
template <int NPER>
__global__ __launch_bounds__(64 * kWavesPerBlock) void topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int Tn, int E, int K,
    int gate_norm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const float* l = logits + static_cast<int64_t>(t) * E;

  double ev[NPER], kv[NPER], S;
  token_exps<NPER>(l, E, lane, ev, S);

#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int j = lane + 64 * i;
    kv[i] = j < E ? ev[i] / S + static_cast<double>(bias[j]) : -INFINITY;
    if (kv[i] != kv[i]) kv[i] = -INFINITY;
  }

  uint32_t taken = 0;  // slots of this lane already picked (or past E)
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (lane + 64 * i >= E) taken |= 1u << i;
  int my_j = 0;
  double my_e = 0.0, den = 0.0;
  for (int r = 0; r < K; ++r) {
    // this lane's best untaken slot, with its e_j
    double bk = -INFINITY, be_l = 0.0;
    int bj = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int j = lane + 64 * i;
      const bool take = static_cast<bool>(static_cast<int>(((taken >> i) & 1u) == 0u) &
                                          static_cast<int>(ahead_nb(kv[i], j, bk, bj)));
      bk = take ? kv[i] : bk;
      bj = take ? j : bj;
      be_l = take ? ev[i] : be_l;
    }
    argmax_dpp<0xB1>(bk, bj);   // quad_perm [1,0,3,2]: lane xor 1
    argmax_dpp<0x4E>(bk, bj);   // quad_perm [2,3,0,1]: lane xor 2
    argmax_dpp<0x141>(bk, bj);  // row_half_mirror: lane i <-> 7 - i in each 8
    argmax_dpp<0x140>(bk, bj);  // row_mirror: lane i <-> 15 - i in each 16
    argmax_xor16(bk, bj);
    {
      const double k0 = readlane_f64(bk, 0), k1 = readlane_f64(bk, 32);
      const int j0 = __builtin_amdgcn_readlane(bj, 0), j1 = __builtin_amdgcn_readlane(bj, 32);
      const bool second = ahead_nb(k1, j1, k0, j0);
      bj = second ? j1 : j0;
    }
    // bj is wave-uniform and below E (at most E picks are made, K <= E); the
    // lane holding it has it as its own best, with its e_j
    const int ws = bj >> 6, wl = bj & 63;
    const double be = readlane_f64(be_l, wl);
    if (wl == lane) taken |= 1u << ws;
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


// ------------------------------------------------------------------------
// Device-level load-balance loss, "LongCat-Flash Technical Report", section
// 2.1.2: L = alpha * sum_j f_j P_j over D groups of G = N/D consecutive FFN
// experts plus one group holding every zero-computation expert.  P_j
// (Eq.(4)) is the group's softmax mass averaged over the T tokens, f_j
// (Eq.(5)) the number of picks that land in the group times D/(K_e T), or
// 1/((K-K_e) T) for the extra group (left out when Z = 0).  The softmax is
// the routing one above (binary64), so P follows the same R the picks saw.
//
// lb_colsum_kernel: wave w of block b walks tokens b*4+w, b*4+w+4*nblk, ...
//   ascending, adding each token's e_j / S to a binary64 register per
//   expert; the block adds its four waves in wave order into part[b][E].
// lb_reduce_kernel: col[j] = part[0..nblk)[j], four consecutive quarters
//   of b (one per wave, ascending) added in wave order.
// lb_finish_kernel: per group, col and counts summed over ascending j;
//   out = [L, f_1..f_{D+1}, P_1..P_{D+1}]; L summed over the groups in a
//   fixed tree.  Every order is fixed, so the result is reproducible.
template <int NPER>
__global__ __launch_bounds__(64 * kWavesPerBlock) void lb_colsum_kernel(
    const float* __restrict__ logits, int Tn, int E, double* __restrict__ part) {
  __shared__ double s_col[kWavesPerBlock][64 * NPER];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double col[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) col[i] = 0.0;
  for (int t = blockIdx.x * kWavesPerBlock + w; t < Tn; t += gridDim.x * kWavesPerBlock) {
    double ev[NPER], S;
    token_exps<NPER>(logits + static_cast<int64_t>(t) * E, E, lane, ev, S);
#pragma unroll
    for (int i = 0; i < NPER; ++i) col[i] = col[i] + ev[i] / S;
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) s_col[w][lane + 64 * i] = col[i];
  __syncthreads();
  for (int j = threadIdx.x; j < E; j += 64 * kWavesPerBlock)
    part[static_cast<int64_t>(blockIdx.x) * E + j] =
        ((s_col[0][j] + s_col[1][j]) + s_col[2][j]) + s_col[3][j];
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void lb_reduce_kernel(
    const double* __restrict__ part, int nblk, int E, double* __restrict__ col) {
  __shared__ double s_r[kWavesPerBlock][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int q = (nblk + kWavesPerBlock - 1) / kWavesPerBlock;
  const int b1 = min(nblk, (w + 1) * q);
  double v = 0.0;
  if (j < E)
    for (int b = w * q; b < b1; ++b) v = v + part[static_cast<int64_t>(b) * E + j];
  s_r[w][lane] = v;
  __syncthreads();
  if (w == 0 && j < E) col[j] = ((s_r[0][lane] + s_r[1][lane]) + s_r[2][lane]) + s_r[3][lane];
}

// Pick frequency f_g of group g (D/(K_e T) or 1/((K-K_e) T) times the
// group's picks), from the per-expert pick counts.
__device__ __forceinline__ double lb_freq(const int32_t* __restrict__ counts, int g, int G, int N,
                                          int E, int D, int K, double K_e, int Tn) {
  const int lo = g < D ? g * G : N, hi = g < D ? lo + G : E;
  int64_t c = 0;
  for (int j = lo; j < hi; ++j) c += counts[j];
  if (g < D) return static_cast<double>(D) / (K_e * static_cast<double>(Tn)) * static_cast<double>(c);
  if (E == N) return 0.0;
  return 1.0 / ((static_cast<double>(K) - K_e) * static_cast<double>(Tn)) * static_cast<double>(c);
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void lb_finish_kernel(
    const double* __restrict__ col, const int32_t* __restrict__ counts, int Tn, int N, int E,
    int K, int D, double K_e, double alpha, double* __restrict__ out) {
  __shared__ double s_red[kWavesPerBlock];
  const int ng = D + 1, G = N / D;
  double acc = 0.0;
  for (int g = threadIdx.x; g < ng; g += 64 * kWavesPerBlock) {
    double f = 0.0, P = 0.0;
    if (Tn > 0) {
      const int lo = g < D ? g * G : N, hi = g < D ? lo + G : E;
      double p = 0.0;
      for (int j = lo; j < hi; ++j) p = p + col[j];
      P = p / static_cast<double>(Tn);
      f = lb_freq(counts, g, G, N, E, D, K, K_e, Tn);
    }
    out[1 + g] = f;
    out[1 + ng + g] = P;
    acc = acc + f * P;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = alpha * (((s_red[0] + s_red[1]) + s_red[2]) + s_red[3]);
}

// Per-expert coefficient of the loss's score gradient,
// c_j = (float)(alpha * f_{g(j)} / T): dL/dl_{t,j} = R_{t,j} (c_j - sum_k R_{t,k} c_k).
__global__ __launch_bounds__(64 * kWavesPerBlock) void lb_coef_kernel(
    const int32_t* __restrict__ counts, int Tn, int N, int E, int K, int D, double K_e,
    double alpha, float* __restrict__ coef) {
  __shared__ double s_f[kMaxExperts + 1];
  const int ng = D + 1, G = N / D;
  for (int g = threadIdx.x; g < ng; g += 64 * kWavesPerBlock)
    s_f[g] = Tn > 0 ? lb_freq(counts, g, G, N, E, D, K, K_e, Tn) : 0.0;
  __syncthreads();
  for (int j = threadIdx.x; j < E; j += 64 * kWavesPerBlock) {
    const double f = s_f[j < N ? j / G : D];
    coef[j] = Tn > 0 ? static_cast<float>(alpha * f / static_cast<double>(Tn)) : 0.f;
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

int lb_blocks(int64_t Tn) {
  const int64_t b = (Tn + 31) / 32;
  return static_cast<int>(b < 1 ? 1 : (b > 256 ? 256 : b));
}

size_t lb_scratch_bytes(int64_t Tn, int64_t E) {
  return static_cast<size_t>(lb_blocks(Tn) + 1) * static_cast<size_t>(E) * sizeof(double);
}

hipError_t launch_lb_loss(const float* logits, const int32_t* counts, int Tn, int N, int E, int K,
                          int D, double K_e, double alpha, double* out, void* scratch,
                          hipStream_t s) {
  const int nblk = lb_blocks(Tn);
  double* part = static_cast<double*>(scratch);
  double* col = part + static_cast<int64_t>(nblk) * E;
  const dim3 block(64 * kWavesPerBlock);
  if (Tn > 0) {
    const int nper = (E + 63) / 64;
#define ZC_LBC(NP) \
  hipLaunchKernelGGL((lb_colsum_kernel<NP>), dim3(nblk), block, 0, s, logits, Tn, E, part)
    if (nper <= 1) ZC_LBC(1);
    else if (nper <= 2) ZC_LBC(2);
    else if (nper <= 4) ZC_LBC(4);
    else if (nper <= 8) ZC_LBC(8);
    else if (nper <= 12) ZC_LBC(12);
    else ZC_LBC(16);
#undef ZC_LBC
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lb_reduce_kernel, dim3((E + 63) / 64), block, 0, s, part, nblk, E, col);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lb_finish_kernel, dim3(1), block, 0, s, col, counts, Tn, N, E, K, D, K_e,
                     alpha, out);
  return hipGetLastError();
}

hipError_t launch_lb_coef(const int32_t* counts, int Tn, int N, int E, int K, int D, double K_e,
                          double alpha, float* coef, hipStream_t s) {
  hipLaunchKernelGGL(lb_coef_kernel, dim3(1), dim3(64 * kWavesPerBlock), 0, s, counts, Tn, N, E, K,
                     D, K_e, alpha, coef);
  return hipGetLastError();
}

}  // namespace zc

// Weighted combine with the zero-computation experts folded in, and the
// token-side pieces of the backward pass.
//
// "LongCat-Flash Technical Report", section 2.1: the layer output is
// sum_i g_i E_i(x_t) with E_i(x_t) = x_t for the zero-computation experts,
// so those experts reduce to one scalar per token,
//   c_t = sum of the gates of the token's zero-computation picks,
// and the output is c_t x_t + sum over FFN picks of g_r y_r.  Every sum runs
// in slot order in fp32, one workgroup per token, so results do not depend
// on scheduling (no atomics).  Inputs and outputs are in the layer dtype;
// y rows are found through the inverse dispatch map.
#include "zc_common.h"

namespace zc {
namespace {

constexpr int kThreads = 256;
constexpr int kCombineMaxThreads = 1024;
constexpr int kMaxK = 32;

// 16-byte vector of the layer dtype, widened to fp32.
template <typename T> struct V16;
template <> struct V16<bf16_t> {
  static constexpr int n = 8;
  typedef u32x4_t raw_t;  // the 16 bytes as loaded
  static __device__ __forceinline__ raw_t ld_raw(const bf16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
  }
  // for data read exactly once (the expert output rows)
  static __device__ __forceinline__ raw_t ld_raw_once(const bf16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  }
  static __device__ __forceinline__ void unpack(const raw_t& v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(v[e] << 16);
      f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load(const bf16_t* p, float* f) { unpack(ld_raw(p), f); }
  static __device__ __forceinline__ void store(bf16_t* p, const float* f) {
    u32x4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = static_cast<uint32_t>(f2bf(f[2 * e])) | (static_cast<uint32_t>(f2bf(f[2 * e + 1])) << 16);
    *reinterpret_cast<u32x4_t*>(p) = v;
  }
};
template <> struct V16<float> {
  static constexpr int n = 4;
  typedef f32x4_t raw_t;
  static __device__ __forceinline__ raw_t ld_raw(const float* p) {
    return *reinterpret_cast<const f32x4_t*>(p);
  }
  static __device__ __forceinline__ raw_t ld_raw_once(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  }
  static __device__ __forceinline__ void unpack(const raw_t& v, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = v[e];
  }
  static __device__ __forceinline__ void load(const float* p, float* f) { unpack(ld_raw(p), f); }
  static __device__ __forceinline__ void store(float* p, const float* f) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{f[0], f[1], f[2], f[3]};
  }
};

// V consecutive fp32 values (V = 4 or 8, 16-byte aligned).
template <int V>
__device__ __forceinline__ void load_f32_n(const float* p, float* f) {
#pragma unroll
  for (int c = 0; c < V / 4; ++c) {
    const f32x4_t v = reinterpret_cast<const f32x4_t*>(p)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * c + e] = v[e];
  }
}

// Token's picks into LDS; returns c_t (sum of zero-computation gates).
__device__ __forceinline__ float load_picks(const int32_t* topk_idx, const float* gate,
                                            const int32_t* inv, int64_t t, int N, int K,
                                            float* s_g, int32_t* s_inv, float* s_c) {
  if (threadIdx.x < K) {
    const int64_t o = t * K + threadIdx.x;
    const int e = topk_idx[o];
    s_g[threadIdx.x] = gate[o];
    s_inv[threadIdx.x] = e < N ? inv[o] : -1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float c = 0.f;
    for (int r = 0; r < K; ++r)
      if (s_inv[r] < 0) c += s_g[r];
    *s_c = c;
  }
  __syncthreads();
  return *s_c;
}

// G: picks whose row loads are issued together (4, 8, 12 or 16; the
// smallest covering K, so a token's rows are in flight at once).  The
// workgroup has one thread per 16-byte piece of a row (at most 1024), so
// at the usual widths a token's loads all go out in one pass.
template <typename T, int G>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(
    const T* __restrict__ x, const T* __restrict__ y, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ gate, const int32_t* __restrict__ inv, int d, int N, int K,
    float out_scale, T* __restrict__ out) {
  __shared__ float s_g[kMaxK];
  __shared__ int32_t s_inv[kMaxK];
  __shared__ float s_c;
  const int64_t t = blockIdx.x;
  const float c = load_picks(topk_idx, gate, inv, t, N, K, s_g, s_inv, &s_c);
  constexpr int V = V16<T>::n;
  for (int j = threadIdx.x * V; j < d; j += blockDim.x * V) {
    float acc[V], v[V];
    V16<T>::load(x + t * d + j, v);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = c * v[e];
    // picks in groups of G: the group's row loads are issued together,
    // then added in slot order
    for (int r0 = 0; r0 < K; r0 += G) {
      // (a slot past K or of a zero-computation pick loads nothing and is
      // skipped below; each y row is read by its one token only, so its
      // loads carry the non-temporal hint)
      typename V16<T>::raw_t w[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int q = r0 + u < K ? s_inv[r0 + u] : -1;
        w[u] = q >= 0 ? V16<T>::ld_raw_once(y + static_cast<int64_t>(q) * d + j) : typename V16<T>::raw_t{};
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (r0 + u >= K || s_inv[r0 + u] < 0) continue;
        const float g = s_g[r0 + u];
        V16<T>::unpack(w[u], v);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += g * v[e];
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] *= out_scale;
    V16<T>::store(out + t * d + j, acc);
  }
}

// Fixed-order block sum of one value per thread (wave butterflies, then the
// four wave results in order).  All threads get the result.
__device__ __forceinline__ float block_sum(float v, float* s_red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

// Backward of the combine for one token (one workgroup):
//   dg_r = <out_scale * dout_t, y_r> for FFN picks, <out_scale * dout_t, x_t>
//          for zero-computation picks (fixed-order block sums);
//   gs[inv] = out_scale * g_r, the row scale the expert GEMMs apply;
//   dl = gradient of the router scores through the gates: the softmax
//        Jacobian restricted to the picks (renormalised gates) or over all
//        experts (Eq.(1) gates), written as one fp32 row of width ldl;
//        with lbc, plus the device-level load-balance loss's gradient
//        p_j (lbc_j - sum_k p_k lbc_k) (section 2.1.2, f held fixed).
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(
    const T* __restrict__ x, const T* __restrict__ y, const T* __restrict__ dout,
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ gate, const int32_t* __restrict__ inv, int d, int N, int E, int K,
    int gate_norm, float out_scale, const float* __restrict__ lbc, float* __restrict__ gs,
    float* __restrict__ dg_out, float* __restrict__ dl, int ldl) {
  __shared__ float s_g[kMaxK];
  __shared__ int32_t s_inv[kMaxK];
  __shared__ int32_t s_e[kMaxK];
  __shared__ float s_dg[kMaxK];
  __shared__ float s_c;
  __shared__ float s_red[4];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) s_e[threadIdx.x] = topk_idx[t * K + threadIdx.x];
  load_picks(topk_idx, gate, inv, t, N, K, s_g, s_inv, &s_c);
  if (threadIdx.x < K && s_inv[threadIdx.x] >= 0) gs[s_inv[threadIdx.x]] = out_scale * s_g[threadIdx.x];
  constexpr int V = V16<T>::n;
  // picks in groups of four: one pass over dout for the group, the four
  // rows' loads issued together; each pick's partial sum runs over j in the
  // same order as a pass of its own would
  for (int r0 = 0; r0 < K; r0 += 4) {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    const T* src[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = r0 + u < K ? s_inv[r0 + u] : -1;
      src[u] = q >= 0 ? y + static_cast<int64_t>(q) * d : x + t * d;
    }
    for (int j = threadIdx.x * V; j < d; j += kThreads * V) {
      float dv[V], v[V];
      typename V16<T>::raw_t w[4];
      V16<T>::load(dout + t * d + j, dv);
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = V16<T>::ld_raw(src[u] + j);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        V16<T>::unpack(w[u], v);
#pragma unroll
        for (int e = 0; e < V; ++e) part[u] += (out_scale * dv[e]) * v[e];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r0 + u >= K) break;
      const float tot = block_sum(part[u], s_red);
      if (threadIdx.x == 0) s_dg[r0 + u] = tot;
    }
  }
  __syncthreads();
  if (threadIdx.x < K) dg_out[t * K + threadIdx.x] = s_dg[threadIdx.x];
  float sgd = 0.f;
  for (int r = 0; r < K; ++r) sgd += s_g[r] * s_dg[r];
  float* dlr = dl + t * ldl;
  if (gate_norm && !lbc) {
    for (int j = threadIdx.x; j < ldl; j += kThreads) dlr[j] = 0.f;
    __syncthreads();
    if (threadIdx.x < K) dlr[s_e[threadIdx.x]] = s_g[threadIdx.x] * (s_dg[threadIdx.x] - sgd);
    return;
  }
  // the full softmax p of the token's scores
  const float* l = logits + t * E;
  float m = -INFINITY;
  for (int j = threadIdx.x; j < E; j += kThreads) m = fmaxf(m, l[j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float part = 0.f;
  for (int j = threadIdx.x; j < E; j += kThreads) part += __expf(l[j] - m);
  const float S = block_sum(part, s_red);
  float sc = 0.f;
  if (lbc) {
    part = 0.f;
    for (int j = threadIdx.x; j < E; j += kThreads) part += (__expf(l[j] - m) / S) * lbc[j];
    sc = block_sum(part, s_red);
  }
  for (int j = threadIdx.x; j < ldl; j += kThreads) {
    float v = 0.f;
    if (j < E) {
      const float pj = __expf(l[j] - m) / S;
      int r = -1;
      for (int q = 0; q < K; ++q)
        if (s_e[q] == j) r = q;
      if (gate_norm)
        v = r >= 0 ? s_g[r] * (s_dg[r] - sgd) : 0.f;
      else
        v = pj * ((r >= 0 ? s_dg[r] : 0.f) - sgd);
      if (lbc) v += pj * (lbc[j] - sc);
    }
    dlr[j] = v;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dx_gather_kernel(
    const T* __restrict__ dout, const float* __restrict__ dxp, const float* __restrict__ dxr,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ gate,
    const int32_t* __restrict__ inv, int d, int N, int K, float out_scale, T* __restrict__ dx) {
  __shared__ float s_g[kMaxK];
  __shared__ int32_t s_inv[kMaxK];
  __shared__ float s_c;
  const int64_t t = blockIdx.x;
  const float c = load_picks(topk_idx, gate, inv, t, N, K, s_g, s_inv, &s_c) * out_scale;
  constexpr int V = V16<T>::n;
  auto load_f32 = [](const float* p, float* f) { load_f32_n<V>(p, f); };
  for (int j = threadIdx.x * V; j < d; j += kThreads * V) {
    float acc[V], v[V];
    V16<T>::load(dout + t * d + j, v);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = c * v[e];
    for (int r0 = 0; r0 < K; r0 += 4) {  // as in the combine: loads of four picks together
      // (a slot past K or of a zero-computation pick loads the token's own
      // router-dx piece, read below anyway, and is skipped)
      float w[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = r0 + u < K ? s_inv[r0 + u] : -1;
        load_f32(q >= 0 ? dxp + static_cast<int64_t>(q) * d + j : dxr + t * d + j, w[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (r0 + u >= K || s_inv[r0 + u] < 0) continue;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += w[u][e];
      }
    }
    load_f32(dxr + t * d + j, v);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] += v[e];
    V16<T>::store(dx + t * d + j, acc);
  }
}

// Workgroup size of the combine: one thread per V-element piece of a row of
// d, a multiple of 64 between 64 and kCombineMaxThreads.
int combine_threads(int d, int V) {
  const int pieces = (d + V - 1) / V;
  return pieces < 64 ? 64 : (pieces > kCombineMaxThreads ? kCombineMaxThreads : (pieces + 63) / 64 * 64);
}

}  // namespace

template <typename T>
hipError_t launch_combine(const T* x, const T* y, const int32_t* topk_idx, const float* gate,
                          const int32_t* inv, int Tn, int d, int N, int K, float out_scale, T* out,
                          hipStream_t s) {
  if (Tn == 0) return hipSuccess;
  const int threads = combine_threads(d, V16<T>::n);
#define ZC_COMBINE(G)                                                                      \
  hipLaunchKernelGGL((combine_kernel<T, G>), dim3(Tn), dim3(threads), 0, s, x, y, topk_idx, \
                     gate, inv, d, N, K, out_scale, out)
  if (K <= 4) ZC_COMBINE(4);
  else if (K <= 8) ZC_COMBINE(8);
  else if (K <= 12) ZC_COMBINE(12);
  else ZC_COMBINE(16);
#undef ZC_COMBINE
  return hipGetLastError();
}

template <typename T>
hipError_t launch_combine_bwd(const T* x, const T* y, const T* dout, const float* logits,
                              const int32_t* topk_idx, const float* gate, const int32_t* inv,
                              int Tn, int d, int N, int E, int K, int gate_norm, float out_scale,
                              const float* lb_coef, float* gs, float* dg, float* dl, int ldl,
                              hipStream_t s) {
  if (Tn == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_bwd_kernel<T>, dim3(Tn), dim3(kThreads), 0, s, x, y, dout, logits,
                     topk_idx, gate, inv, d, N, E, K, gate_norm, out_scale, lb_coef, gs, dg, dl,
                     ldl);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dx_gather(const T* dout, const float* dxp, const float* dxr, const int32_t* topk_idx,
                            const float* gate, const int32_t* inv, int Tn, int d, int N, int K,
                            float out_scale, T* dx, hipStream_t s) {
  if (Tn == 0) return hipSuccess;
  hipLaunchKernelGGL(dx_gather_kernel<T>, dim3(Tn), dim3(kThreads), 0, s, dout, dxp, dxr, topk_idx,
                     gate, inv, d, N, K, out_scale, dx);
  return hipGetLastError();
}

#define ZC_INST(T)                                                                              \
  template hipError_t launch_combine<T>(const T*, const T*, const int32_t*, const float*,       \
                                        const int32_t*, int, int, int, int, float, T*,          \
                                        hipStream_t);                                           \
  template hipError_t launch_combine_bwd<T>(const T*, const T*, const T*, const float*,         \
                                            const int32_t*, const float*, const int32_t*, int,  \
                                            int, int, int, int, int, float, const float*,       \
                                            float*, float*, float*, int, hipStream_t);          \
  template hipError_t launch_dx_gather<T>(const T*, const float*, const float*, const int32_t*, \
                                          const float*, const int32_t*, int, int, int, int,     \
                                          float, T*, hipStream_t);
ZC_INST(bf16_t)
ZC_INST(float)
#undef ZC_INST

}  // namespace zc

// Dispatch: per-expert token counts (the T_i of Eq.(2), "LongCat-Flash
// Technical Report" section 2.1.1), their prefix sum over the FFN experts,
// and the canonical dispatch order perm = FFN picks sorted by
// (expert, token), with its inverse.
//
// Each token picks an expert at most once, so (expert, token) keys are
// unique and a stable order needs no sort: tokens are cut into blocks of 64;
// a block records, per expert, the 64-bit mask of its tokens that picked the
// expert.  The rank of a pick inside its expert's segment is then
//   (picks of that expert in earlier blocks) + popcount(mask & lower tokens),
// which is exact integer work with no atomics on the order.
#include "zc_common.h"

namespace zc {
namespace {

constexpr int kTokPerBlk = 64;
constexpr int kThreads = 256;

struct Scratch {
  uint64_t* mask;  // [nblk][E]
  int32_t* cnt;    // [nblk][E]
  int32_t* base;   // [nblk][E]
};

__host__ __device__ inline int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

Scratch carve(void* p, int64_t nblk, int64_t E) {
  char* c = static_cast<char*>(p);
  Scratch s;
  s.mask = reinterpret_cast<uint64_t*>(c);
  c += align256(nblk * E * 8);
  s.cnt = reinterpret_cast<int32_t*>(c);
  c += align256(nblk * E * 4);
  s.base = reinterpret_cast<int32_t*>(c);
  return s;
}

__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ topk_idx,
                                                        int Tn, int E, int K, uint64_t* mask,
                                                        int32_t* cnt) {
  extern __shared__ uint64_t smask[];
  const int b = blockIdx.x;
  const int t0 = b * kTokPerBlk;
  const int nt = min(kTokPerBlk, Tn - t0);
  for (int e = threadIdx.x; e < E; e += kThreads) smask[e] = 0;
  __syncthreads();
  const int n = nt * K;
  const int32_t* idx = topk_idx + static_cast<int64_t>(t0) * K;
  for (int i = threadIdx.x; i < n; i += kThreads)
    atomicOr(reinterpret_cast<unsigned long long*>(&smask[idx[i]]), 1ull << (i / K));
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const uint64_t m = smask[e];
    mask[static_cast<int64_t>(b) * E + e] = m;
    cnt[static_cast<int64_t>(b) * E + e] = __popcll(m);
  }
}

// One block of 1024 threads (E <= 1024): counts, offsets, tile prefix and
// per-(block, expert) bases.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ cnt, int nblk,
                                                    int E, int N, int bm, int bm2,
                                                    int32_t* counts, int32_t* offsets,
                                                    int32_t* tile_off, int32_t* tile_off2,
                                                    int32_t* tile_exp, int32_t* tile_exp1,
                                                    int32_t* sched, int32_t* base) {
  __shared__ int32_t s_off[1024];
  __shared__ int32_t s_til[1024];
  __shared__ int32_t s_til2[1024];
  const int e = threadIdx.x;
  int32_t tot = 0;
  // unrolled so that each thread keeps 16 independent loads in flight
  if (e < E) {
#pragma unroll 16
    for (int b = 0; b < nblk; ++b) tot += cnt[static_cast<int64_t>(b) * E + e];
  }
  if (e < E) counts[e] = tot;
  // inclusive scans over FFN experts (Hillis-Steele; integer, order-free)
  s_off[e] = (e < N) ? tot : 0;
  s_til[e] = (e < N) ? (tot + bm - 1) / bm : 0;
  s_til2[e] = (e < N) ? (tot + bm2 - 1) / bm2 : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t a = e >= o ? s_off[e - o] : 0;
    const int32_t c = e >= o ? s_til[e - o] : 0;
    const int32_t c2 = e >= o ? s_til2[e - o] : 0;
    __syncthreads();
    s_off[e] += a;
    s_til[e] += c;
    s_til2[e] += c2;
    __syncthreads();
  }
  const int32_t excl = (e > 0 && e <= N) ? s_off[e - 1] : 0;
  if (e < N) {
    offsets[e] = excl;
    tile_off[e] = e > 0 ? s_til[e - 1] : 0;
    tile_off2[e] = e > 0 ? s_til2[e - 1] : 0;
  }
  if (e == 0) {
    offsets[N] = N > 0 ? s_off[N - 1] : 0;
    tile_off[N] = N > 0 ? s_til[N - 1] : 0;
    tile_off2[N] = N > 0 ? s_til2[N - 1] : 0;
  }
  if (sched && e < kSchedInts) sched[e] = 0;
  // expert of every bm2-row tile, so a GEMM tile finds its expert in one load
  if (tile_exp && e < N) {
    const int32_t t1 = s_til2[e], t0 = e > 0 ? s_til2[e - 1] : 0;
    for (int32_t t = t0; t < t1; ++t) tile_exp[t] = e;
  }
  // and of every bm-row tile
  if (tile_exp1 && e < N) {
    const int32_t t1 = s_til[e], t0 = e > 0 ? s_til[e - 1] : 0;
    for (int32_t t = t0; t < t1; ++t) tile_exp1[t] = e;
  }
  if (e < N) {
    int32_t run = excl;
#pragma unroll 16
    for (int b = 0; b < nblk; ++b) {
      const int64_t o = static_cast<int64_t>(b) * E + e;
      base[o] = run;
      run += cnt[o];
    }
  }
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                           int Tn, int E, int N, int K,
                                                           const uint64_t* __restrict__ mask,
                                                           const int32_t* __restrict__ base,
                                                           int32_t* perm, int32_t* inv) {
  extern __shared__ uint64_t smask[];
  const int b = blockIdx.x;
  const int t0 = b * kTokPerBlk;
  const int nt = min(kTokPerBlk, Tn - t0);
  for (int e = threadIdx.x; e < E; e += kThreads) smask[e] = mask[static_cast<int64_t>(b) * E + e];
  __syncthreads();
  const int n = nt * K;
  const int64_t s0 = static_cast<int64_t>(t0) * K;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int e = topk_idx[s0 + i];
    if (e >= N) {
      inv[s0 + i] = -1;
      continue;
    }
    const int tl = i / K;
    const uint64_t below = tl == 0 ? 0ull : (smask[e] & ((1ull << tl) - 1ull));
    const int32_t pos = base[static_cast<int64_t>(b) * E + e] + __popcll(below);
    perm[pos] = static_cast<int32_t>(s0 + i);
    inv[s0 + i] = pos;
  }
}

// Row-tile prefixes from offsets alone: tile_off for bm-row tiles and, if
// tile_off2 is set, tile_off2 for bm2-row tiles with the expert of each of
// those tiles (tile_exp2); zeroes the nsched (<= 1024) counters of sched if set.
__global__ __launch_bounds__(1024) void tile_off_kernel(const int32_t* __restrict__ offsets, int N,
                                                       int bm, int32_t* tile_off, int bm2,
                                                       int32_t* tile_off2, int32_t* tile_exp2,
                                                       int32_t* sched, int nsched) {
  __shared__ int32_t s_til[1024];
  __shared__ int32_t s_til2[1024];
  const int e = threadIdx.x;
  const int32_t rows = e < N ? offsets[e + 1] - offsets[e] : 0;
  const int32_t w = (rows + bm - 1) / bm;
  const int32_t w2 = tile_off2 ? (rows + bm2 - 1) / bm2 : 0;
  s_til[e] = w;
  s_til2[e] = w2;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t c = e >= o ? s_til[e - o] : 0;
    const int32_t c2 = e >= o ? s_til2[e - o] : 0;
    __syncthreads();
    s_til[e] += c;
    s_til2[e] += c2;
    __syncthreads();
  }
  if (e < N) tile_off[e] = s_til[e] - w;
  if (e == 0) tile_off[N] = N > 0 ? s_til[N - 1] : 0;
  if (tile_off2) {
    if (e < N) tile_off2[e] = s_til2[e] - w2;
    if (e == 0) tile_off2[N] = N > 0 ? s_til2[N - 1] : 0;
    if (e < N)
      for (int32_t t = s_til2[e] - w2; t < s_til2[e]; ++t) tile_exp2[t] = e;
  }
  if (sched && e < nsched) sched[e] = 0;
}


// Budget-control telemetry (section 2.1.1 of the report tracks the mean and
// the standard deviation of the FFN experts each token activates, Fig.3b/c).
// stats_partial_kernel: each block histograms n_t = (FFN picks of token t)
// over its grid-stride share of the tokens (LDS integer atomics: the
// counts do not depend on their order) into part[b][K+1].
// stats_finish_kernel: hist[k] = sum over blocks; mean = sum_k k hist[k] / T
// (an exact integer sum, one division); std = sqrt(sum_k hist[k] (k - mean)^2 / T).
__global__ __launch_bounds__(kThreads) void stats_partial_kernel(
    const int32_t* __restrict__ topk_idx, int Tn, int N, int K, int32_t* __restrict__ part) {
  __shared__ int32_t s_h[33];
  if (threadIdx.x <= K) s_h[threadIdx.x] = 0;
  __syncthreads();
  for (int t = blockIdx.x * kThreads + threadIdx.x; t < Tn; t += gridDim.x * kThreads) {
    const int32_t* row = topk_idx + static_cast<int64_t>(t) * K;
    int c = 0;
    for (int r = 0; r < K; ++r) c += row[r] < N ? 1 : 0;
    atomicAdd(&s_h[c], 1);
  }
  __syncthreads();
  if (threadIdx.x <= K) part[blockIdx.x * (K + 1) + threadIdx.x] = s_h[threadIdx.x];
}

__global__ __launch_bounds__(64) void stats_finish_kernel(const int32_t* __restrict__ part,
                                                          int nblk, int Tn, int K,
                                                          int32_t* __restrict__ hist,
                                                          double* __restrict__ moments) {
  __shared__ int32_t s_h[33];
  const int k = threadIdx.x;
  if (k <= K) {
    int32_t h = 0;
    for (int b = 0; b < nblk; ++b) h += part[b * (K + 1) + k];
    s_h[k] = h;
    hist[k] = h;
  }
  __syncthreads();
  if (k == 0) {
    double mean = 0.0, var = 0.0;
    if (Tn > 0) {
      int64_t sum = 0;
      for (int j = 0; j <= K; ++j) sum += static_cast<int64_t>(j) * s_h[j];
      mean = static_cast<double>(sum) / static_cast<double>(Tn);
      for (int j = 0; j <= K; ++j) {
        const double dv = static_cast<double>(j) - mean;
        var += static_cast<double>(s_h[j]) * (dv * dv);
      }
      var /= static_cast<double>(Tn);
    }
    moments[0] = mean;
    moments[1] = sqrt(var);
  }
}

__global__ __launch_bounds__(kThreads) void accumulate_kernel(const int32_t* __restrict__ counts,
                                                              int E, int32_t* __restrict__ acc) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < E) acc[i] += counts[i];
}

}  // namespace

int stats_blocks(int64_t Tn) {
  const int64_t b = (Tn + kThreads - 1) / kThreads;
  return static_cast<int>(b < 1 ? 1 : (b > 256 ? 256 : b));
}

size_t stats_scratch_bytes(int64_t Tn, int64_t K) {
  return static_cast<size_t>(stats_blocks(Tn)) * static_cast<size_t>(K + 1) * sizeof(int32_t);
}

hipError_t launch_route_stats(const int32_t* topk_idx, int Tn, int N, int K, int32_t* hist,
                              double* moments, void* scratch, hipStream_t s) {
  const int nblk = Tn > 0 ? stats_blocks(Tn) : 0;
  int32_t* part = static_cast<int32_t*>(scratch);
  if (nblk > 0) {
    hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(kThreads), 0, s, topk_idx, Tn, N, K,
                       part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(stats_finish_kernel, dim3(1), dim3(64), 0, s, part, nblk, Tn, K, hist,
                     moments);
  return hipGetLastError();
}

hipError_t launch_accumulate_counts(const int32_t* counts, int E, int32_t* acc, hipStream_t s) {
  hipLaunchKernelGGL(accumulate_kernel, dim3((E + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                     counts, E, acc);
  return hipGetLastError();
}

hipError_t launch_tile_offsets(const int32_t* offsets, int N, int bm, int32_t* tile_off,
                               hipStream_t s) {
  hipLaunchKernelGGL(tile_off_kernel, dim3(1), dim3(1024), 0, s, offsets, N, bm, tile_off, bm,
                     nullptr, nullptr, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_tile_offsets2(const int32_t* offsets, int N, int bm, int32_t* tile_off, int bm2,
                                int32_t* tile_off2, int32_t* tile_exp2, int32_t* sched, int nsched,
                                hipStream_t s) {
  hipLaunchKernelGGL(tile_off_kernel, dim3(1), dim3(1024), 0, s, offsets, N, bm, tile_off, bm2,
                     tile_off2, tile_exp2, sched, nsched);
  return hipGetLastError();
}

size_t dispatch_scratch_bytes(int64_t Tn, int64_t E, int64_t N) {
  (void)N;
  const int64_t nblk = (Tn + kTokPerBlk - 1) / kTokPerBlk;
  return static_cast<size_t>(align256(nblk * E * 8) + align256(nblk * E * 4) +
                             align256(nblk * E * 4));
}

hipError_t launch_dispatch(const int32_t* topk_idx, int Tn, int E, int N, int K, int bm, int bm2,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                           int32_t* tile_off, int32_t* tile_off2, int32_t* tile_exp,
                           int32_t* tile_exp1, int32_t* sched, void* scratch, hipStream_t s) {
  const int nblk = (Tn + kTokPerBlk - 1) / kTokPerBlk;
  Scratch sc = carve(scratch, nblk, E);
  if (nblk > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(kThreads), E * sizeof(uint64_t), s,
                       topk_idx, Tn, E, K, sc.mask, sc.cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, sc.cnt, nblk, E, N, bm, bm2, counts,
                     offsets, tile_off, tile_off2, tile_exp, tile_exp1, sched, sc.base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(kThreads), E * sizeof(uint64_t), s,
                     topk_idx, Tn, E, N, K, sc.mask, sc.base, perm, inv);
  return hipGetLastError();
}

}  // namespace zc

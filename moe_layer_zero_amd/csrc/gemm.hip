// Grouped and dense GEMMs of the layer on gfx950 matrix cores.
//
// One persistent, XCD-aware kernel template covers every contraction of the
// forward and backward pass ("LongCat-Flash Technical Report", section 2.1:
// FFN experts evaluated only on the tokens routed to them; the expert form
// is SwiGLU without biases).  C = A * B per group, fp32 accumulation:
//
//   mode        A (M x K)                 B (K x N)                  used for
//   F1          x rows                    W_r rows (k-contig)        router scores
//   F4          x rows gathered by perm   W_g / W_u rows             h = silu(a)*u
//   F5          h rows                    W_d rows                   y
//   B2a         dy rows                   W_d as K x N (n-contig)    da, du (SwiGLU bwd)
//   B4a         [da | du] rows            [W_g ; W_u] as K x N       expert dx
//   B2b (Kgrp)  dy^T (m-contig)           h (n-contig)               dW_d[e]
//   B4b (Kgrp)  da^T or du^T              x gathered by perm         dW_g[e], dW_u[e]
//   B5          dl^T / dl                 x / W_r                    dW_r, router dx
//
// M-grouped modes run over the rows of each FFN expert's segment of the
// dispatch order (offsets[e] .. offsets[e+1]); K-grouped modes reduce over
// that segment and write one output matrix per expert.  Every output element
// is produced by exactly one workgroup with a fixed k order, so results are
// bitwise reproducible.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (four wave64s, each
// 64 x 64 as 4 x 4 MFMA 16x16 tiles), K staged through LDS in slabs of 64
// (bf16, v_mfma_f32_16x16x32_bf16) or 32 (fp32, v_mfma_f32_16x16x4_f32),
// double-buffered with a register prefetch of the next slab.  Operands whose
// reduction dimension is contiguous are copied to LDS with 16-byte vector
// loads and stores; the others are transposed on the way into LDS.
// Workgroups are persistent: block b handles tiles b', b'+G, ... where b' is
// b remapped so that the 1/8 of the grid that lands on one XCD (blocks are
// dealt to the 8 XCDs round-robin) owns a contiguous range of tiles, and
// tiles are ordered in groups of 8 m-tiles sharing each n-tile, so the
// operand panels that a group re-reads stay in that XCD's L2.
#include <algorithm>

#include "zc_common.h"

namespace zc {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NTHR = 256;
constexpr int GM = 8;

enum Grouping { DENSE = 0, MGROUP = 1, KGROUP = 2 };
enum Epi { EPI_STORE = 0, EPI_F32 = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3 };

template <typename T> struct TileCfg;
template <> struct TileCfg<bf16_t> {
  static constexpr int BK = 64, VEC = 8, PAD = 8, KS = 32;
};
template <> struct TileCfg<float> {
  static constexpr int BK = 32, VEC = 4, PAD = 4, KS = 4;
};

struct Params {
  int M, N, K;  // DENSE: all three; MGROUP: N, K; KGROUP: M, N
  int ngroups;
  const int32_t* goff;      // [ngroups+1] segment bounds (MGROUP rows / KGROUP k)
  const int32_t* tile_off;  // MGROUP: [ngroups+1] prefix of m-tiles per segment
  // A: KC -> A[g*a_gs + row(m)*lda + k]; MN -> A[g*a_gs + row(k)*lda + m]
  const void* A;
  int64_t lda, a_gs;
  const int32_t* amap;  // gather: row(i) = amap[i] / adiv (nullptr: row(i) = i)
  int adiv;
  int a_ext;            // MN: valid extent of m (multiple of the vector width)
  // B: KC -> B[g*b_gs + n*ldb + k]; MN -> B[g*b_gs + row(k)*ldb + n]
  const void* B;
  const void* B2;       // SwiGLU: up-projection rows; K-split: k >= b_split
  int64_t ldb, b_gs;
  const int32_t* bmap;
  int bdiv;
  int b_split;
  int b_ext;            // MN: valid extent of n
  // C
  void* C;
  int64_t ldc, c_gs, c2_off;
  const void* sa;  // SwiGLU bwd: saved a, u
  const void* su;
  int64_t ld_au;
  void* wa;        // SwiGLU fwd: where to save a, u (nullable)
  void* wu;
};

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

template <typename T>
__device__ __forceinline__ void mfma_step(f32x4_t& c, const T* a, const T* b);

template <>
__device__ __forceinline__ void mfma_step<bf16_t>(f32x4_t& c, const bf16_t* a, const bf16_t* b) {
  const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(a);
  const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(b);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(f32x4_t& c, const float* a, const float* b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void store_vec_transposed(T* s, int ldsw, int mc, int krow,
                                                     const u32x4_t& v);

template <>
__device__ __forceinline__ void store_vec_transposed<bf16_t>(bf16_t* s, int ldsw, int mc,
                                                             int krow, const u32x4_t& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[(mc + 2 * e) * ldsw + krow] = static_cast<bf16_t>(v[e] & 0xffffu);
    s[(mc + 2 * e + 1) * ldsw + krow] = static_cast<bf16_t>(v[e] >> 16);
  }
}

template <>
__device__ __forceinline__ void store_vec_transposed<float>(float* s, int ldsw, int mc, int krow,
                                                            const u32x4_t& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) s[(mc + e) * ldsw + krow] = __uint_as_float(v[e]);
}

template <typename T, bool AKC, bool BKC, int GRP, int EPI, bool AG, bool BG, bool BKS>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(Params p) {
  using Cfg = TileCfg<T>;
  constexpr int BK = Cfg::BK, VEC = Cfg::VEC, KS = Cfg::KS;
  constexpr int LDSW = BK + Cfg::PAD;   // LDS row pitch in elements
  constexpr int KCH = BK / VEC;         // vector chunks per row (k-contiguous)
  constexpr int MNCH = 128 / VEC;       // vector chunks per k-row (m/n-contiguous)
  constexpr int BNOUT = EPI == EPI_SWIGLU ? BN / 2 : BN;
  __shared__ __align__(16) T sA[2][BM * LDSW];
  __shared__ __align__(16) T sB[2][BN * LDSW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const T* Ab = static_cast<const T*>(p.A);
  const T* Bb = static_cast<const T*>(p.B);
  const T* B2b = static_cast<const T*>(p.B2);

  const int ntile_n = (p.N + BNOUT - 1) / BNOUT;
  int mt_tot;
  int64_t total;
  if constexpr (GRP == MGROUP) {
    mt_tot = p.tile_off[p.ngroups];
    total = static_cast<int64_t>(mt_tot) * ntile_n;
  } else if constexpr (GRP == DENSE) {
    mt_tot = (p.M + BM - 1) / BM;
    total = static_cast<int64_t>(mt_tot) * ntile_n;
  } else {
    mt_tot = (p.M + BM - 1) / BM;
    total = static_cast<int64_t>(mt_tot) * ntile_n * p.ngroups;
  }
  const int G = gridDim.x;
  const int first = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;

  for (int64_t L = first; L < total; L += G) {
    // ---- tile decode
    int g = 0;
    int64_t Lr = L;
    if constexpr (GRP == KGROUP) {
      const int64_t per = static_cast<int64_t>(mt_tot) * ntile_n;
      g = static_cast<int>(L / per);
      Lr = L - static_cast<int64_t>(g) * per;
    }
    const int64_t grp = Lr / (static_cast<int64_t>(GM) * ntile_n);
    const int fm = static_cast<int>(grp * GM);
    const int gsz = min(GM, mt_tot - fm);
    const int r = static_cast<int>(Lr - grp * GM * ntile_n);
    const int mt = fm + r % gsz;
    const int nt = r / gsz;
    int m0, mcount, kbeg = 0, kend = p.K;
    if constexpr (GRP == MGROUP) {
      int lo = 0, hi = p.ngroups - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.tile_off[mid] <= mt) lo = mid;
        else hi = mid - 1;
      }
      g = lo;
      m0 = p.goff[g] + (mt - p.tile_off[g]) * BM;
      mcount = min(BM, p.goff[g + 1] - m0);
    } else {
      m0 = mt * BM;
      mcount = min(BM, p.M - m0);
      if constexpr (GRP == KGROUP) {
        kbeg = p.goff[g];
        kend = p.goff[g + 1];
      }
    }
    const int n0 = nt * BNOUT;

    // ---- per-thread row pointers of k-contiguous operands (fixed per tile)
    const T* arow[4];
    const T* brow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = (tid + NTHR * q) / KCH;
      if constexpr (AKC) {
        arow[q] = nullptr;
        if (rr < mcount) {
          const int gm = m0 + rr;
          const int64_t ph = AG ? p.amap[gm] / p.adiv : gm;
          arow[q] = Ab + g * p.a_gs + ph * p.lda;
        }
      }
      if constexpr (BKC) {
        brow[q] = nullptr;
        if constexpr (EPI == EPI_SWIGLU) {
          const int col = n0 + (rr & 63);
          if (col < p.N) brow[q] = (rr < 64 ? Bb : B2b) + g * p.b_gs + static_cast<int64_t>(col) * p.ldb;
        } else {
          const int col = n0 + rr;
          if (col < p.N) brow[q] = Bb + g * p.b_gs + static_cast<int64_t>(col) * p.ldb;
        }
      }
    }

    u32x4_t ra[4], rb[4];
    auto fetch = [&](int k0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid + NTHR * q;
        // A
        if constexpr (AKC) {
          const int kc = (c % KCH) * VEC;
          ra[q] = u32x4_t{0, 0, 0, 0};
          if (arow[q] && k0 + kc < kend) ra[q] = *reinterpret_cast<const u32x4_t*>(arow[q] + k0 + kc);
        } else {
          const int krow = c / MNCH, mc = (c % MNCH) * VEC;
          const int k = k0 + krow;
          ra[q] = u32x4_t{0, 0, 0, 0};
          if (k < kend && m0 + mc < p.a_ext) {
            const int64_t ph = AG ? p.amap[k] / p.adiv : k;
            ra[q] = *reinterpret_cast<const u32x4_t*>(Ab + g * p.a_gs + ph * p.lda + m0 + mc);
          }
        }
        // B
        if constexpr (BKC) {
          const int kc = (c % KCH) * VEC;
          rb[q] = u32x4_t{0, 0, 0, 0};
          if (brow[q] && k0 + kc < kend) rb[q] = *reinterpret_cast<const u32x4_t*>(brow[q] + k0 + kc);
        } else {
          const int krow = c / MNCH, nc = (c % MNCH) * VEC;
          int k = k0 + krow;
          rb[q] = u32x4_t{0, 0, 0, 0};
          if (k < kend && n0 + nc < p.b_ext) {
            const T* src = Bb;
            if constexpr (BKS) {
              if (k >= p.b_split) {
                src = B2b;
                k -= p.b_split;
              }
            }
            const int64_t ph = BG ? p.bmap[k] / p.bdiv : k;
            rb[q] = *reinterpret_cast<const u32x4_t*>(src + g * p.b_gs + ph * p.ldb + n0 + nc);
          }
        }
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid + NTHR * q;
        if constexpr (AKC) {
          *reinterpret_cast<u32x4_t*>(&sA[buf][(c / KCH) * LDSW + (c % KCH) * VEC]) = ra[q];
        } else {
          store_vec_transposed<T>(sA[buf], LDSW, (c % MNCH) * VEC, c / MNCH, ra[q]);
        }
        if constexpr (BKC) {
          *reinterpret_cast<u32x4_t*>(&sB[buf][(c / KCH) * LDSW + (c % KCH) * VEC]) = rb[q];
        } else {
          store_vec_transposed<T>(sB[buf], LDSW, (c % MNCH) * VEC, c / MNCH, rb[q]);
        }
      }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int a_row0 = wm * 64 + (lane & 15);
    int b_row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (EPI == EPI_SWIGLU)
        b_row[j] = (j < 2 ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16) + (lane & 15);
      else
        b_row[j] = wn * 64 + j * 16 + (lane & 15);
    }
    const int kl = (lane >> 4) * (KS / 4);

    __syncthreads();  // previous tile's readers are done with both buffers
    if (kbeg < kend) {
      fetch(kbeg);
      stash(0);
    }
    __syncthreads();
    int cur = 0;
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
      const bool more = k0 + BK < kend;
      if (more) fetch(k0 + BK);
      const T* a_s = sA[cur];
      const T* b_s = sB[cur];
#pragma unroll
      for (int ks = 0; ks < BK; ks += KS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mfma_step<T>(acc[i][j], a_s + (a_row0 + i * 16) * LDSW + ks + kl,
                         b_s + b_row[j] * LDSW + ks + kl);
      }
      if (more) stash(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }

    // ---- epilogue (lane holds rows 4*(lane/16)+v, column lane%16 of each 16x16)
    const int rbase = wm * 64 + 4 * (lane >> 4);
    if constexpr (EPI == EPI_SWIGLU) {
      T* h = static_cast<T*>(p.C);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = rbase + i * 16 + v;
            if (rl < mcount && col < p.N) {
              const int64_t row = m0 + rl;
              const float a = acc[i][j][v], u = acc[i][j + 2][v];
              Elem<T>::st(h + row * p.ldc + col, silu_f(a) * u);
              if (p.wa) {
                Elem<T>::st(static_cast<T*>(p.wa) + row * p.ld_au + col, a);
                Elem<T>::st(static_cast<T*>(p.wu) + row * p.ld_au + col, u);
              }
            }
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rl = rbase + i * 16 + v;
            if (rl < mcount && col < p.N) {
              const int64_t row = m0 + rl;
              const float c = acc[i][j][v];
              if constexpr (EPI == EPI_F32) {
                static_cast<float*>(p.C)[g * p.c_gs + row * p.ldc + col] = c;
              } else if constexpr (EPI == EPI_STORE) {
                Elem<T>::st(static_cast<T*>(p.C) + g * p.c_gs + row * p.ldc + col, c);
              } else {  // SwiGLU backward: c = dh
                const float a = Elem<T>::ld(static_cast<const T*>(p.sa) + row * p.ld_au + col);
                const float u = Elem<T>::ld(static_cast<const T*>(p.su) + row * p.ld_au + col);
                const float sg = 1.0f / (1.0f + __expf(-a));
                T* o = static_cast<T*>(p.C) + row * p.ldc + col;
                Elem<T>::st(o, c * u * (sg * (1.0f + a * (1.0f - sg))));
                Elem<T>::st(o + p.c2_off, c * (a * sg));
              }
            }
          }
        }
    }
  }
}

Params blank() {
  Params p{};
  p.adiv = 1;
  p.bdiv = 1;
  p.ngroups = 1;
  return p;
}

template <typename T, bool AKC, bool BKC, int GRP, int EPI, bool AG, bool BG, bool BKS>
hipError_t run(const Params& p, int64_t total_ub, int cu, hipStream_t s) {
  int64_t G = std::min<int64_t>(total_ub, static_cast<int64_t>(cu) * 2);
  if (G <= 0) return hipSuccess;
  G = (G + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<T, AKC, BKC, GRP, EPI, AG, BG, BKS>), dim3(G), dim3(NTHR), 0, s,
                     p);
  return hipGetLastError();
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// F1: logits[T][E] = x[T][d] * wr[E][d]^T.
template <typename T>
hipError_t launch_router_gemm(const T* x, const T* wr, float* logits, int Tn, int E, int d,
                              int cu, hipStream_t s) {
  Params p = blank();
  p.M = Tn; p.N = E; p.K = d;
  p.A = x; p.lda = d;
  p.B = wr; p.ldb = d;
  p.C = logits; p.ldc = E;
  return run<T, true, true, DENSE, EPI_F32, false, false, false>(p, cdiv(Tn, BM) * cdiv(E, BN),
                                                                 cu, s);
}

// F4: h = silu(x_e W_g[e]^T) * (x_e W_u[e]^T) over each expert's rows.
template <typename T>
hipError_t launch_ffn_gateup(const T* x, const T* wg, const T* wu, const int32_t* offsets,
                             const int32_t* perm, const int32_t* tile_off, int N, int I, int d,
                             int K, int64_t max_rows, T* h, T* save_a, T* save_u, int cu,
                             hipStream_t s) {
  Params p = blank();
  p.N = I; p.K = d; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = x; p.lda = d; p.amap = perm; p.adiv = K;
  p.B = wg; p.B2 = wu; p.ldb = d; p.b_gs = static_cast<int64_t>(I) * d;
  p.C = h; p.ldc = I;
  p.wa = save_a; p.wu = save_u; p.ld_au = I;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(I, BN / 2);
  return run<T, true, true, MGROUP, EPI_SWIGLU, true, false, false>(p, ub, cu, s);
}

// F5: y = h W_d[e]^T.
template <typename T>
hipError_t launch_ffn_down(const T* h, const T* wd, const int32_t* offsets,
                           const int32_t* tile_off, int N, int I, int d, int64_t max_rows, T* y,
                           int cu, hipStream_t s) {
  Params p = blank();
  p.N = d; p.K = I; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = h; p.lda = I;
  p.B = wd; p.ldb = I; p.b_gs = static_cast<int64_t>(d) * I;
  p.C = y; p.ldc = d;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(d, BN);
  return run<T, true, true, MGROUP, EPI_STORE, false, false, false>(p, ub, cu, s);
}

// B2a + B3: dh = dy W_d[e]; da = dh*u*silu'(a), du = dh*silu(a) -> dadu[P][2I].
template <typename T>
hipError_t launch_bwd_down_dh(const T* dyg, const T* wd, const T* sa, const T* su,
                              const int32_t* offsets, const int32_t* tile_off, int N, int I,
                              int d, int64_t max_rows, T* dadu, int cu, hipStream_t s) {
  Params p = blank();
  p.N = I; p.K = d; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = dyg; p.lda = d;
  p.B = wd; p.ldb = I; p.b_gs = static_cast<int64_t>(d) * I; p.b_ext = I;
  p.C = dadu; p.ldc = 2 * static_cast<int64_t>(I); p.c2_off = I;
  p.sa = sa; p.su = su; p.ld_au = I;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(I, BN);
  return run<T, true, false, MGROUP, EPI_SWIGLU_BWD, false, false, false>(p, ub, cu, s);
}

// B2b: dW_d[e] = dy_e^T h_e  (reduction over the expert's rows).
template <typename T>
hipError_t launch_bwd_down_dw(const T* dyg, const T* h, const int32_t* offsets, int N, int I,
                              int d, T* dwd, int cu, hipStream_t s) {
  Params p = blank();
  p.M = d; p.N = I; p.ngroups = N; p.goff = offsets;
  p.A = dyg; p.lda = d; p.a_ext = d;
  p.B = h; p.ldb = I; p.b_ext = I;
  p.C = dwd; p.ldc = I; p.c_gs = static_cast<int64_t>(d) * I;
  const int64_t tot = cdiv(d, BM) * cdiv(I, BN) * N;
  return run<T, false, false, KGROUP, EPI_STORE, false, false, false>(p, tot, cu, s);
}

// B4a: dx_perm = [da | du] [W_g[e] ; W_u[e]].
template <typename T>
hipError_t launch_bwd_gateup_dx(const T* dadu, const T* wg, const T* wu, const int32_t* offsets,
                                const int32_t* tile_off, int N, int I, int d, int64_t max_rows,
                                T* dxp, int cu, hipStream_t s) {
  Params p = blank();
  p.N = d; p.K = 2 * I; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = dadu; p.lda = 2 * static_cast<int64_t>(I);
  p.B = wg; p.B2 = wu; p.ldb = d; p.b_gs = static_cast<int64_t>(I) * d; p.b_split = I;
  p.b_ext = d;
  p.C = dxp; p.ldc = d;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(d, BN);
  return run<T, true, false, MGROUP, EPI_STORE, false, false, true>(p, ub, cu, s);
}

// B4b: dW_g[e] = da_e^T x_e, dW_u[e] = du_e^T x_e (x rows gathered by perm).
template <typename T>
hipError_t launch_bwd_gateup_dw(const T* dadu, const T* x, const int32_t* offsets,
                                const int32_t* perm, int N, int I, int d, int K, T* dwg, T* dwu,
                                int cu, hipStream_t s) {
  Params p = blank();
  p.M = I; p.N = d; p.ngroups = N; p.goff = offsets;
  p.lda = 2 * static_cast<int64_t>(I); p.a_ext = I;
  p.B = x; p.ldb = d; p.bmap = perm; p.bdiv = K; p.b_ext = d;
  p.ldc = d; p.c_gs = static_cast<int64_t>(I) * d;
  const int64_t tot = cdiv(I, BM) * cdiv(d, BN) * N;
  p.A = dadu; p.C = dwg;
  hipError_t e = run<T, false, false, KGROUP, EPI_STORE, false, true, false>(p, tot, cu, s);
  if (e != hipSuccess) return e;
  p.A = dadu + I; p.C = dwu;
  return run<T, false, false, KGROUP, EPI_STORE, false, true, false>(p, tot, cu, s);
}

// B5: dW_r = dl^T x   (dl [T][ldl], zero-padded columns E..ldl).
template <typename T>
hipError_t launch_router_dw(const T* dl, int ldl, const T* x, int Tn, int E, int d, T* dwr, int cu,
                            hipStream_t s) {
  Params p = blank();
  p.M = E; p.N = d; p.K = Tn;
  p.A = dl; p.lda = ldl; p.a_ext = ldl;
  p.B = x; p.ldb = d; p.b_ext = d;
  p.C = dwr; p.ldc = d;
  return run<T, false, false, DENSE, EPI_STORE, false, false, false>(p, cdiv(E, BM) * cdiv(d, BN),
                                                                    cu, s);
}

// B5: router part of dx = dl W_r.
template <typename T>
hipError_t launch_router_dx(const T* dl, int ldl, const T* wr, int Tn, int E, int d, T* dxr,
                            int cu, hipStream_t s) {
  Params p = blank();
  p.M = Tn; p.N = d; p.K = E;
  p.A = dl; p.lda = ldl;
  p.B = wr; p.ldb = d; p.b_ext = d;
  p.C = dxr; p.ldc = d;
  return run<T, true, false, DENSE, EPI_STORE, false, false, false>(p, cdiv(Tn, BM) * cdiv(d, BN),
                                                                   cu, s);
}

#define ZC_INST(T)                                                                              \
  template hipError_t launch_router_gemm<T>(const T*, const T*, float*, int, int, int, int,     \
                                            hipStream_t);                                       \
  template hipError_t launch_ffn_gateup<T>(const T*, const T*, const T*, const int32_t*,        \
                                           const int32_t*, const int32_t*, int, int, int, int,  \
                                           int64_t, T*, T*, T*, int, hipStream_t);              \
  template hipError_t launch_ffn_down<T>(const T*, const T*, const int32_t*, const int32_t*,    \
                                         int, int, int, int64_t, T*, int, hipStream_t);         \
  template hipError_t launch_bwd_down_dh<T>(const T*, const T*, const T*, const T*,             \
                                            const int32_t*, const int32_t*, int, int, int,      \
                                            int64_t, T*, int, hipStream_t);                     \
  template hipError_t launch_bwd_down_dw<T>(const T*, const T*, const int32_t*, int, int, int,  \
                                            T*, int, hipStream_t);                              \
  template hipError_t launch_bwd_gateup_dx<T>(const T*, const T*, const T*, const int32_t*,     \
                                              const int32_t*, int, int, int, int64_t, T*, int,  \
                                              hipStream_t);                                     \
  template hipError_t launch_bwd_gateup_dw<T>(const T*, const T*, const int32_t*,               \
                                              const int32_t*, int, int, int, int, T*, T*, int,  \
                                              hipStream_t);                                     \
  template hipError_t launch_router_dw<T>(const T*, int, const T*, int, int, int, T*, int,      \
                                          hipStream_t);                                         \
  template hipError_t launch_router_dx<T>(const T*, int, const T*, int, int, int, T*, int,      \
                                          hipStream_t);
ZC_INST(bf16_t)
ZC_INST(float)
#undef ZC_INST

}  // namespace zc

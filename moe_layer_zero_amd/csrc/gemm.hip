// Grouped and dense GEMMs of the layer on gfx950 matrix cores.
//
// One persistent, XCD-aware kernel template covers every contraction of the
// forward and backward pass ("LongCat-Flash Technical Report", section 2.1:
// FFN experts evaluated only on the tokens routed to them; the expert form
// is SwiGLU without biases).  C = A * B per group, fp32 accumulation:
//
//   contraction        A (M x K)                  B (K x N)
//   router scores      x rows                     W_r rows
//   gate/up + SwiGLU   x rows gathered by perm    W_g, W_u rows
//   down               h rows                     W_d rows
//   dh + SwiGLU bwd    dout rows gathered         W_d as K x N (n-contiguous)
//   expert dx          [da | du] rows             [W_g ; W_u] as K x N
//   dW_d  (per expert) dout^T gathered            g * h  (reduction over rows)
//   dW_g, dW_u         da^T, du^T                 x gathered by perm
//   dW_r, router dx    dl^T / dl                  x / W_r
//
// M-grouped modes run over the rows of each FFN expert's segment of the
// dispatch order (offsets[e] .. offsets[e+1]); K-grouped modes reduce over
// that segment and write one output matrix per expert.  Every output element
// is produced by exactly one workgroup with a fixed k order, so results are
// bitwise reproducible.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (four wave64s, each
// 64 x 64 as 4 x 4 MFMA 16x16 tiles), K staged through LDS in slabs of 64
// bf16 (v_mfma_f32_16x16x32_bf16) or 32 fp32 (v_mfma_f32_16x16x4_f32),
// double-buffered with a register prefetch of the next slab.  Operand modes:
//   KC      reduction dim contiguous: 16-byte loads, 16-byte LDS stores
//   MN      m (or n) contiguous: 16-byte loads, transposed into LDS
//   SPLIT   an fp32 operand of a bf16 GEMM: each value v becomes the pair
//           hi = bf16(v), lo = bf16(v - hi) in two adjacent k slots
//   DUP     the exact bf16 partner of a SPLIT operand: each value written to
//           both slots, so hi*b + lo*b sums to v*b with ~16 mantissa bits
// SPLIT/DUP keep the backward's fp32 intermediates (da, du, g*h, dl) from
// being rounded to bf16 before they are contracted.
// Workgroups are persistent: block b handles tiles b', b'+G, ... where b' is
// b remapped so that the 1/8 of the grid that lands on one XCD (blocks are
// dealt to the 8 XCDs round-robin) owns a contiguous range of tiles, and
// tiles are ordered in groups of 8 m-tiles sharing each n-tile, so the
// operand panels that a group re-reads stay in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "zc_common.h"

namespace zc {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NTHR = 256;
constexpr int GM = 8;

enum Grouping { DENSE = 0, MGROUP = 1, KGROUP = 2 };
enum Epi { EPI_STORE = 0, EPI_F32 = 1, EPI_SWIGLU = 2, EPI_SWIGLU_BWD = 3 };
enum OpMode { OP_KC = 0, OP_MN = 1, OP_SPLIT_KC = 2, OP_SPLIT_MN = 3, OP_DUP_MN = 4 };

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
  int kchunk;               // KGROUP without goff: segment g is k in [g kchunk, (g+1) kchunk)
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
  const float* kscale;  // fp32 m/n-contiguous B: row k scaled by kscale[k] (nullable)
  // C
  void* C;
  int64_t ldc, c_gs, c2_off;
  const float* rscale;  // SwiGLU bwd: row scale of dh
  const float* sa;      // SwiGLU bwd: saved a, u (fp32)
  const float* su;
  int64_t ld_au;
  float* wa;            // SwiGLU fwd: where to save a, u, h in fp32 (nullable)
  float* wu;
  float* wh;
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

// (hi, lo) bf16 pair of an fp32 value, packed hi in the low half.
__device__ __forceinline__ uint32_t split_pair(float v) {
  const bf16_t hi = f2bf(v);
  const bf16_t lo = f2bf(v - bf2f(hi));
  return static_cast<uint32_t>(hi) | (static_cast<uint32_t>(lo) << 16);
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

// Registers one thread stages per operand per k-slab.
template <int MODE> struct Chunks { static constexpr int n = 4; };
template <> struct Chunks<OP_DUP_MN> { static constexpr int n = 2; };

template <typename T, int AM, int BM_, int GRP, int EPI, bool AG, bool BG, bool BKS>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(Params p) {
  using Cfg = TileCfg<T>;
  constexpr bool SPLIT = AM >= OP_SPLIT_KC || BM_ >= OP_SPLIT_KC;
  static_assert(!SPLIT || std::is_same<T, bf16_t>::value, "split operands feed bf16 MFMA only");
  using TA = typename std::conditional<AM == OP_SPLIT_KC || AM == OP_SPLIT_MN, float, T>::type;
  using TB = typename std::conditional<BM_ == OP_SPLIT_KC || BM_ == OP_SPLIT_MN, float, T>::type;
  constexpr int BK = Cfg::BK, VEC = Cfg::VEC, KS = Cfg::KS;
  constexpr int KT = SPLIT ? BK / 2 : BK;  // original k per slab
  constexpr int LDSW = BK + Cfg::PAD;      // LDS row pitch in elements
  constexpr int KCH = 8;                   // 16-byte chunks per row and slab (k-contiguous)
  constexpr int MNCH = 128 / VEC;          // 16-byte chunks per k-row (plain m/n-contiguous)
  constexpr int BNOUT = EPI == EPI_SWIGLU ? BN / 2 : BN;
  constexpr int CA = Chunks<AM>::n, CB = Chunks<BM_>::n;
  __shared__ __align__(16) T sA[2][BM * LDSW];
  __shared__ __align__(16) T sB[2][BN * LDSW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const TA* Ab = static_cast<const TA*>(p.A);
  const TB* Bb = static_cast<const TB*>(p.B);
  const TB* B2b = static_cast<const TB*>(p.B2);

  const int ntile_n = (p.N + BNOUT - 1) / BNOUT;
  int mt_tot;
  int64_t total;
  if constexpr (GRP == MGROUP) {
    mt_tot = ld_scalar(p.tile_off + p.ngroups);
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
        if (ld_scalar(p.tile_off + mid) <= mt) lo = mid;
        else hi = mid - 1;
      }
      g = lo;
      m0 = ld_scalar(p.goff + g) + (mt - ld_scalar(p.tile_off + g)) * BM;
      mcount = min(BM, ld_scalar(p.goff + g + 1) - m0);
    } else {
      m0 = mt * BM;
      mcount = min(BM, p.M - m0);
      if constexpr (GRP == KGROUP) {
        if (p.goff) {
          kbeg = ld_scalar(p.goff + g);
          kend = ld_scalar(p.goff + g + 1);
        } else {
          kbeg = g * p.kchunk;
          kend = min(p.K, kbeg + p.kchunk);
        }
      }
    }
    const int n0 = nt * BNOUT;

    // ---- per-thread row pointers of k-contiguous operands (fixed per tile)
    const TA* arow[4];
    const TB* brow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = (tid + NTHR * q) / KCH;
      if constexpr (AM == OP_KC || AM == OP_SPLIT_KC) {
        arow[q] = nullptr;
        if (rr < mcount) {
          const int gm = m0 + rr;
          const int64_t ph = AG ? p.amap[gm] / p.adiv : gm;
          arow[q] = Ab + g * p.a_gs + ph * p.lda;
        }
      }
      if constexpr (BM_ == OP_KC || BM_ == OP_SPLIT_KC) {
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

    u32x4_t ra[CA], rb[CB];
    // One operand's slab into registers.  `row_ptr` resolves a k-row of an
    // m/n-contiguous operand (gather, K-split, group offset).
    auto fetch_op = [&](auto mode_tag, u32x4_t* rg, const auto* const* rowk, auto row_ptr, int x0,
                        int ext, const float* ksc, int k0) {
      constexpr int MODE = decltype(mode_tag)::value;
      constexpr int NC = Chunks<MODE>::n;
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int c = tid + NTHR * q;
        rg[q] = u32x4_t{0, 0, 0, 0};
        if constexpr (MODE == OP_KC || MODE == OP_SPLIT_KC) {
          constexpr int EPC = MODE == OP_KC ? VEC : 4;  // original k per chunk
          const int kc = (c % KCH) * EPC;
          if (rowk[q] && k0 + kc < kend) rg[q] = *reinterpret_cast<const u32x4_t*>(rowk[q] + k0 + kc);
        } else {
          constexpr int PER = MODE == OP_MN ? MNCH : (MODE == OP_SPLIT_MN ? 32 : 16);
          constexpr int EPC = MODE == OP_SPLIT_MN ? 4 : VEC;
          const int krow = c / PER, mc = (c % PER) * EPC;
          const int k = k0 + krow;
          if (k < kend && x0 + mc < ext) {
            rg[q] = *reinterpret_cast<const u32x4_t*>(row_ptr(k) + x0 + mc);
            if constexpr ((MODE == OP_SPLIT_MN) || (MODE == OP_MN && std::is_same<T, float>::value)) {
              if (ksc) {
                const float sc = ksc[k];
#pragma unroll
                for (int e = 0; e < 4; ++e) rg[q][e] = __float_as_uint(__uint_as_float(rg[q][e]) * sc);
              }
            }
          }
        }
      }
    };
    auto stash_op = [&](auto mode_tag, const u32x4_t* rg, T* s) {
      constexpr int MODE = decltype(mode_tag)::value;
      constexpr int NC = Chunks<MODE>::n;
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const int c = tid + NTHR * q;
        if constexpr (MODE == OP_KC) {
          *reinterpret_cast<u32x4_t*>(&s[(c / KCH) * LDSW + (c % KCH) * VEC]) = rg[q];
        } else if constexpr (MODE == OP_MN) {
          store_vec_transposed<T>(s, LDSW, (c % MNCH) * VEC, c / MNCH, rg[q]);
        } else if constexpr (MODE == OP_SPLIT_KC) {
          u32x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = split_pair(__uint_as_float(rg[q][e]));
          *reinterpret_cast<u32x4_t*>(&s[(c / KCH) * LDSW + (c % KCH) * 8]) = w;
        } else if constexpr (MODE == OP_SPLIT_MN) {
          const int krow = c / 32, mc = (c % 32) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<uint32_t*>(&s[(mc + e) * LDSW + 2 * krow]) =
                split_pair(__uint_as_float(rg[q][e]));
        } else {  // OP_DUP_MN
          const int krow = c / 16, mc = (c % 16) * 8;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = rg[q][e] & 0xffffu, hi = rg[q][e] >> 16;
            *reinterpret_cast<uint32_t*>(&s[(mc + 2 * e) * LDSW + 2 * krow]) = lo | (lo << 16);
            *reinterpret_cast<uint32_t*>(&s[(mc + 2 * e + 1) * LDSW + 2 * krow]) = hi | (hi << 16);
          }
        }
      }
    };
    auto a_rowk = [&](int k) -> const TA* {
      const int64_t ph = AG ? p.amap[k] / p.adiv : k;
      return Ab + g * p.a_gs + ph * p.lda;
    };
    auto b_rowk = [&](int k) -> const TB* {
      const TB* src = Bb;
      if constexpr (BKS) {
        if (k >= p.b_split) {
          src = B2b;
          k -= p.b_split;
        }
      }
      const int64_t ph = BG ? p.bmap[k] / p.bdiv : k;
      return src + g * p.b_gs + ph * p.ldb;
    };
    auto fetch = [&](int k0) {
      fetch_op(std::integral_constant<int, AM>{}, ra, arow, a_rowk, m0, p.a_ext, nullptr, k0);
      fetch_op(std::integral_constant<int, BM_>{}, rb, brow, b_rowk, n0, p.b_ext, p.kscale, k0);
    };
    auto stash = [&](int buf) {
      stash_op(std::integral_constant<int, AM>{}, ra, sA[buf]);
      stash_op(std::integral_constant<int, BM_>{}, rb, sB[buf]);
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
    for (int k0 = kbeg; k0 < kend; k0 += KT) {
      const bool more = k0 + KT < kend;
      if (more) fetch(k0 + KT);
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
              const float hv = silu_f(a) * u;
              Elem<T>::st(h + row * p.ldc + col, hv);
              if (p.wa) {
                p.wa[row * p.ld_au + col] = a;
                p.wu[row * p.ld_au + col] = u;
                p.wh[row * p.ld_au + col] = hv;
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
              } else {  // SwiGLU backward: dh = rscale[row] * c
                const float dh = c * p.rscale[row];
                const float a = p.sa[row * p.ld_au + col];
                const float u = p.su[row * p.ld_au + col];
                const float sg = 1.0f / (1.0f + __expf(-a));
                float* o = static_cast<float*>(p.C) + row * p.ldc + col;
                o[0] = dh * u * (sg * (1.0f + a * (1.0f - sg)));
                o[p.c2_off] = dh * (a * sg);
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

template <typename T, int AM, int BMD, int GRP, int EPI, bool AG, bool BG, bool BKS>
hipError_t run(const Params& p, int64_t total_ub, int cu, hipStream_t s) {
  int64_t G = std::min<int64_t>(total_ub, static_cast<int64_t>(cu) * 2);
  if (G <= 0) return hipSuccess;
  G = (G + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<T, AM, BMD, GRP, EPI, AG, BG, BKS>), dim3(G), dim3(NTHR), 0, s,
                     p);
  return hipGetLastError();
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename T>
constexpr bool is_bf16() {
  return std::is_same<T, bf16_t>::value;
}

}  // namespace

// Partial sums of a GEMM whose reduction was cut into chunks: out[i] = sum
// over chunks g = 0, 1, ... of part[g][i], added in chunk order (a fixed
// order: reproducible).
__global__ __launch_bounds__(256) void add_partials_kernel_f32(const float* __restrict__ part,
                                                               int splits, int64_t n, float* out) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float acc = 0.f;
    for (int g = 0; g < splits; ++g) acc += part[g * n + i];
    out[i] = acc;
  }
}
__global__ __launch_bounds__(256) void add_partials_kernel_bf16(const float* __restrict__ part,
                                                                int splits, int64_t n,
                                                                bf16_t* out) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float acc = 0.f;
    for (int g = 0; g < splits; ++g) acc += part[g * n + i];
    out[i] = f2bf(acc);
  }
}

int router_dw_splits(int64_t Tn, int64_t E, int64_t d) {
  const int64_t tiles = cdiv(E, BM) * cdiv(d, BN);
  int64_t s = 256 / (tiles > 0 ? tiles : 1);
  if (s > Tn / 256) s = Tn / 256;
  if (s > 32) s = 32;
  return s < 1 ? 1 : static_cast<int>(s);
}

int router_gemm_splits(int64_t Tn, int64_t E, int64_t d) {
  const int64_t tiles = cdiv(Tn, BM) * cdiv(E, BN);
  int64_t s = 256 / (tiles > 0 ? tiles : 1);
  if (s > d / 512) s = d / 512;  // at least 512 reduction steps per chunk
  if (s > 32) s = 32;
  return s < 1 ? 1 : static_cast<int>(s);
}

// Router scores: logits[T][E] = x[T][d] * wr[E][d]^T.
template <typename T>
hipError_t launch_router_gemm(const T* x, const T* wr, float* logits, int Tn, int E, int d,
                              float* part, int cu, hipStream_t s) {
  Params p = blank();
  p.M = Tn; p.N = E; p.K = d;
  p.A = x; p.lda = d;
  p.B = wr; p.ldb = d;
  p.C = logits; p.ldc = E;
  const int splits = router_gemm_splits(Tn, E, d);
  if (splits <= 1 || !part)
    return run<T, OP_KC, OP_KC, DENSE, EPI_F32, false, false, false>(
        p, cdiv(Tn, BM) * cdiv(E, BN), cu, s);
  // few tokens (decode): too few output tiles to fill the GPU, so the
  // hidden dimension is cut into chunks whose fp32 partials are then added
  p.ngroups = splits;
  p.kchunk = static_cast<int>(cdiv(cdiv(d, splits), 64) * 64);
  p.C = part; p.c_gs = static_cast<int64_t>(Tn) * E;
  hipError_t e = run<T, OP_KC, OP_KC, KGROUP, EPI_F32, false, false, false>(
      p, cdiv(Tn, BM) * cdiv(E, BN) * splits, cu, s);
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(Tn) * E;
  const int grid = static_cast<int>(std::min<int64_t>(cdiv(n, 256), 4096));
  hipLaunchKernelGGL(add_partials_kernel_f32, dim3(grid), dim3(256), 0, s, part, splits, n, logits);
  return hipGetLastError();
}

// h = silu(x_e W_g[e]^T) * (x_e W_u[e]^T) over each expert's rows; a, u, h
// also saved in fp32 for the backward pass when save_a is set.
template <typename T>
hipError_t launch_ffn_gateup(const T* x, const T* wg, const T* wu, const int32_t* offsets,
                             const int32_t* perm, const int32_t* tile_off, int N, int I, int d,
                             int K, int64_t max_rows, T* h, float* save_a, float* save_u,
                             float* save_h, int cu, hipStream_t s) {
  Params p = blank();
  p.N = I; p.K = d; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = x; p.lda = d; p.amap = perm; p.adiv = K;
  p.B = wg; p.B2 = wu; p.ldb = d; p.b_gs = static_cast<int64_t>(I) * d;
  p.C = h; p.ldc = I;
  p.wa = save_a; p.wu = save_u; p.wh = save_h; p.ld_au = I;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(I, BN / 2);
  return run<T, OP_KC, OP_KC, MGROUP, EPI_SWIGLU, true, false, false>(p, ub, cu, s);
}

// y = h W_d[e]^T.
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
  return run<T, OP_KC, OP_KC, MGROUP, EPI_STORE, false, false, false>(p, ub, cu, s);
}

// dh = gs[p] * (dout[tok(p)] W_d[e])  (gs = out_scale * gate of the pick),
// then da = dh*u*silu'(a), du = dh*silu(a) into dadu[P][2I] (fp32).
template <typename T>
hipError_t launch_bwd_down_dh(const T* dout, const int32_t* perm, int K, const float* gs,
                              const T* wd, const float* sa, const float* su,
                              const int32_t* offsets, const int32_t* tile_off, int N, int I,
                              int d, int64_t max_rows, float* dadu, int cu, hipStream_t s) {
  Params p = blank();
  p.N = I; p.K = d; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = dout; p.lda = d; p.amap = perm; p.adiv = K;
  p.B = wd; p.ldb = I; p.b_gs = static_cast<int64_t>(d) * I; p.b_ext = I;
  p.C = dadu; p.ldc = 2 * static_cast<int64_t>(I); p.c2_off = I;
  p.rscale = gs; p.sa = sa; p.su = su; p.ld_au = I;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(I, BN);
  return run<T, OP_KC, OP_MN, MGROUP, EPI_SWIGLU_BWD, true, false, false>(p, ub, cu, s);
}

// dW_d[e] = sum over the expert's rows p of dout[tok(p)]^T (gs[p] h[p]).
template <typename T>
hipError_t launch_bwd_down_dw(const T* dout, const int32_t* perm, int K, const float* hsave,
                              const float* gs, const int32_t* offsets, int N, int I, int d,
                              T* dwd, int cu, hipStream_t s) {
  Params p = blank();
  p.M = d; p.N = I; p.ngroups = N; p.goff = offsets;
  p.A = dout; p.lda = d; p.a_ext = d; p.amap = perm; p.adiv = K;
  p.B = hsave; p.ldb = I; p.b_ext = I; p.kscale = gs;
  p.C = dwd; p.ldc = I; p.c_gs = static_cast<int64_t>(d) * I;
  const int64_t tot = cdiv(d, BM) * cdiv(I, BN) * N;
  if constexpr (is_bf16<T>())
    return run<T, OP_DUP_MN, OP_SPLIT_MN, KGROUP, EPI_STORE, true, false, false>(p, tot, cu, s);
  else
    return run<T, OP_MN, OP_MN, KGROUP, EPI_STORE, true, false, false>(p, tot, cu, s);
}

// Expert dx in dispatch order: dxp = [da | du] [W_g[e] ; W_u[e]] (fp32 out).
template <typename T>
hipError_t launch_bwd_gateup_dx(const float* dadu, const T* wg, const T* wu,
                                const int32_t* offsets, const int32_t* tile_off, int N, int I,
                                int d, int64_t max_rows, float* dxp, int cu, hipStream_t s) {
  Params p = blank();
  p.N = d; p.K = 2 * I; p.ngroups = N; p.goff = offsets; p.tile_off = tile_off;
  p.A = dadu; p.lda = 2 * static_cast<int64_t>(I);
  p.B = wg; p.B2 = wu; p.ldb = d; p.b_gs = static_cast<int64_t>(I) * d; p.b_split = I;
  p.b_ext = d;
  p.C = dxp; p.ldc = d;
  const int64_t ub = (cdiv(max_rows, BM) + N) * cdiv(d, BN);
  if constexpr (is_bf16<T>())
    return run<T, OP_SPLIT_KC, OP_DUP_MN, MGROUP, EPI_F32, false, false, true>(p, ub, cu, s);
  else
    return run<T, OP_KC, OP_MN, MGROUP, EPI_F32, false, false, true>(p, ub, cu, s);
}

// dW_g[e] = da_e^T x_e, dW_u[e] = du_e^T x_e (x rows gathered by perm).
template <typename T>
hipError_t launch_bwd_gateup_dw(const float* dadu, const T* x, const int32_t* offsets,
                                const int32_t* perm, int N, int I, int d, int K, T* dwg, T* dwu,
                                int cu, hipStream_t s) {
  Params p = blank();
  p.M = I; p.N = d; p.ngroups = N; p.goff = offsets;
  p.lda = 2 * static_cast<int64_t>(I); p.a_ext = I;
  p.B = x; p.ldb = d; p.bmap = perm; p.bdiv = K; p.b_ext = d;
  p.ldc = d; p.c_gs = static_cast<int64_t>(I) * d;
  const int64_t tot = cdiv(I, BM) * cdiv(d, BN) * N;
  for (int half = 0; half < 2; ++half) {
    p.A = dadu + static_cast<int64_t>(half) * I;
    p.C = half ? dwu : dwg;
    hipError_t e;
    if constexpr (is_bf16<T>())
      e = run<T, OP_SPLIT_MN, OP_DUP_MN, KGROUP, EPI_STORE, false, true, false>(p, tot, cu, s);
    else
      e = run<T, OP_MN, OP_MN, KGROUP, EPI_STORE, false, true, false>(p, tot, cu, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// dW_r = dl^T x   (dl [T][ldl] fp32, zero-padded columns E..ldl).  The
// output is small (E x d) and the reduction long (T), so with splits > 1 the
// tokens are cut into `splits` chunks, each chunk's product goes to its own
// fp32 partial in `part` ([splits][E][d]), and a second kernel adds the
// partials in chunk order (a fixed order: reproducible).
template <typename T>
hipError_t launch_router_dw(const float* dl, int ldl, const T* x, int Tn, int E, int d, T* dwr,
                            float* part, int cu, hipStream_t s) {
  Params p = blank();
  p.M = E; p.N = d; p.K = Tn;
  p.A = dl; p.lda = ldl; p.a_ext = ldl;
  p.B = x; p.ldb = d; p.b_ext = d;
  p.C = dwr; p.ldc = d;
  const int splits = router_dw_splits(Tn, E, d);
  if (splits <= 1 || !part) {
    const int64_t tot = cdiv(E, BM) * cdiv(d, BN);
    if constexpr (is_bf16<T>())
      return run<T, OP_SPLIT_MN, OP_DUP_MN, DENSE, EPI_STORE, false, false, false>(p, tot, cu, s);
    else
      return run<T, OP_MN, OP_MN, DENSE, EPI_STORE, false, false, false>(p, tot, cu, s);
  }
  p.ngroups = splits;
  p.kchunk = static_cast<int>(cdiv(Tn, splits));
  p.C = part; p.c_gs = static_cast<int64_t>(E) * d;
  const int64_t tot = cdiv(E, BM) * cdiv(d, BN) * splits;
  hipError_t e;
  if constexpr (is_bf16<T>())
    e = run<T, OP_SPLIT_MN, OP_DUP_MN, KGROUP, EPI_F32, false, false, false>(p, tot, cu, s);
  else
    e = run<T, OP_MN, OP_MN, KGROUP, EPI_F32, false, false, false>(p, tot, cu, s);
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(E) * d;
  const int grid = static_cast<int>(std::min<int64_t>(cdiv(n, 256), 4096));
  if constexpr (is_bf16<T>())
    hipLaunchKernelGGL(add_partials_kernel_bf16, dim3(grid), dim3(256), 0, s, part, splits, n, dwr);
  else
    hipLaunchKernelGGL(add_partials_kernel_f32, dim3(grid), dim3(256), 0, s, part, splits, n, dwr);
  return hipGetLastError();
}

// Router part of dx: dxr = dl W_r (fp32 out).
template <typename T>
hipError_t launch_router_dx(const float* dl, int ldl, const T* wr, int Tn, int E, int d,
                            float* dxr, int cu, hipStream_t s) {
  Params p = blank();
  p.M = Tn; p.N = d; p.K = E;
  p.A = dl; p.lda = ldl;
  p.B = wr; p.ldb = d; p.b_ext = d;
  p.C = dxr; p.ldc = d;
  const int64_t tot = cdiv(Tn, BM) * cdiv(d, BN);
  if constexpr (is_bf16<T>())
    return run<T, OP_SPLIT_KC, OP_DUP_MN, DENSE, EPI_F32, false, false, false>(p, tot, cu, s);
  else
    return run<T, OP_KC, OP_MN, DENSE, EPI_F32, false, false, false>(p, tot, cu, s);
}

#define ZC_INST(T)                                                                               \
  template hipError_t launch_router_gemm<T>(const T*, const T*, float*, int, int, int, float*,   \
                                            int, hipStream_t);                                   \
  template hipError_t launch_ffn_gateup<T>(const T*, const T*, const T*, const int32_t*,         \
                                           const int32_t*, const int32_t*, int, int, int, int,   \
                                           int64_t, T*, float*, float*, float*, int,             \
                                           hipStream_t);                                         \
  template hipError_t launch_ffn_down<T>(const T*, const T*, const int32_t*, const int32_t*,     \
                                         int, int, int, int64_t, T*, int, hipStream_t);          \
  template hipError_t launch_bwd_down_dh<T>(const T*, const int32_t*, int, const float*,         \
                                            const T*, const float*, const float*,                \
                                            const int32_t*, const int32_t*, int, int, int,       \
                                            int64_t, float*, int, hipStream_t);                  \
  template hipError_t launch_bwd_down_dw<T>(const T*, const int32_t*, int, const float*,         \
                                            const float*, const int32_t*, int, int, int, T*,     \
                                            int, hipStream_t);                                   \
  template hipError_t launch_bwd_gateup_dx<T>(const float*, const T*, const T*,                  \
                                              const int32_t*, const int32_t*, int, int, int,     \
                                              int64_t, float*, int, hipStream_t);                \
  template hipError_t launch_bwd_gateup_dw<T>(const float*, const T*, const int32_t*,            \
                                              const int32_t*, int, int, int, int, T*, T*, int,   \
                                              hipStream_t);                                      \
  template hipError_t launch_router_dw<T>(const float*, int, const T*, int, int, int, T*,        \
                                          float*, int, hipStream_t);                             \
  template hipError_t launch_router_dx<T>(const float*, int, const T*, int, int, int, float*,    \
                                          int, hipStream_t);
ZC_INST(bf16_t)
ZC_INST(float)
#undef ZC_INST

}  // namespace zc

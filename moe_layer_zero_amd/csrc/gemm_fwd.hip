// Forward expert GEMMs of bf16 layers: gate/up (+ SwiGLU) and down, for
// row-major weights the kernels of gemm_rmw.hip do not take (d or I not a
// multiple of 256).
//
// "LongCat-Flash Technical Report", section 2.1: each FFN expert runs only on
// the tokens routed to it; zero-computation experts never reach this file.
// At the LongCat-Flash shape (d = 6144, I = 2048, section 2.4) most experts
// receive a few hundred rows, so these GEMMs stream every touched expert's
// weights about once and sit near the HBM/matrix-core balance point; the
// design goal is to read each weight panel once and keep the matrix cores fed.
//
//   gate/up: h[p][n] = silu(x[tok(p)] . W_g[e][n]) * (x[tok(p)] . W_u[e][n])
//   down:    y[p][n] = h[p] . W_d[e][n]
// for the rows p of expert e's segment of the dispatch order.
//
// Tiles: 256 rows x 256 MFMA columns per 256-thread workgroup (gate/up: 128
// gate + 128 up columns = 128 columns of h), four wave64s of 128 x 128 each as
// 4 x 4 v_mfma_f32_32x32x16_bf16 blocks accumulating in fp32 (256 accumulator
// registers per lane).  K is staged through LDS in slabs of 64, double-
// buffered: the next slab goes straight from global memory into LDS
// (global_load_lds_dwordx4, no register staging) while the current one is
// multiplied.  An LDS row is 64 bf16 = eight 16-byte chunks; chunk c of row r
// is stored at slot c ^ (r & 7), so the 32 rows a fragment read touches at one
// k land in distinct bank groups.  One workgroup per CU (128 KB of LDS).
// Rows past the end of an expert's segment (and columns past the output)
// load a valid row instead and are never stored.  The training forward's
// variant also writes the gate and up sums a, u and h = silu(a) u in fp32
// (the backward's operands), straight from the accumulators: each half wave
// stores 32 consecutive columns of one row.
// Tile order: expert-major; inside an expert, groups of up to 8 row tiles,
// row tile fastest.  Workgroup b takes logical tiles (b mod 8) * G/8 + b/8 +
// i * G, so each XCD (blocks are dealt to the 8 XCDs round-robin) works on 32
// consecutive tiles at a time: two whole experts of a few hundred rows (their
// x rows read once, each weight panel once), or an 8 x 4 block of a hot
// expert's tiles.
#include "zc_common.h"

namespace zc {
namespace {

constexpr int TM = 256;          // rows per tile
constexpr int TN = 256;          // MFMA columns per tile
constexpr int BK = 32;           // k per slab (one 64-byte LDS row)
constexpr int NSTAGE = 4;        // slabs in flight (LDS ring)
constexpr int NTHR = 256;
constexpr int GMV = 8;           // row tiles per group inside an expert

// FWD_SWIGLU_SAVE: gate/up that also writes a, u and h in fp32 (the training
// forward keeps them for the backward)
enum { FWD_SWIGLU = 0, FWD_STORE = 1, FWD_SWIGLU_SAVE = 2 };

typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct FwdParams {
  int N;                    // experts
  int ncols;                // output columns (I for gate/up, d for down)
  int K;                    // reduction length (d for gate/up, I for down)
  const int32_t* offsets;   // [N+1] rows of each expert in dispatch order
  const int32_t* mt_off;    // [N+1] prefix of ceil(rows / TM)
  const bf16_t* A;          // gate/up: x [T][d] gathered through perm; down: h [P][I]
  const int32_t* perm;      // gate/up only
  int kdiv;                 // K of the layer (slot -> token)
  const bf16_t* B;          // W_g [N][I][d] or W_d [N][d][I]
  const bf16_t* B2;         // W_u (gate/up)
  bf16_t* C;                // h [P][I] or y [P][d]
  float* wa;                // FWD_SWIGLU_SAVE: a, u, h in fp32, [P][I]
  float* wu;
  float* wh;
};

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

typedef __attribute__((address_space(3))) void lds_void;

template <int EPI>
__global__ __launch_bounds__(NTHR, 1) void fwd_kernel(FwdParams p) {
  // NSTAGE (A, B) slab pairs; reused as the output staging tile after the k loop
  __shared__ __align__(16) bf16_t smem[NSTAGE * (TM + TN) * BK];
  auto sA = [&](int buf) { return smem + buf * ((TM + TN) * BK); };
  auto sB = [&](int buf) { return smem + buf * ((TM + TN) * BK) + TM * BK; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool GU = EPI != FWD_STORE;  // gate/up: SwiGLU of gate and up columns
  constexpr int OUTN = GU ? TN / 2 : TN;  // output columns per tile
  const int NT = (p.ncols + OUTN - 1) / OUTN;
  const int64_t total = static_cast<int64_t>(p.mt_off[p.N]) * NT;
  const int G = gridDim.x;
  const int first = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;

  // Slab copy: a slab row is 32 bf16 = four 16-byte chunks; chunk c of row r
  // sits in slot c ^ ((r >> 1) & 3).  Wave w, instruction q fills slots
  // (4w + q) * 64 + lane: row 64w + 16q + lane/4, slot lane%4, holding logical
  // chunk (lane%4) ^ ((row >> 1) & 3).
  const int lrow = 64 * wave + (lane >> 2);
  const int lchunk = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;  // (row >> 1) & 3 == (lane >> 3) & 3

  for (int64_t L = first; L < total; L += G) {
    // ---- which expert, row tile and column tile
    const int lmt = static_cast<int>(L / NT);
    int lo = 0, hi = p.N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.mt_off[mid] <= lmt) lo = mid;
      else hi = mid - 1;
    }
    const int e = lo;
    const int mte = p.mt_off[e + 1] - p.mt_off[e];
    const int q = static_cast<int>(L - static_cast<int64_t>(p.mt_off[e]) * NT);
    const int grp = q / (GMV * NT);
    const int fm = grp * GMV;
    const int gsz = min(GMV, mte - fm);
    const int rr = q - grp * GMV * NT;
    const int mt = fm + rr % gsz;
    const int nt = rr / gsz;
    const int m0 = p.offsets[e] + mt * TM;
    const int mcount = min(TM, p.offsets[e + 1] - m0);
    const int n0 = nt * OUTN;

    // ---- source element offsets of the 8 A rows and 8 B rows this lane copies
    int aoff[4], boff[4];
    const bf16_t* bb0 = p.B + static_cast<int64_t>(e) * p.ncols * p.K;
    const bf16_t* bb1 = GU ? p.B2 + static_cast<int64_t>(e) * p.ncols * p.K : bb0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(lrow + 16 * i, mcount - 1);  // past the segment: any valid row
      const int gm = m0 + row;
      const int src = GU ? p.perm[gm] / p.kdiv : gm;
      aoff[i] = src * p.K + lchunk;
      int col;
      if constexpr (GU)
        col = n0 + ((lrow + 16 * i) & 127);  // rows 0..127 gate, 128..255 up, same columns
      else
        col = n0 + lrow + 16 * i;
      boff[i] = min(col, p.ncols - 1) * p.K + lchunk;
    }
    const bool b_up = GU && wave >= 2;  // this wave's B rows are 128..255

    // 8 loads per wave per slab (4 of A, 4 of B)
    auto fetch = [&](int k0, int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lds_void* da = (lds_void*)(sA(buf) + (64 * wave + 16 * i) * BK);
        __builtin_amdgcn_global_load_lds(p.A + aoff[i] + k0, da, 16, 0, 0);
        lds_void* db = (lds_void*)(sB(buf) + (64 * wave + 16 * i) * BK);
        __builtin_amdgcn_global_load_lds((b_up ? bb1 : bb0) + boff[i] + k0, db, 16, 0, 0);
      }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Fragment addresses.  Block rows differ by multiples of 32, so every
    // row this lane reads has the same (row >> 1) & 3 = (lane >> 1) & 3 and
    // the swizzled chunk offset depends only on the k step: one register per
    // k step, the per-block row offsets are compile-time constants.
    const int s7 = (lane >> 1) & 3;
    const int a_lane = (wm * 128 + (lane & 31)) * BK;
    const int b_lane = ((GU ? wn * 64 : wn * 128) + (lane & 31)) * BK;
    constexpr int jrow[4] = {0, 32, GU ? 128 : 64, GU ? 160 : 96};
    const int khalf = lane >> 5;  // which 8-element half of a 16-k step

    // k loop over a ring of NSTAGE slabs, NSTAGE-1 in flight.  Each slab
    // is 8 loads per wave; every iteration issues one more slab (clamped to
    // the last one, whose repeat lands in a buffer nobody reads again), so
    // exactly 16 loads of this wave are younger than slab kt when it is
    // needed: wait for vmcnt <= 16, then a barrier makes every wave's part
    // of slab kt visible and frees the buffer refilled next.
    const int nk = p.K / BK;
    __syncthreads();  // the previous tile is done with the ring
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s) fetch(min(s, nk - 1) * BK, s);
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt <= 16 (expcnt, lgkmcnt not waited)
      __builtin_amdgcn_s_barrier();
      const bf16_t* a_s = sA(kt % NSTAGE);
      const bf16_t* b_s = sB(kt % NSTAGE);
      bf16x8_t af[2][4], bfr[2][4];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int co = ((2 * ks + khalf) ^ s7) << 3;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[ks][i] = *reinterpret_cast<const bf16x8_t*>(a_s + a_lane + co + 32 * i * BK);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[ks][j] = *reinterpret_cast<const bf16x8_t*>(b_s + b_lane + co + jrow[j] * BK);
      }
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j],
                                                                0, 0, 0);
      // refill the buffer every wave finished with (slab kt-1) with slab kt+3
      fetch(min(kt + NSTAGE - 1, nk - 1) * BK, (kt + NSTAGE - 1) % NSTAGE);
      // issue order: step-0 fragments, then step-0 MFMAs interleaved with the
      // step-1 fragment reads, then step-1 MFMAs interleaved with the 8 slab
      // loads, so neither the LDS nor the load path stalls the matrix pipe
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // all loads landed (the fence waits for them), ring free

    // ---- epilogue: lane holds column lane%32, rows 8*(v/4) + 4*(lane/32) + v%4
    // of each 32 x 32 block.  Results go to an LDS tile first, then out with
    // 16-byte row-contiguous stores.  (32-bit element offsets: the caller
    // keeps rows * columns below 2^31.)
    const int rb0 = wm * 128 + 4 * (lane >> 5);
    bf16_t* st = smem;  // OUTN columns per row
    // saved a, u, h: buffers spanning exactly this tile's rows, so stores to
    // rows past the segment are out of range and dropped by the hardware
    // (unused, and dropped by the compiler, in the other variants)
    // (tile row range made visibly uniform: descriptors live in scalar registers)
    const int64_t so0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(m0)) * p.ncols;
    const int snb = __builtin_amdgcn_readfirstlane(mcount) * p.ncols * 4;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(p.wa + so0, (short)0, snb, 0x00020000);
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(p.wu + so0, (short)0, snb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(p.wh + so0, (short)0, snb, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < (GU ? 2 : 4); ++j) {
        const int cl = (GU ? wn * 64 : wn * 128) + j * 32 + (lane & 31);
        // byte offset of (row rb0 + 32 i, column n0 + cl) from the tile's
        // first row; a column past the output gets an offset past the end
        const int svo = n0 + cl < p.ncols ? ((rb0 + 32 * i) * p.ncols + n0 + cl) * 4 : 0x7fffffff;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = rb0 + 32 * i + 8 * (v >> 2) + (v & 3);
          float val = acc[i][j][v];
          if constexpr (GU) {
            const float u = acc[i][j + 2][v];
            const float hv = silu_f(val) * u;
            if constexpr (EPI == FWD_SWIGLU_SAVE) {
              // one row of 32 consecutive columns per half wave (128-byte
              // pieces); the row step is uniform and goes in the scalar offset
              const int so = (8 * (v >> 2) + (v & 3)) * p.ncols * 4;
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), ra, svo, so, 0);
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, u), ru, svo, so, 0);
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hv), rh, svo, so, 0);
            }
            val = hv;
          }
          st[rl * OUTN + cl] = f2bf(val);
        }
        // keep the scheduler from pulling every accumulator into VGPRs at once
        __builtin_amdgcn_sched_barrier(0);
      }
    __syncthreads();
    constexpr int RC = OUTN / 8;  // 16-byte chunks per row
#pragma unroll 4
    for (int c = tid; c < TM * RC; c += NTHR) {
      const int rl = c / RC, cc = (c % RC) * 8;
      if (rl < mcount && n0 + cc < p.ncols)
        *reinterpret_cast<u32x4_t*>(p.C + (m0 + rl) * p.ncols + n0 + cc) =
            *reinterpret_cast<const u32x4_t*>(st + rl * OUTN + cc);
    }
  }
}

}  // namespace

hipError_t launch_fwd_gateup(const bf16_t* x, const bf16_t* wg, const bf16_t* wu,
                             const int32_t* offsets, const int32_t* perm, const int32_t* mt_off,
                             int N, int I, int d, int K, bf16_t* h, float* save_a, float* save_u,
                             float* save_h, int cu, hipStream_t s) {
  FwdParams p{};
  p.N = N; p.ncols = I; p.K = d;
  p.offsets = offsets; p.mt_off = mt_off;
  p.A = x; p.perm = perm; p.kdiv = K;
  p.B = wg; p.B2 = wu; p.C = h;
  p.wa = save_a; p.wu = save_u; p.wh = save_h;
  if (save_a || save_u || save_h) {
    if (!save_a || !save_u || !save_h) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fwd_kernel<FWD_SWIGLU_SAVE>, dim3(cu), dim3(NTHR), 0, s, p);
  } else {
    hipLaunchKernelGGL(fwd_kernel<FWD_SWIGLU>, dim3(cu), dim3(NTHR), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_down(const bf16_t* h, const bf16_t* wd, const int32_t* offsets,
                           const int32_t* mt_off, int N, int I, int d, bf16_t* y, int cu,
                           hipStream_t s) {
  FwdParams p{};
  p.N = N; p.ncols = d; p.K = I;
  p.offsets = offsets; p.mt_off = mt_off;
  p.A = h; p.B = wd; p.C = y;
  hipLaunchKernelGGL(fwd_kernel<FWD_STORE>, dim3(cu), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace zc

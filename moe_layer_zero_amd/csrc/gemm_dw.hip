// Weight gradients of the FFN experts on gfx950 matrix cores.
//
// "LongCat-Flash Technical Report", section 2.1: each FFN expert sees only
// the tokens routed to it, so its weight gradient is a sum over its own
// rows of the dispatch order:
//   dW_g[e] = sum_p da_p^T x_p,  dW_u[e] = sum_p du_p^T x_p,
//   dW_d[e] = sum_p dout_p^T (g_p h_p),
// for p in offsets[e] .. offsets[e+1].  Generally, per expert,
//   C_e[m][n] = sum_p X[p][m] Y[p][n]
// with both operands stored row by row (the reduction index p is the row).
// X, the fp32 operand (da / du, or g h), comes as an exact bf16 pair
// (hi, lo = bf16(v - hi)) and is contracted twice against its exact bf16
// partner Y, so no value is rounded before the contraction.  dW_d is the
// transpose of such a product (X = g h, Y = dout) and is stored transposed.
//
// Tile: 256 x 256 outputs per 256-thread workgroup; wave w owns rows
// 64w .. 64w+63 of the tile and all 256 columns (2 x 8 blocks of 32 x 32
// fp32 accumulators).  Operand rows stream through a 3-slot LDS ring in
// slabs of 32 rows x 256 columns (16 KB per operand), two slabs in flight
// while one is multiplied, filled by buffer_load ... lds.  The matrix cores
// want 8 consecutive reduction steps
// per lane; ds_read_b64_tr_b16 gives each lane of a 16-lane group one
// column of a 4-row x 16-column block (lane s of the group addresses row
// s/4, columns 4(s%4) .. +3; measured on MI355X), so two such reads turn
// the row-major slab into an MFMA operand without a transposed copy in
// memory.  Inside a slab the 16-byte chunk c of row r is stored at chunk
// c ^ 2(r & 3), which puts the four rows of a transposed read on different
// banks.  Tiles are dealt to the XCDs like the forward GEMMs' (contiguous
// chunks per XCD, claimed from per-XCD counters, then the other XCDs').
#include <utility>

#include "zc_common.h"

namespace zc {
namespace {

constexpr int DK = 32;                 // rows per slab
constexpr int DT = 256;                // tile edge
constexpr int SLAB = DK * DT * 2;      // bytes of one operand slab (16 KB)
constexpr int SLOT = 3 * SLAB;         // split hi, split lo, exact partner
constexpr int NSL = 3;                 // ring slots

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

struct DParams {
  int N;                    // experts
  int M, Ncol;              // product [M][Ncol] per expert (stored transposed if asked)
  const int32_t* offsets;   // [N+1] rows of each expert in dispatch order
  int32_t* sched;           // [8] per-XCD tile counters, zero at launch
  const bf16_t* X;          // split operand, hi part: rows [P][ldx]
  const bf16_t* XL;         // split operand, lo part (same pitch)
  int64_t ldx;
  const bf16_t* Y;          // exact partner: rows [P][ldy]
  int64_t ldy;
  int64_t rows;             // rows of X and Y (range of the loads)
  bf16_t* C;                // output per expert: [M][Ncol], or [Ncol][M] when transposed
};

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// One 16-byte-per-lane copy from a buffer straight into LDS at the
// wave-uniform byte address lds (64 lanes -> 1 KB).  Written as inline asm:
// the compiler would make every transposing LDS read wait for all such
// copies in flight, which would drain the ring each slab.  The copy has no
// register result; the explicit vmcnt waits and barriers of the k loop order
// it with the reads, and nothing else in this kernel uses m0.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

// Fragment f of a slab in read order (see the k loop): kind 0 / 1 = split
// hi / lo column block rb, kind 2 = partner column block nb; ks = 16-row half.
struct Frag { int kind, ks, blk; };
constexpr Frag kFrag[24] = {
    {0, 0, 0}, {0, 0, 1}, {1, 0, 0}, {1, 0, 1}, {2, 0, 0}, {2, 0, 1}, {2, 0, 2}, {2, 0, 3},
    {0, 1, 0}, {2, 0, 4}, {0, 1, 1}, {2, 0, 5}, {1, 1, 0}, {2, 0, 6}, {1, 1, 1}, {2, 0, 7},
    {2, 1, 0}, {2, 1, 1}, {2, 1, 2}, {2, 1, 3}, {2, 1, 4}, {2, 1, 5}, {2, 1, 6}, {2, 1, 7}};
constexpr int frag_index(int kind, int ks, int blk) {
  for (int f = 0; f < 24; ++f)
    if (kFrag[f].kind == kind && kFrag[f].ks == ks && kFrag[f].blk == blk) return f;
  return -1;
}
// MFMA group g = (ks, nb) = (g / 8, g % 8) needs fragments 0 .. need(g) - 1
constexpr int need(int g) {
  int n = frag_index(2, g / 8, g % 8);
  for (int k = 0; k < 2; ++k)
    for (int r = 0; r < 2; ++r) {
      const int f = frag_index(k, g / 8, r);
      n = f > n ? f : n;
    }
  return n + 1;
}
constexpr int kAhead = 2;  // groups between a fragment's read and its first use
// fragments read before group g's MFMAs are issued
constexpr int reads_before(int g) { return need(g + kAhead < 16 ? g + kAhead : 15); }

template <int... G, class F>
__device__ __forceinline__ void each_group(std::integer_sequence<int, G...>, F&& f) {
  (f(std::integral_constant<int, G>{}), ...);
}

// Only for values the compiler has moved out of AGPR accumulators (its
// own, hazard-checked moves): an MFMA result still in a VGPR, read by inline
// asm, is outside the compiler's hazard tracking.
__device__ __forceinline__ bf16_t cvt_bf16(float f) {
  uint32_t r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, 0" : "=v"(r) : "v"(f));
  return static_cast<bf16_t>(r);
}

// One 32x32x16 operand: lane l gets column col0 + l % 32 of rows k0 + 8 (l / 32)
// .. + 7 of a row-major 32 x 256 slab at `slab`.
__device__ __forceinline__ bf16x8_t tr_operand(lds_u8* slab, int k0, int col0, int lane) {
  const int s = lane & 15;
  const int c = col0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);   // first column of the lane's read
  const int kb = k0 + 8 * (lane >> 5) + (s >> 2);
  s16x4_t q[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int k = kb + 4 * r;
    const int a = k * (DT * 2) + (((c >> 3) ^ ((k & 3) << 1)) << 4) + (c & 7) * 2;
    q[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(slab + a));
  }
  // whole-vector casts: a bit cast of a single vector element reads
  // element 0 whatever the index with this compiler
  const bf16x4_t lo = __builtin_bit_cast(bf16x4_t, q[0]);
  const bf16x4_t hi = __builtin_bit_cast(bf16x4_t, q[1]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// TOUT: store the product transposed ([Ncol][M] per expert).
template <bool TOUT>
__global__ __launch_bounds__(256, 1) void dw_kernel(DParams p) {
  __shared__ __align__(16) uint8_t ring[NSL * SLOT + 16];
  int32_t* const s_claim = reinterpret_cast<int32_t*>(ring + NSL * SLOT);
  lds_u8* const ring_lds = (lds_u8*)ring;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int MT = p.M / DT, NT = p.Ncol / DT;
  const int64_t total = static_cast<int64_t>(p.N) * MT * NT;
  const int G = gridDim.x;
  const int C = G / 8;
  int cx = blockIdx.x % 8;
  int hops = 0;
  auto tile_of = [&](int x, int n) -> int64_t {
    return static_cast<int64_t>(n / C) * 8 * C + x * C + n % C;
  };
  // a claimed index n on counter cx -> a tile, or -1 when all are taken
  auto resolve = [&](int n) -> int64_t {
    for (;;) {
      const int64_t L = tile_of(cx, n);
      if (L < total) return L;
      if (++hops == 8) return -1;
      cx = (cx + 1) & 7;
      __syncthreads();
      if (tid == 0) s_claim[0] = atomicAdd(p.sched + cx, 1);
      __syncthreads();
      n = __builtin_amdgcn_readfirstlane(s_claim[0]);
    }
  };

  // Tiles are claimed one ahead: the claim of the next tile is made when a
  // tile starts and published after its k loop, so its atomic's round trip
  // is hidden and no claim waits for the previous tile's output stores.
  if (tid == 0) s_claim[0] = atomicAdd(p.sched + cx, 1);
  __syncthreads();
  int64_t L = resolve(__builtin_amdgcn_readfirstlane(s_claim[0]));
  // operand order in a slot: 0 = split hi, 1 = split lo, 2 = exact partner
  while (L >= 0) {
    int32_t pre = 0;
    if (tid == 0) pre = atomicAdd(p.sched + cx, 1);
    // wave-uniform tile coordinates and row range, in scalar registers (the
    // buffer resources below are built from them; a value the compiler
    // cannot prove uniform would wrap every load in a per-lane loop)
    const int e = __builtin_amdgcn_readfirstlane(static_cast<int>(L / (MT * NT)));
    const int rem = __builtin_amdgcn_readfirstlane(static_cast<int>(L - static_cast<int64_t>(e) * MT * NT));
    const int m0 = (rem / NT) * DT, n0 = (rem % NT) * DT;
    const int r0 = ld_scalar(p.offsets + e);
    const int r1 = ld_scalar(p.offsets + e + 1);
    const int nslab = (r1 - r0 + DK - 1) / DK;
    const int tail = (r1 - r0) - DK * (nslab - 1);   // rows of the last slab
    // the expert's rows only: a load past them returns zeros and reads nothing
    const uint32_t xbytes = static_cast<uint32_t>((r1 - r0) * p.ldx * 2);
    const uint32_t ybytes = static_cast<uint32_t>((r1 - r0) * p.ldy * 2);
    const int xcol = m0, ycol = n0;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(p.X + r0 * p.ldx + xcol), (short)0, xbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rxl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(p.XL + r0 * p.ldx + xcol), (short)0, xbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(p.Y + r0 * p.ldy + ycol), (short)0, ybytes, 0x00020000);
    // lane's rows and source chunks: instruction i of wave w copies rows
    // 8w + 2i + lane/32, chunk lane%32 of the slab from source chunk
    // (lane%32) ^ 2(row & 3)
    uint32_t xo[4], yo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * wave + 2 * i + (lane >> 5);
      const int ch = (lane & 31) ^ ((row & 3) << 1);
      xo[i] = static_cast<uint32_t>(row * p.ldx * 2 + ch * 16);
      yo[i] = static_cast<uint32_t>(row * p.ldy * 2 + ch * 16);
    }
    const uint32_t xstep = static_cast<uint32_t>(DK * p.ldx * 2);
    const uint32_t ystep = static_cast<uint32_t>(DK * p.ldy * 2);
    const uint32_t ring_addr = static_cast<uint32_t>((uintptr_t)ring_lds);  // LDS byte address
    auto issue = [&](int kt, int slot) {
      const uint32_t base = __builtin_amdgcn_readfirstlane(
          ring_addr + slot * SLOT + (8 * wave) * (DT * 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lds_dma16(rx, base + 0 * SLAB + 2 * i * DT * 2, xo[i] + kt * xstep);
        lds_dma16(rxl, base + 1 * SLAB + 2 * i * DT * 2, xo[i] + kt * xstep);
        lds_dma16(ry, base + 2 * SLAB + 2 * i * DT * 2, yo[i] + kt * ystep);
      }
    };

    f32x16_t acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Slab kt (slot kt % 3): the fragments are read in kFrag order, each
    // kAhead MFMA groups before its first use (written out in that order and
    // held there by scheduling groups); slab kt+2's copies go out after the
    // first reads.  Group g = (ks, nb) adds, for rb = 0, 1, the hi and then
    // the lo product of rows 16 ks .. +15 into acc[rb][nb].
    auto step = [&](int kt, int slot) {
      lds_u8* const sb = ring_lds + slot * SLOT;
      bf16x8_t fr[24];
      auto read = [&](int f) {
        const Frag q = kFrag[f];
        fr[f] = q.kind < 2 ? tr_operand(sb + q.kind * SLAB, 16 * q.ks, 64 * wave + 32 * q.blk, lane)
                           : tr_operand(sb + 2 * SLAB, 16 * q.ks, 32 * q.blk, lane);
      };
#pragma unroll
      for (int f = 0; f < reads_before(0); ++f) read(f);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 2 < nslab) issue(kt + 2, (slot + 2) % 3);
      __builtin_amdgcn_sched_barrier(0);
      each_group(std::make_integer_sequence<int, 16>{}, [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int ks = g / 8, nb = g % 8;
        constexpr int f0 = reads_before(g), f1 = g < 15 ? reads_before(g + 1) : 24;
#pragma unroll
        for (int f = f0; f < f1; ++f) read(f);
        const bf16x8_t y = fr[frag_index(2, ks, nb)];
        acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[frag_index(0, ks, 0)], y, acc[0][nb], 0, 0, 0);
        acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[frag_index(0, ks, 1)], y, acc[1][nb], 0, 0, 0);
        acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[frag_index(1, ks, 0)], y, acc[0][nb], 0, 0, 0);
        acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[frag_index(1, ks, 1)], y, acc[1][nb], 0, 0, 0);
      });
      each_group(std::make_integer_sequence<int, 16>{}, [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int nr = (g < 15 ? reads_before(g + 1) : 24) - reads_before(g);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * nr, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      });
      __builtin_amdgcn_sched_barrier(0);
    };

    // per slab: this wave's copies of slab kt done (slab kt+1's may still be
    // in flight), barrier (slab kt visible to every wave, every read of slab
    // kt-1 done, so its slot may refill with slab kt+2).  The rows of the
    // last slab past the expert's end are cleared before use, so the sums do
    // not depend on what an out-of-range lane leaves in LDS.
    __builtin_amdgcn_sched_barrier(0);
    if (nslab > 0) issue(0, 0);
    if (nslab > 1) issue(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < nslab; ++kt) {
      if (kt + 1 < nslab)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int slot = kt % 3;
      if (kt == nslab - 1 && tail < DK) {
        lds_u8* const sb = ring_lds + slot * SLOT + tail * (DT * 2);
        const int per = (DK - tail) * (DT * 2 / 16);   // 16-byte pieces per operand
        const u32x4_t z = {0u, 0u, 0u, 0u};
        for (int q = tid; q < 3 * per; q += 256) {
          const int op = q / per;
          *reinterpret_cast<lds_u32x4*>(sb + op * SLAB + (q - op * per) * 16) = z;
        }
        __syncthreads();
      }
      step(kt, slot);
    }
    __syncthreads();  // every wave done with the ring before the next tile's loads
    if (tid == 0) s_claim[0] = pre;
    __syncthreads();  // published (every thread read the previous claim a tile ago)
    const int next_n = __builtin_amdgcn_readfirstlane(s_claim[0]);

    // ---- epilogue: lane holds column lane%32 of block nb, rows
    // 64 w + 32 rb + 8 (v/4) + 4 (lane/32) + v%4
    bf16_t* Ce = p.C + static_cast<int64_t>(e) * p.M * p.Ncol;
    if constexpr (TOUT) {
      // Transposed: in two passes (rb = 0, 1: product rows 64 w + 32 rb ..
      // + 31 of every wave), the tile goes through the idle ring as output
      // rows n x 128 columns mc = 32 w + (row - 64 w - 32 rb), pitch padded
      // to PT elements against bank conflicts, then out in 16-byte pieces
      // (every 32 columns are contiguous in the output row).
      constexpr int PT = 136;
      bf16_t* st = reinterpret_cast<bf16_t*>(ring);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int nl = 32 * nb + (lane & 31);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int mc = 32 * wave + 8 * g4 + 4 * (lane >> 5);
            const uint32_t w0 = cvt_bf16(acc[rb][nb][4 * g4]) |
                                (static_cast<uint32_t>(cvt_bf16(acc[rb][nb][4 * g4 + 1])) << 16);
            const uint32_t w1 = cvt_bf16(acc[rb][nb][4 * g4 + 2]) |
                                (static_cast<uint32_t>(cvt_bf16(acc[rb][nb][4 * g4 + 3])) << 16);
            *reinterpret_cast<uint2*>(st + nl * PT + mc) = make_uint2(w0, w1);
          }
        }
        __syncthreads();
        for (int c = tid; c < DT * 16; c += 256) {
          const int nl = c >> 4, cc = c & 15;
          const int m = m0 + 32 * rb + 64 * (cc >> 2) + 8 * (cc & 3);
          *reinterpret_cast<u32x4_t*>(Ce + static_cast<int64_t>(n0 + nl) * p.M + m) =
              *reinterpret_cast<const u32x4_t*>(st + nl * PT + 8 * cc);
        }
        __syncthreads();
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int n = n0 + 32 * nb + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int m = m0 + 64 * wave + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            Ce[static_cast<int64_t>(m) * p.Ncol + n] = cvt_bf16(acc[rb][nb][v]);
          }
        }
    }
    L = resolve(next_n);
  }
}

// dst[p] = src[perm[p] / K] for the P rows of the dispatch order (width w
// bf16, a multiple of 8).
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t* __restrict__ src,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets,
                                                          int N, int K, int w,
                                                          bf16_t* __restrict__ dst) {
  const int P = offsets[N];
  const int cpr = w / 8;
  for (int64_t q = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
       q < static_cast<int64_t>(P) * cpr; q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = q / cpr;
    const int c = static_cast<int>(q - row * cpr) * 8;
    const int64_t t = perm[row] / K;
    *reinterpret_cast<u32x4_t*>(dst + row * w + c) =
        *reinterpret_cast<const u32x4_t*>(src + t * w + c);
  }
}

}  // namespace

hipError_t launch_gather_rows(const bf16_t* src, const int32_t* perm, const int32_t* offsets,
                              int N, int K, int w, int64_t max_rows, bf16_t* dst, hipStream_t s) {
  const int64_t want = (max_rows * (w / 8) + 255) / 256;
  const int grid = static_cast<int>(want < 1 ? 1 : (want > 16384 ? 16384 : want));
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, s, src, perm, offsets, N, K, w,
                     dst);
  return hipGetLastError();
}

hipError_t launch_dw(bool transposed, int N, int M, int Ncol, const int32_t* offsets,
                     int32_t* sched, const bf16_t* X, const bf16_t* XL, int64_t ldx, const bf16_t* Y,
                     int64_t ldy, int64_t rows, bf16_t* C, int cu, hipStream_t s) {
  DParams p{};
  p.N = N; p.M = M; p.Ncol = Ncol; p.offsets = offsets; p.sched = sched;
  p.X = X; p.XL = XL; p.ldx = ldx; p.Y = Y; p.ldy = ldy; p.rows = rows; p.C = C;
  if (transposed)
    hipLaunchKernelGGL(dw_kernel<true>, dim3(cu), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(dw_kernel<false>, dim3(cu), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace zc

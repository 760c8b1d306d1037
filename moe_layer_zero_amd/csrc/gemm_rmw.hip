// Grouped expert GEMMs on row-major bf16 weights: the forward (for
// inference, and for training with its activations kept), the backward's dh
// and expert dx, and, on the same pipeline, the dense router product of large
// batches.
//
// "LongCat-Flash Technical Report", section 2.1: each FFN expert runs on the
// rows routed to it (its segment of the dispatch order); zero-computation
// experts never reach these GEMMs.  For the rows p of expert e's segment:
//   gate/up: a = x W_g[e]^T, u = x W_u[e]^T, h = silu(a) u   (training: a, u, h also kept in fp32)
//   down:    y = h W_d[e]^T
//   dh:      dh = g (dout W_d[e])        (fp32; g = out_scale * gate of the row)
//   dx:      dx_e = da W_g[e] + du W_u[e] (fp32; da, du as exact bf16 hi + lo pairs)
//   router:  logits = x W_r^T over all T rows (fp32; section 2.1's router scores)
// with W_g, W_u [N][I][d] and W_d [N][d][I].  The forward contracts weight
// rows with activation rows (the reduction runs along a weight row); dh and
// dx contract over the weight's rows.  The matrix cores want 8 consecutive
// reduction steps per lane: forward weight slabs are read like the
// activations, backward ones with ds_read_b64_tr_b16, which turns a
// row-major slab of 32 weight rows x 256 columns into the operand without a
// transposed copy of the weights in memory (lane s of a 16-lane group reads
// row s/4, columns 4(s%4) .. +3 of a 4 x 16 block and receives one column of
// it).
//
// Tile: up to TM rows (an expert's 32-row blocks spread evenly over its row
// tiles, so its tiles do equal work) x 256 MFMA columns per 256-thread
// workgroup.  Wave w owns columns 64w .. 64w+63 (gate/up: gate and up
// columns 32w .. 32w+31 of h) for every 32-row block that holds rows, as
// 32x32x16 bf16 MFMA blocks accumulating in fp32; a ragged tile multiplies
// only its filled blocks.  Activations and weights stream through a 4-slot
// LDS ring of 32-step slabs, loaded straight into LDS (buffer_load ... lds);
// three slabs are in flight while one is multiplied.  Tiles are dealt to the
// XCDs in contiguous chunks and claimed from per-XCD counters, then from the
// other XCDs' (the scheme of the packed-weight kernels), so the row tiles of
// an expert meet its weight panel in one L2.  Every output element sums its
// 16-step MFMA products in increasing reduction order (dx: hi then lo piece
// at each step).
#include "zc_common.h"

namespace zc {
namespace {

constexpr int BK = 32;             // reduction steps per slab
constexpr int NST = 4;             // ring slots
constexpr int NTHR = 256;
constexpr int GMV = 8;             // row tiles per group inside an expert
constexpr int WSLAB = 256 * BK;    // bf16 of a weight slab (256 x 32, or 32 x 256)

// R_SWIGLU: gate/up with a, u, h also stored in fp32 (training); R_GLU: the
// same product storing h only (inference).  R_DENSE: one dense product
// C = A B^T in fp32 over M rows (the router scores logits = x W_r^T), tiles
// assigned statically instead of claimed.
enum { R_SWIGLU = 0, R_STORE = 1, R_DSWIGLU = 2, R_DX = 3, R_DENSE = 4, R_GLU = 5 };

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16_t lds_bf16;

struct RParams {
  int N;                    // experts
  int M;                    // R_DENSE: rows of the product
  int ncols;                // output columns (gate/up: I, columns of h)
  int K;                    // reduction steps per weight matrix (dx: I, run twice)
  const int32_t* offsets;   // [N+1] rows of each expert in dispatch order
  const int32_t* mt_off;    // [N+1] prefix of the experts' row tiles
  const int32_t* tile_exp;  // [mt_off[N]] expert of each row tile
  int32_t* sched;           // [8] per-XCD tile counters, zero at launch
  const bf16_t* A;          // x [T][d] (gate/up, through perm), h [P][I], dout rows
                            // [P][d], or [da_hi | da_lo | du_hi | du_lo] [P][4I]
  uint32_t a_bytes;         // bytes of A (buffer range; offsets past it load zeros)
  int lda;                  // elements per A row
  const int32_t* perm;      // gate/up: A row of dispatch row p is perm[p] / kdiv
  int kdiv;
  const bf16_t* B;          // W_g (gate/up, dx) or W_d
  const bf16_t* B2;         // W_u (gate/up, dx)
  int ldb;                  // elements per weight row
  int64_t mat;              // elements per expert matrix
  bf16_t* C;                // gate/up: h, down: y ([P][ncols] bf16)
  float* Cf;                // dh or expert dx ([P][ncols] fp32)
  const float* gs;          // dh: out_scale * gate of each dispatch row
  float* sa;                // gate/up: a, u, h in fp32 ([P][I])
  float* su;
  float* sh;
};

// One 16-byte-per-lane buffer load straight into LDS (64 lanes -> 1 KB at dst).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff,
                                          int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// s_waitcnt immediate for "vmcnt <= n" (expcnt and lgkmcnt not waited)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// silu(a) = a / (1 + e^-a) with the hardware reciprocal (about 1 ulp) in
// place of an IEEE division, whose ten-instruction sequence per element would
// make the gate/up epilogue spill.
__device__ __forceinline__ float silu_f(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// fp32 -> bf16, round to nearest even, one instruction per value (the down
// projection's epilogue; as a plain cast the compiler pairs and hoists the
// conversions and the 256-row kernel spills).  Only for values the compiler
// has moved out of AGPR accumulators: an MFMA result still in a VGPR, read
// by inline asm, is outside the compiler's hazard tracking.
__device__ __forceinline__ bf16_t cvt_bf16(float f) {
  uint32_t r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, 0" : "=v"(r) : "v"(f));
  return static_cast<bf16_t>(r);
}

// The four weight operands of a backward slab for one wave: b[ks][cb] holds
// column 64 w + 32 cb + lane%32 of rows 16 ks + 8 (lane/32) .. +7 (two
// transposing reads of 4 rows each).  base[cb] is the lane's LDS byte
// address for ks = 0, first read; the other reads sit at fixed offsets.
// Written as one asm block that waits for its reads: the compiler would
// otherwise make every transposing read wait for all LDS-bound loads in
// flight, which would drain the ring's prefetch each slab.
__device__ __forceinline__ void tr_operands(uint32_t base0, uint32_t base1, bf16x8_t (&b)[2][2]) {
  u32x2_t q0, q1, q2, q3, q4, q5, q6, q7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:8192\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:10240\n\t"
      "ds_read_b64_tr_b16 %4, %9 offset:0\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:8192\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:10240\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(q4), "=&v"(q5), "=&v"(q6), "=&v"(q7)
      : "v"(base0), "v"(base1)
      : "memory");
  auto join = [](u32x2_t lo, u32x2_t hi) {
    const bf16x4_t l = __builtin_bit_cast(bf16x4_t, lo);
    const bf16x4_t h = __builtin_bit_cast(bf16x4_t, hi);
    return __builtin_shufflevector(l, h, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  b[0][0] = join(q0, q1);
  b[1][0] = join(q2, q3);
  b[0][1] = join(q4, q5);
  b[1][1] = join(q6, q7);
}

template <int EPI, int TM>
__global__ __launch_bounds__(NTHR, 1) void rmw_kernel(RParams p) {
  constexpr int RB = TM / 32;                       // 32-row blocks per tile
  constexpr int APC = EPI == R_DX ? 2 : 1;          // dx slabs: hi and lo pieces
  constexpr int AIW = APC * TM / 64;                // A copies per wave per slab (1 KB each)
  constexpr int V = AIW + 4;                        // loads per wave per slab
  constexpr int ASLAB = TM * BK;                    // bf16 of one A piece
  constexpr int SLOT = APC * ASLAB + WSLAB;         // bf16 per ring slot
  constexpr bool TR = EPI == R_DSWIGLU || EPI == R_DX;  // weight rows are reduction steps
  constexpr bool DENSE = EPI == R_DENSE;
  constexpr bool F32OUT = TR || DENSE;              // fp32 results stored from the accumulators
  constexpr bool SWI = EPI == R_SWIGLU || EPI == R_GLU;  // gate/up product
  constexpr bool GATHER = SWI;                      // A rows are token rows
  constexpr int OUTN = SWI ? 128 : 256;             // output columns per tile
  static_assert(TM == 64 || TM == 128 || TM == 256, "tile height");
  static_assert(NST * SLOT * 2 + 64 <= 160 * 1024, "LDS");
  __shared__ __align__(16) bf16_t ring[NST * SLOT + 16];
  int32_t* const s_claim = reinterpret_cast<int32_t*>(ring + NST * SLOT);
  const uint32_t ring_addr = static_cast<uint32_t>((uintptr_t)((lds_bf16*)ring));  // LDS byte address

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = p.ncols / OUTN;
  // dense: one segment of M rows, ceil(M / TM) row tiles
  const int mtd = (p.M + TM - 1) / TM;
  const int64_t total =
      static_cast<int64_t>(DENSE ? mtd : ld_scalar(p.mt_off + p.N)) * NT;
  const int G = gridDim.x;
  const int C = G / 8;
  int cx = blockIdx.x % 8;
  int hops = 0;
  auto tile_of = [&](int x, int n) -> int64_t {
    return static_cast<int64_t>(n / C) * 8 * C + x * C + n % C;
  };
  int cur_n = 0;
  // dense: workgroup b takes tiles (b mod 8) C + b / 8 + i G (a contiguous
  // range per XCD: a row tile's column tiles share their A rows in one L2)
  int64_t Ld = static_cast<int64_t>(blockIdx.x % 8) * C + blockIdx.x / 8;
  if constexpr (!DENSE) {
    if (tid == 0) s_claim[0] = atomicAdd(p.sched + cx, 1);
    __syncthreads();
    cur_n = __builtin_amdgcn_readfirstlane(s_claim[0]);
  }
  const int kseg = p.K / BK;                  // slabs per weight matrix
  const int nk = (EPI == R_DX ? 2 : 1) * kseg;
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.A), (short)0, p.a_bytes, 0x00020000);

  // Slab layouts.  A piece and forward weight slab: rows of 32 steps = four
  // 16-byte chunks, chunk c of row r at c ^ ((r >> 1) & 3); 1 KB copy block b
  // holds rows 16 b .. 16 b + 15 (lane: row 16 b + lane/4, chunk lane%4).
  // Backward weight slab: 32 rows of 256 columns, chunk c of row r at
  // c ^ 2 (r & 3); copy block i of wave w holds rows 8 w + 2 i, +1.
  const int s3 = (lane >> 1) & 3;  // (row >> 1) & 3 of every fragment row of this lane
  const int khalf = lane >> 5;
  const int lchunk = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;  // source chunk of an A / NT copy
  // backward weight reads: byte offset of this lane's first transposing read
  // in a slab, per column block (rows 8 (lane/32) + s/4, columns c .. c+3)
  uint32_t trb[2];
  {
    const int s = lane & 15;
    const int kr = 8 * khalf + (s >> 2);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int c = 64 * wave + 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
      trb[cb] = kr * 512 + (((c >> 3) ^ ((kr & 3) << 1)) << 4) + (c & 7) * 2;
    }
  }

  for (;;) {
    int64_t L;
    int32_t next_n = 0;
    if constexpr (DENSE) {
      L = Ld;
      if (L >= total) break;
      Ld += G;
    } else {
      L = tile_of(cx, cur_n);
      if (L >= total) {
        if (++hops == 8) break;
        cx = (cx + 1) & 7;
        __syncthreads();  // every thread has read the last claim
        if (tid == 0) s_claim[0] = atomicAdd(p.sched + cx, 1);
        __syncthreads();
        cur_n = __builtin_amdgcn_readfirstlane(s_claim[0]);
        continue;
      }
      if (tid == 0) next_n = atomicAdd(p.sched + cx, 1);
    }
    // ---- expert, row tile, column tile (wave-uniform)
    const int lmt = static_cast<int>(L / NT);
    const int e = DENSE ? 0 : ld_scalar(p.tile_exp + lmt);
    const int mt_e = DENSE ? 0 : ld_scalar(p.mt_off + e);
    const int mte = DENSE ? mtd : ld_scalar(p.mt_off + e + 1) - mt_e;
    const int q = static_cast<int>(L - static_cast<int64_t>(mt_e) * NT);
    const int grp = q / (GMV * NT);
    const int fm = grp * GMV;
    const int gsz = min(GMV, mte - fm);
    const int rr = q - grp * GMV * NT;
    const int mt = fm + rr % gsz;
    const int nt = rr / gsz;
    const int seg0 = DENSE ? 0 : ld_scalar(p.offsets + e);
    const int seg1 = DENSE ? p.M : ld_scalar(p.offsets + e + 1);
    const int nbe = (seg1 - seg0 + 31) >> 5;
    const int blo = nbe * mt / mte, bhi = nbe * (mt + 1) / mte;
    const int m0 = seg0 + 32 * blo;
    const int mcount = min(seg0 + 32 * bhi, seg1) - m0;
    const int n0 = nt * OUTN;

    // ---- A copies: this wave's AIW / APC blocks of each piece.  The
    // gathered rows' slots are loaded all at once and without a branch (rows
    // past the tile read its last row's slot, unused), so the loads wait
    // once together instead of one round trip each.
    int src[AIW / APC];
#pragma unroll
    for (int i = 0; i < AIW / APC; ++i) {
      const int gm = m0 + min(16 * ((AIW / APC) * wave + i) + (lane >> 2), mcount - 1);
      src[i] = GATHER ? p.perm[gm] : gm;
    }
    uint32_t aoff[AIW / APC];
#pragma unroll
    for (int i = 0; i < AIW / APC; ++i) {
      const int row = 16 * ((AIW / APC) * wave + i) + (lane >> 2);
      const int tok = GATHER ? src[i] / p.kdiv : src[i];
      // past the tile's rows: out of range, the copy writes zeros, reads nothing
      aoff[i] = row < mcount
                    ? (static_cast<uint32_t>(tok) * static_cast<uint32_t>(p.lda) + lchunk) * 2u
                    : p.a_bytes;
    }
    // ---- weight copies: buffers over expert e's matrices
    const uint32_t mbytes = static_cast<uint32_t>(p.mat * 2);
    const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(p.B + e * p.mat), (short)0, mbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t brsrc2 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>((SWI || EPI == R_DX ? p.B2 : p.B) + e * p.mat), (short)0,
        mbytes, 0x00020000);
    uint32_t boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (TR) {
        const int r = 8 * wave + 2 * i + (lane >> 5);
        const int sc = (lane & 31) ^ ((r & 3) << 1);
        boff[i] = static_cast<uint32_t>((r * p.ldb + n0 + sc * 8) * 2);
      } else {
        const int r = 16 * (4 * wave + i) + (lane >> 2);  // slab row
        const int n = SWI ? n0 + (r & 127) : n0 + r;
        boff[i] = static_cast<uint32_t>((n * p.ldb + lchunk) * 2);
      }
    }
    // gate/up: waves 0, 1 copy gate rows, waves 2, 3 up rows
    const bool b_second = SWI && wave >= 2;

    const int nrb = (mcount + 31) >> 5;
    auto run = [&](auto nrb_c) {
      constexpr int NRB = decltype(nrb_c)::value;
      auto issue = [&](int kt, int slot) {
        bf16_t* const sl = ring + slot * SLOT;
        int ka, kw;  // A column and weight step of the slab
        bool second = b_second;
        if constexpr (EPI == R_DX) {
          const int seg = kt >= kseg ? 1 : 0;
          const int ks = kt - seg * kseg;
          ka = 2 * seg * p.K + ks * BK;  // hi piece; the lo piece is p.K further
          kw = ks * BK;
          second = seg == 1;
        } else {
          ka = kt * BK;
          kw = kt * BK;
        }
#pragma unroll
        for (int h = 0; h < APC; ++h)
#pragma unroll
          for (int i = 0; i < AIW / APC; ++i)
            lds_dma16(arsrc, (lds_void*)(sl + h * ASLAB + ((AIW / APC) * wave + i) * 512), aoff[i],
                      (ka + h * p.K) * 2);
        const int wsoff = TR ? kw * p.ldb * 2 : kw * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lds_void* dst = (lds_void*)(sl + APC * ASLAB + (TR ? (8 * wave + 2 * i) * 256
                                                             : (4 * wave + i) * 512));
          lds_dma16(second ? brsrc2 : brsrc, dst, boff[i], wsoff);
        }
      };

      f32x16_t acc[NRB][2];
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

      // Issue order inside a slab: the weight operands, then the activation
      // fragment reads, each issued three MFMA pairs ahead of the pair that
      // uses it (written out in that order, and held there by scheduling
      // groups: left to itself the compiler reads each fragment just in
      // time and waits for it).  Fragment f = (ks, rb, piece) in that order.
      constexpr int NDS = 2 * APC * NRB;  // activation fragment reads per slab
      constexpr int DS0 = NDS < 3 ? NDS : 3;
      constexpr int BDS = TR ? 0 : 4;     // forward: weight fragment reads
      auto compute = [&](int slot) {
        const bf16_t* const a_s = ring + slot * SLOT + (lane & 31) * BK;
        bf16x8_t b[2][2];
        if constexpr (TR) {
          const uint32_t sb = ring_addr + (slot * SLOT + APC * ASLAB) * 2;
          tr_operands(sb + trb[0], sb + trb[1], b);
          __builtin_amdgcn_sched_barrier(0);
        } else {
          const bf16_t* const w_s = ring + slot * SLOT + ASLAB + (lane & 31) * BK;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int co = ((2 * ks + khalf) ^ s3) << 3;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              const int r0 = SWI ? 128 * cb + 32 * wave : 64 * wave + 32 * cb;
              b[ks][cb] = *reinterpret_cast<const bf16x8_t*>(w_s + r0 * BK + co);
            }
          }
        }
        auto frag = [&](int f) {
          const int ks = f / (APC * NRB), rb = (f / APC) % NRB, piece = f % APC;
          const int co = ((2 * ks + khalf) ^ s3) << 3;
          return *reinterpret_cast<const bf16x8_t*>(a_s + piece * ASLAB + rb * 32 * BK + co);
        };
        bf16x8_t af[NDS];
#pragma unroll
        for (int f = 0; f < DS0; ++f) af[f] = frag(f);
#pragma unroll
        for (int f = 0; f < NDS; ++f) {
          if (f + DS0 < NDS) af[f + DS0] = frag(f + DS0);
          const int ks = f / (APC * NRB), rb = (f / APC) % NRB;
          acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[f], b[ks][0], acc[rb][0], 0, 0, 0);
          acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[f], b[ks][1], acc[rb][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, BDS + DS0, 0);
#pragma unroll
        for (int g = 0; g < NDS - DS0; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * DS0, 0);
      };

      // Slab kt: wait until only the younger slabs' loads (V per slab per
      // wave) are outstanding, barrier (slab kt visible to every wave, the
      // slot of slab kt-1 free), refill that slot with slab kt+3, multiply.
      // Scheduling barriers keep each slab's loads together and in order,
      // which the wait counts assume.
      __builtin_amdgcn_sched_barrier(0);
      issue(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (nk > 1) issue(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      if (nk > 2) issue(2, 2);
      __builtin_amdgcn_sched_barrier(0);
      // (the last slab is multiplied after the loop: with it inside, the
      // compiler moves every accumulator out to VGPRs at the loop exit and
      // spills)
      for (int kt = 0; kt < nk - 1; ++kt) {
        if (kt + 2 < nk)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(V));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 3 < nk) issue(kt + 3, (kt + 3) & 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      compute((nk - 1) & 3);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DENSE) {
        // the last slab's MFMAs stay here: the compiler otherwise moves them
        // into the epilogue and keeps their operands in scratch
#pragma unroll
        for (int i = 0; i < NRB; ++i) asm volatile("" ::"a"(acc[i][0]), "a"(acc[i][1]));
      }

      // ---- epilogue: lane holds column lane%32 of its column block and rows
      // 32 rb + 8 (v/4) + 4 (lane/32) + v%4
      const int rbase = 4 * khalf;
      if constexpr (EPI == R_DX || DENSE) {
        // fp32 results straight from the accumulators: each store covers 32
        // consecutive columns (128 bytes) of a row, through a buffer that
        // spans exactly the tile's rows (stores past them are dropped, no
        // branch per row): expert dx 0.83 -> 0.81 ms per training step.
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            p.Cf + static_cast<int64_t>(m0) * p.ncols, (short)0,
            static_cast<uint32_t>(mcount) * static_cast<uint32_t>(p.ncols) * 4u, 0x00020000);
        // (router: the row pitch made opaque here, otherwise the compiler
        // computes every store's offset once, before the tile loop, and keeps
        // the 256 of them in scratch: router scores 0.274 -> 0.252 ms at
        // prefill; the expert dx kernel does not spill and is faster without)
        int pitch = p.ncols;
        if constexpr (DENSE) asm volatile("" : "+s"(pitch));
        const int cbase = n0 + 64 * wave + (lane & 31);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              // (expert dx: written as below it measured 1% faster than
              // with the router's form)
              const uint32_t off =
                  DENSE ? static_cast<uint32_t>(rl * pitch + cbase + 32 * cb) * 4u
                        : static_cast<uint32_t>(rl * p.ncols + n0 + 64 * wave + 32 * cb +
                                                (lane & 31)) * 4u;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rb][cb][v]), cr, off, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!DENSE) {
          if (tid == 0) s_claim[0] = next_n;
        }
        __syncthreads();  // every wave done reading the ring before the next tile's loads
        return;
      } else if constexpr (F32OUT) {
        // fp32 results straight from the accumulators: each store covers 32
        // consecutive columns (128 bytes) of a row.  (For dh the form above
        // with the gate scales staged in LDS measured 0.38 against 0.30 ms.)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
            if (rl < mcount) {
              const int64_t gm = m0 + rl;
              const float g = EPI == R_DSWIGLU ? p.gs[gm] : 1.0f;
#pragma unroll
              for (int cb = 0; cb < 2; ++cb) {
                const int n = n0 + 64 * wave + 32 * cb + (lane & 31);
                p.Cf[gm * p.ncols + n] = EPI == R_DSWIGLU ? acc[rb][cb][v] * g : acc[rb][cb][v];
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!DENSE) {
          if (tid == 0) s_claim[0] = next_n;
        }
        __syncthreads();  // every wave done reading the ring before the next tile's loads
        return;
      }
      // bf16 output staged in the ring (free once every wave is past the
      // barrier), then written with 16-byte row-contiguous stores
      __syncthreads();
      bf16_t* const st = ring;  // OUTN columns per row
      if constexpr (EPI == R_SWIGLU) {
        // a, u, h in fp32 go out from the accumulators through buffers that
        // span exactly this tile's rows: a store to a row past the segment
        // is out of range and dropped
        const int64_t so0 = static_cast<int64_t>(m0) * p.ncols;
        const uint32_t snb = static_cast<uint32_t>(mcount * p.ncols * 4);
        const __amdgpu_buffer_rsrc_t ra =
            __builtin_amdgcn_make_buffer_rsrc(p.sa + so0, (short)0, snb, 0x00020000);
        const __amdgpu_buffer_rsrc_t ru =
            __builtin_amdgcn_make_buffer_rsrc(p.su + so0, (short)0, snb, 0x00020000);
        const __amdgpu_buffer_rsrc_t rh =
            __builtin_amdgcn_make_buffer_rsrc(p.sh + so0, (short)0, snb, 0x00020000);
        const int cl = 32 * wave + (lane & 31);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const int vo = ((rbase + 32 * rb) * p.ncols + n0 + cl) * 4;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
            const float av = acc[rb][0][v], uv = acc[rb][1][v];
            const float hv = silu_f(av) * uv;
            const int so = (8 * (v >> 2) + (v & 3)) * p.ncols * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, av), ra, vo, so, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, uv), ru, vo, so, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hv), rh, vo, so, 0);
            st[rl * OUTN + cl] = f2bf(hv);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else if constexpr (EPI == R_GLU) {
        const int cl = 32 * wave + (lane & 31);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
            st[rl * OUTN + cl] = f2bf(silu_f(acc[rb][0][v]) * acc[rb][1][v]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              st[rl * OUTN + 64 * wave + 32 * cb + (lane & 31)] = cvt_bf16(acc[rb][cb][v]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      constexpr int RC = OUTN / 8;  // 16-byte chunks per row
#pragma unroll 4
      for (int c = tid; c < mcount * RC; c += NTHR) {
        const int rl = c / RC, cc = (c % RC) * 8;
        *reinterpret_cast<u32x4_t*>(p.C + static_cast<int64_t>(m0 + rl) * p.ncols + n0 + cc) =
            *reinterpret_cast<const u32x4_t*>(st + rl * OUTN + cc);
      }
      if (tid == 0) s_claim[0] = next_n;
      __syncthreads();  // staging read before the next tile's loads refill the ring
    };
    switch (nrb) {
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: if constexpr (RB >= 2) run(std::integral_constant<int, 2>{}); break;
      case 3: if constexpr (RB >= 4) run(std::integral_constant<int, 3>{}); break;
      case 4: if constexpr (RB >= 4) run(std::integral_constant<int, 4>{}); break;
      case 5: if constexpr (RB >= 8) run(std::integral_constant<int, 5>{}); break;
      case 6: if constexpr (RB >= 8) run(std::integral_constant<int, 6>{}); break;
      case 7: if constexpr (RB >= 8) run(std::integral_constant<int, 7>{}); break;
      default: if constexpr (RB >= 8) run(std::integral_constant<int, 8>{}); break;
    }
    if constexpr (!DENSE) cur_n = __builtin_amdgcn_readfirstlane(s_claim[0]);
  }
}

typedef void (*rmw_fn)(RParams);
rmw_fn pick(int epi, int tm) {
#define ZC_RMW_TM(E)                              \
  switch (tm) {                                   \
    case 64: return rmw_kernel<E, 64>;            \
    case 128: return rmw_kernel<E, 128>;          \
    case 256: return rmw_kernel<E, 256>;          \
  }                                               \
  return nullptr;
  switch (epi) {
    case R_SWIGLU: ZC_RMW_TM(R_SWIGLU)
    case R_GLU: ZC_RMW_TM(R_GLU)
    case R_STORE: ZC_RMW_TM(R_STORE)
    case R_DSWIGLU:  // backward: up to 128 rows (dx's two A pieces fill the ring;
                     // a 256-row dh tile would spill)
      switch (tm) {
        case 64: return rmw_kernel<R_DSWIGLU, 64>;
        case 128: return rmw_kernel<R_DSWIGLU, 128>;
      }
      return nullptr;
    case R_DX:
      switch (tm) {
        case 64: return rmw_kernel<R_DX, 64>;
        case 128: return rmw_kernel<R_DX, 128>;
      }
      return nullptr;
    case R_DENSE:
      return tm == 256 ? rmw_kernel<R_DENSE, 256> : nullptr;
  }
#undef ZC_RMW_TM
  return nullptr;
}

hipError_t launch(int epi, int tm, const RParams& p, int cu, hipStream_t s) {
  rmw_fn k = pick(epi, tm);
  const int outn = epi == R_SWIGLU || epi == R_GLU ? 128 : 256;
  if (!k || cu % 8 || p.ncols % outn || p.K % BK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, dim3(cu), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool rmw_fwd_supported(int64_t rows, int64_t Tn, int64_t d, int64_t I) {
  // buffer offsets into x (gate/up), h (down) and one weight matrix; h, y and
  // the fp32 saves are addressed with 64-bit row offsets
  const int64_t lim = int64_t(1) << 31;
  return d % 256 == 0 && I % 256 == 0 && d * I * 2 < lim && Tn * d * 2 < lim &&
         (rows + 64) * I * 2 < lim;
}

bool rmw_supported(int64_t rows, int64_t Tn, int64_t d, int64_t I) {
  const int64_t lim = int64_t(1) << 31;
  return d % 256 == 0 && I % 256 == 0 && d * I * 2 < lim && (rows + 64) * 4 * I * 2 < lim &&
         (rows + 64) * d * 2 < lim && Tn * d * 2 < lim && rows * I * 4 < lim && rows * d * 4 < lim;
}

hipError_t launch_rmw_gateup(const bf16_t* x, int64_t Tn, const bf16_t* wg, const bf16_t* wu,
                             const int32_t* offsets, const int32_t* perm, const int32_t* mt_off,
                             const int32_t* tile_exp, int32_t* sched, int tm, int N, int I, int d,
                             int K, bf16_t* h, float* sa, float* su, float* sh, int cu,
                             hipStream_t s) {
  const bool save = sa != nullptr;  // training: a, u, h in fp32 as well
  if (save != (su != nullptr) || save != (sh != nullptr)) return hipErrorInvalidValue;
  RParams p{};
  p.N = N; p.ncols = I; p.K = d;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = x; p.a_bytes = static_cast<uint32_t>(Tn * d * 2); p.lda = d; p.perm = perm; p.kdiv = K;
  p.B = wg; p.B2 = wu; p.ldb = d; p.mat = static_cast<int64_t>(I) * d;
  p.C = h; p.sa = sa; p.su = su; p.sh = sh;
  return launch(save ? R_SWIGLU : R_GLU, tm, p, cu, s);
}

hipError_t launch_rmw_down(const bf16_t* h, int64_t rows, const bf16_t* wd,
                           const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                           int32_t* sched, int tm, int N, int I, int d, bf16_t* y, int cu,
                           hipStream_t s) {
  RParams p{};
  p.N = N; p.ncols = d; p.K = I;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = h; p.a_bytes = static_cast<uint32_t>(rows * I * 2); p.lda = I;
  p.B = wd; p.ldb = I; p.mat = static_cast<int64_t>(d) * I;
  p.C = y;
  return launch(R_STORE, tm, p, cu, s);
}

hipError_t launch_rmw_dh(const bf16_t* doutd, int64_t rows, const bf16_t* wd,
                         const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                         int32_t* sched, int tm, int N, int I, int d, const float* gs, float* dh,
                         int cu, hipStream_t s) {
  RParams p{};
  p.N = N; p.ncols = I; p.K = d;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = doutd; p.a_bytes = static_cast<uint32_t>(rows * d * 2); p.lda = d;
  p.B = wd; p.ldb = I; p.mat = static_cast<int64_t>(d) * I;
  p.gs = gs; p.Cf = dh;
  return launch(R_DSWIGLU, tm, p, cu, s);
}

bool rmw_dense_supported(int64_t M, int64_t n, int64_t K) {
  const int64_t lim = int64_t(1) << 31;
  return n % 256 == 0 && K % BK == 0 && M * K * 2 < lim && n * K * 2 < lim && M * n * 4 < lim;
}

hipError_t launch_rmw_dense(const bf16_t* a, int64_t M, const bf16_t* b, int n, int K, float* c,
                            int cu, hipStream_t s) {
  if (!rmw_dense_supported(M, n, K)) return hipErrorInvalidValue;
  RParams p{};
  p.N = 1; p.M = static_cast<int>(M); p.ncols = n; p.K = K;
  p.A = a; p.a_bytes = static_cast<uint32_t>(M * K * 2); p.lda = K;
  p.B = b; p.ldb = K; p.mat = static_cast<int64_t>(n) * K;
  p.Cf = c;
  return launch(R_DENSE, 256, p, cu, s);
}

hipError_t launch_rmw_dx(const bf16_t* hilo, int64_t rows, const bf16_t* wg, const bf16_t* wu,
                         const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                         int32_t* sched, int tm, int N, int I, int d, float* dxp, int cu,
                         hipStream_t s) {
  RParams p{};
  p.N = N; p.ncols = d; p.K = I;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = hilo; p.a_bytes = static_cast<uint32_t>(rows * 4 * I * 2); p.lda = 4 * I;
  p.B = wg; p.B2 = wu; p.ldb = d; p.mat = static_cast<int64_t>(I) * d;
  p.Cf = dxp;
  return launch(R_DX, tm, p, cu, s);
}

}  // namespace zc

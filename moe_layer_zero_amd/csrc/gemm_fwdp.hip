// Forward expert GEMMs of bf16 inference layers on packed expert weights.
//
// "LongCat-Flash Technical Report", section 2.1: each FFN expert runs only on
// the tokens routed to it; zero-computation experts never reach this file.
//
//   gate/up: h[p][n] = silu(x[tok(p)] . W_g[e][n]) * (x[tok(p)] . W_u[e][n])
//   down:    y[p][n] = h[p] . W_d[e][n]
// for the rows p of expert e's segment of the dispatch order.
//
// At the LongCat-Flash shape (d = 6144, I = 2048, 512 experts, section 2.4)
// an expert gets a few hundred rows, so each weight panel is streamed from
// HBM about once and the GEMMs sit at the HBM/matrix-core balance point.
// Two properties of the memory system shape this kernel:
//  - a compute unit returns its loads in issue order, so loads that hit L2
//    (the gathered activations) wait behind loads that miss to HBM (the
//    weights): both streams get the same prefetch distance;
//  - HBM delivers full speed only for whole 128-byte lines: every request
//    here covers whole lines.
//
// Weights are used in the packed layout of zc_moe_pack_weights: for each 32
// output columns and 16 reduction steps, the 1 KB that a wave's 64 lanes feed
// to one v_mfma_f32_32x32x16_bf16 as its B operand (lane l: column l % 32,
// reduction steps 8 (l / 32) .. + 7).  Weights therefore go straight from
// global memory into registers with 1 KB contiguous loads: no LDS, no barrier.
//
// Tile: 256 rows x 256 MFMA columns per 256-thread workgroup (gate/up: 128
// gate + 128 up columns = 128 columns of h; the 256-row down projection
// runs the eight-wave variant below, down8_kernel).  Wave w owns all 256 rows and 64
// columns (gate/up: 32 gate + the matching 32 up columns, so SwiGLU is done
// in registers): 8 x 2 blocks of 32 x 32 fp32 accumulators (256 registers).
// Activation rows are staged through a 4-slot LDS ring, 64 reduction steps
// (one 128-byte row piece) per slot, filled by buffer_load ... lds; rows past
// the expert's segment load from outside the buffer (no traffic, never
// stored).  Chunk c (16 bytes) of LDS row r sits in slot c ^ ((r >> 1) & 7),
// which keeps every 16-lane phase of a fragment read on distinct banks.
// Three slabs (A and B) are in flight while one is multiplied.
// Tile order: expert-major; inside an expert, groups of up to 8 row tiles,
// row tile fastest.  The tiles are dealt to the 8 XCDs in chunks of
// consecutive tiles, so the row tiles sharing a weight panel read it from
// the same L2, and an XCD's workgroups claim its tiles from a counter.
#include <type_traits>

#include "zc_common.h"

namespace zc {
namespace {

constexpr int BK = 64;      // reduction steps per slab
constexpr int NST = 4;      // LDS ring slots
constexpr int NTHR = 256;
constexpr int GMV = 8;      // row tiles per group inside an expert
constexpr int DSDEPTH = 4;  // fragment reads ahead of their MFMAs (eight-wave kernel)

// P_SWIGLU: gate/up with SwiGLU; P_STORE: down projection (bf16 y).
enum { P_SWIGLU = 0, P_STORE = 1 };

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

struct PParams {
  int N;                    // experts
  int ncols;                // output columns (I for gate/up, d for down)
  int K;                    // reduction length (d for gate/up, I for down)
  const int32_t* offsets;   // [N+1] rows of each expert in dispatch order
  const int32_t* mt_off;    // [N+1] prefix of ceil(rows / TM)
  const int32_t* tile_exp;  // [mt_off[N]] expert of each row tile
  int32_t* sched;           // [8] per-XCD tile counters, zero at launch
  const bf16_t* A;          // gate/up: x [T][d] gathered through perm; down: h [P][I]
  uint32_t a_bytes;         // bytes of A (buffer range; offsets past it load nothing)
  const int32_t* perm;      // gate/up only
  int kdiv;                 // K of the layer (slot -> token)
  const bf16_t* B;          // packed W_g or W_d
  const bf16_t* B2;         // packed W_u (gate/up)
  bf16_t* C;                // h [P][I] or y [P][d]
};

// silu(a) = a / (1 + e^-a) with the hardware reciprocal (about 1 ulp) in
// place of an IEEE division: the result is rounded to bf16 (or quantized to
// FP8) right after, and the division's ten-instruction sequence per element
// is the larger part of the gate/up epilogue.
__device__ __forceinline__ float silu_f(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// fp32 -> bf16, round to nearest even (NaN stays NaN), one conversion
// instruction per value, for the down projection's epilogue.  Written as an
// opaque instruction: as a plain cast the compiler pairs and hoists the
// conversions, and the 256-row kernel then spills inside its k loop.  (The
// gate/up epilogue keeps f2bf: with any branch-free rounding there the
// register allocator spills inside the k loop as well.)
// Only for values the compiler has moved out of AGPR accumulators (its
// own, hazard-checked moves): an MFMA result still in a VGPR, read by inline
// asm, is outside the compiler's hazard tracking.
__device__ __forceinline__ bf16_t cvt_bf16(float f) {
  uint32_t r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, 0" : "=v"(r) : "v"(f));
  return static_cast<bf16_t>(r);
}

// One 16-byte-per-lane buffer load straight into LDS (64 lanes -> 1 KB at
// dst).  Kept out of the kernel templates: the host pass drops template
// kernels that use this builtin in a dependent context.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff,
                                          int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// Workgroup barrier ordering LDS accesses only: unlike __syncthreads it
// does not wait for global loads in flight (the next tile's slabs).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate for "vmcnt <= n" (expcnt and lgkmcnt not waited)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// TM: rows per tile (32, 64, 128 or 256).  A slab's loads are issued right
// after its barrier, ahead of its fragment reads and MFMAs (spreading them
// over the MFMAs measured slower for the 256-row gate/up tiles).  The
// weight fragments are loaded with the non-temporal hint: each weight byte
// is used by the tiles of one expert only, and so marked the stream ran
// 4% faster at prefill (gate/up) and 6% faster at decode, though the
// L2-miss bytes did not drop.  (The eight-wave down kernel keeps plain
// loads: there the hint slowed it and the combine that reads its output.)
template <int EPI, int TM>
__global__ __launch_bounds__(NTHR, 1) void fwdp_kernel(PParams p) {
  constexpr int RB = TM / 32;       // 32-row blocks per tile = A loads per wave per slab
  constexpr int SLOT = TM * BK;  // bf16 per ring slot
  constexpr int V = RB + 8;      // loads per wave per slab (A rows + 8 B blocks)
  static_assert(TM == 32 || TM == 64 || TM == 128 || TM == 256, "tile height");
  // the ring, then one int: the next tile index claimed by thread 0 (kept in
  // the same LDS object, see the note on the tables of the decode)
  __shared__ __align__(16) bf16_t ring[NST * SLOT + 16];
  int32_t* const s_claim = reinterpret_cast<int32_t*>(ring + NST * SLOT);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  constexpr int OUTN = EPI == P_SWIGLU ? 128 : 256;  // output columns per tile
  constexpr bool GATHER = EPI == P_SWIGLU;  // A rows are token rows
  const int NT = p.ncols / OUTN;
  const int64_t total = static_cast<int64_t>(ld_scalar(p.mt_off + p.N)) * NT;
  const int G = gridDim.x;
  // Tiles are dealt to the 8 XCDs in chunks of G/8 consecutive tiles, round
  // robin (blocks are dealt to the XCDs round robin, so block b runs on XCD
  // b mod 8): the row tiles sharing a weight panel meet in one L2.  Inside an
  // XCD the workgroups claim the XCD's tiles in order from a counter, so a
  // workgroup that drew cheap (ragged) tiles takes more of them and all
  // finish together.  Tile n of XCD x is (n / C) * 8C + x C + n % C.
  const int xcd = blockIdx.x % 8;
  const int C = G / 8;
  // When its own XCD's tiles are all claimed, a workgroup goes on with the
  // next XCD's counter, and so on round the 8: the XCDs finish together
  // instead of waiting for the one that drew the most work.
  int cx = xcd;
  int hops = 0;
  auto tile_of = [&](int x, int n) -> int64_t {
    return static_cast<int64_t>(n / C) * 8 * C + x * C + n % C;
  };
  if (tid == 0) s_claim[0] = atomicAdd(p.sched + cx, 1);
  __syncthreads();
  int cur_n = __builtin_amdgcn_readfirstlane(s_claim[0]);
  const int nk = p.K / BK;
  const int kblk = p.K / 16;  // packed 1 KB blocks per 32 output columns

  // A buffer resource: raw, range-checked against a_bytes
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.A), (short)0, p.a_bytes, 0x00020000);

  // Slab copy of A: instruction i of wave w fills the 1 KB block b = RB w + i
  // of a slot, i.e. rows 8b + lane/8, slot lane%8, which holds logical chunk
  // (lane%8) ^ ((row >> 1) & 7) = (lane%8) ^ ((4b + lane/16) & 7).
  // Fragment reads: rows 32 rb + lane%32 all have (row >> 1) & 7 = (lane >> 1) & 7.
  const int s7 = (lane >> 1) & 7;
  const int khalf = lane >> 5;
  const int frag_lane = (lane & 31) * BK;

  for (;;) {
    const int64_t L = tile_of(cx, cur_n);
    if (L >= total) {
      if (++hops == 8) break;
      cx = (cx + 1) & 7;
      __syncthreads();  // every thread has read the last claim
      if (tid == 0) s_claim[0] = atomicAdd(p.sched + cx, 1);
      __syncthreads();
      cur_n = __builtin_amdgcn_readfirstlane(s_claim[0]);
      continue;
    }
    // claim the next tile now; its index is published in the epilogue
    int32_t next_n = 0;
    if (tid == 0) next_n = atomicAdd(p.sched + cx, 1);
    // ---- which expert, row tile and column tile
    const int lmt = static_cast<int>(L / NT);
    const int e = ld_scalar(p.tile_exp + lmt);
    const int mt_e = ld_scalar(p.mt_off + e);
    const int mte = ld_scalar(p.mt_off + e + 1) - mt_e;
    const int q = static_cast<int>(L - static_cast<int64_t>(mt_e) * NT);
    const int grp = q / (GMV * NT);
    const int fm = grp * GMV;
    const int gsz = min(GMV, mte - fm);
    const int rr = q - grp * GMV * NT;
    const int mt = fm + rr % gsz;
    const int nt = rr / gsz;
    // the expert's 32-row blocks spread evenly over its mte row tiles (at
    // most TM / 32 each), so the row tiles that share a weight panel do the
    // same work, stream the panel at the same pace and find it in L2
    const int seg0 = ld_scalar(p.offsets + e), seg1 = ld_scalar(p.offsets + e + 1);
    const int nbe = (seg1 - seg0 + 31) >> 5;
    const int blo = nbe * mt / mte, bhi = nbe * (mt + 1) / mte;
    const int m0 = seg0 + 32 * blo;
    const int mcount = min(seg0 + 32 * bhi, seg1) - m0;
    const int n0 = nt * OUTN;

    // ---- byte offsets of the RB A row pieces this lane copies per slab.
    // The gathered rows' slots are loaded all at once and without a branch
    // (rows past the tile read its last row's slot, unused), so the RB
    // loads wait once together instead of one round trip each.
    int src[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int gm = m0 + min(8 * (RB * wave + i) + (lane >> 3), mcount - 1);
      src[i] = GATHER ? p.perm[gm] : gm;
    }
    uint32_t aoff[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int b = RB * wave + i;
      const int row = 8 * b + (lane >> 3);
      const int chunk = (lane & 7) ^ ((4 * b + (lane >> 4)) & 7);
      const int tok = GATHER ? src[i] / p.kdiv : src[i];
      // past the tile's rows: out of range, the load returns zeros, reads nothing
      aoff[i] = row < mcount
                    ? (static_cast<uint32_t>(tok) * static_cast<uint32_t>(p.K) + chunk * 8) * 2u
                    : p.a_bytes;
    }
    // ---- packed B: this wave's two column groups of 32
    const int64_t mat = static_cast<int64_t>(p.ncols) * p.K;
    const bf16_t* b0;
    const bf16_t* b1;
    if constexpr (EPI == P_SWIGLU) {
      const int g = n0 / 32 + wave;
      b0 = p.B + e * mat + static_cast<int64_t>(g) * kblk * 512 + lane * 8;
      b1 = p.B2 + e * mat + static_cast<int64_t>(g) * kblk * 512 + lane * 8;
    } else {
      const int g = n0 / 32 + 2 * wave;
      b0 = p.B + e * mat + static_cast<int64_t>(g) * kblk * 512 + lane * 8;
      b1 = b0 + static_cast<int64_t>(kblk) * 512;
    }

    // The tile's pipeline, specialised on the number of 32-row blocks that
    // hold rows (NRB): a ragged last tile of an expert multiplies and reads
    // only those, instead of all TM rows.
    const int nrb = (mcount + 31) >> 5;
    auto run = [&](auto nrb_c) {
      constexpr int NRB = decltype(nrb_c)::value;
      bf16x8_t bq[NST][2][4];  // B fragments of the slabs in flight
      auto issue = [&](int kt, int slot, bf16x8_t (&bf)[2][4]) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          lds_void* dst = (lds_void*)(ring + slot * SLOT + (RB * wave + i) * 8 * BK);
          lds_dma16(arsrc, dst, aoff[i], kt * BK * 2);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          bf[0][t] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(b0 + (4 * kt + t) * 512));
          bf[1][t] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(b1 + (4 * kt + t) * 512));
        }
      };

      f32x16_t acc[NRB][2];
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

      // fragment f = t NRB + rb (reduction step t, row block rb).  For 4 to
      // 6 occupied row blocks the scheduler, left to itself, waits for each
      // fragment read right before its MFMAs in two slabs of every four;
      // there the reads are written three fragments ahead in program order.
      auto compute = [&](int slot, const bf16x8_t (&bf)[2][4]) {
        const bf16_t* a_s = ring + slot * SLOT + frag_lane;
        if constexpr (NRB >= 4 && NRB <= 6) {
          constexpr int NF = 4 * NRB;
          auto frag = [&](int f) {
            const int t = f / NRB, rb = f % NRB;
            return *reinterpret_cast<const bf16x8_t*>(a_s + rb * 32 * BK + (((2 * t + khalf) ^ s7) << 3));
          };
          bf16x8_t a[4];
#pragma unroll
          for (int f = 0; f < 3; ++f) a[f] = frag(f);
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            if (f + 3 < NF) a[(f + 3) & 3] = frag(f + 3);
            const int t = f / NRB, rb = f % NRB;
            acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f & 3], bf[0][t], acc[rb][0], 0, 0, 0);
            acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[f & 3], bf[1][t], acc[rb][1], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int co = ((2 * t + khalf) ^ s7) << 3;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
              const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(a_s + rb * 32 * BK + co);
              acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[0][t], acc[rb][0], 0, 0, 0);
              acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[1][t], acc[rb][1], 0, 0, 0);
            }
          }
        }
      };

      // Issue order inside a slab (4 NRB fragment reads, 8 NRB MFMAs, V loads):
      // loads first; fragment reads run up to three ahead of the MFMAs that
      // use them.
      constexpr int NDS = 4 * NRB;
      constexpr int DS0 = NDS < 3 ? NDS : 3;
      auto sched = [&](bool with_loads) {
        if (with_loads) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, DS0, 0);
#pragma unroll
        for (int g = 0; g < NDS - DS0; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * DS0, 0);
      };

      // Slab kt: wait until at most the loads of the two younger slabs in
      // flight are outstanding (V per slab per wave), barrier (slab kt visible
      // to every wave, slot of slab kt-1 free), refill that slot with slab
      // kt+3, multiply slab kt.  K is a multiple of 4 BK, so the loop runs in
      // groups of four slabs with static buffer indexes.  The wait counts
      // assume the loads of different slabs are never interleaved: scheduling
      // barriers keep each slab's loads together, in slab order.
      __builtin_amdgcn_sched_barrier(0);
      issue(0, 0, bq[0]);
      __builtin_amdgcn_sched_barrier(0);
      issue(1, 1, bq[1]);
      __builtin_amdgcn_sched_barrier(0);
      issue(2, 2, bq[2]);
      __builtin_amdgcn_sched_barrier(0);
      int kt = 0;
      for (; kt < nk - 4; kt += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
          __builtin_amdgcn_s_barrier();
          issue(kt + u + 3, (u + 3) & 3, bq[(u + 3) & 3]);
          compute(u, bq[u]);
          sched(true);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // last four slabs: slab nk-1 is issued at nk-4, then the pipeline drains
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      issue(kt + 3, 3, bq[3]);
      compute(0, bq[0]);
      sched(true);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      compute(1, bq[1]);
      sched(false);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(V));
      __builtin_amdgcn_s_barrier();
      compute(2, bq[2]);
      sched(false);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_s_barrier();
      compute(3, bq[3]);
      sched(false);
      __builtin_amdgcn_sched_barrier(0);

      // ---- epilogue: lane holds column lane%32 of its column group and rows
      // 32 rb + 8 (v/4) + 4 (lane/32) + v%4.
      const int rbase = 4 * khalf;
      // The bf16 tile is staged in the ring (free once every wave has passed
      // the barrier below; TM x OUTN bf16 fit in its 4 TM x 64), then written
      // out with 16-byte row-contiguous stores; the last barrier keeps the
      // next tile's loads from refilling the ring before the staging is read.
      __syncthreads();  // every wave done reading the ring
      bf16_t* st = ring;  // OUTN columns per row
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
          if constexpr (EPI == P_SWIGLU) {
            st[rl * OUTN + 32 * wave + (lane & 31)] = f2bf(silu_f(acc[rb][0][v]) * acc[rb][1][v]);
          } else {
            st[rl * OUTN + 64 * wave + (lane & 31)] = cvt_bf16(acc[rb][0][v]);
            st[rl * OUTN + 64 * wave + 32 + (lane & 31)] = cvt_bf16(acc[rb][1][v]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
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
    cur_n = __builtin_amdgcn_readfirstlane(s_claim[0]);
  }
}

constexpr int NTHR8 = 512;

// The down projection on 256-row tiles (the prefill shape), eight waves:
// two per SIMD, each owning all 256 rows of the tile and one group of 32
// output columns (8 accumulator blocks, 128 registers), so the pair of waves
// on a SIMD fits one register file and one wave's matrix work covers the
// other's waits.  Every wave reads the whole A slab from the shared LDS ring
// (LDS reads with eight waves per CU measure above 170 bytes per clock on
// this part).  Each A fragment feeds a single MFMA here, so the fragment
// reads must run ahead of their MFMAs (four in flight): a kernel whose
// register allocation left one fragment register, each read waited for
// before its MFMA, kept the matrix cores about half busy.  What makes room
// for the four fragments: one code path for every tile (all eight row
// blocks multiplied; rows past the tile's end are zeros, at this workload
// 13% of the MFMAs), weight fragments loaded through a buffer resource
// (scalar base, one lane-offset register) and every per-tile value in
// scalar registers.
//
// The next tile's first three slabs are loaded under this tile's last three
// slabs and its epilogue, so the weight stream does not stop between tiles.
// The next tile is known four slabs before the end: its claim went out
// during the previous tile's drain (a vector atomic whose result thread 0
// first reads after more than two slabs of younger loads, so the slab waits
// already cover it).  The epilogue stages the tile in two halves of 128
// rows through ring slot 3 and 32 KB past the ring (slots 0 to 2 are
// receiving the next tile meanwhile) and writes 16-byte row pieces through a
// buffer resource that ends at the tile's last row.  Every slab wait is
// "vmcnt <= 2V": loads return in issue order, so with two younger slabs of V
// loads each in flight the awaited slab has landed, whatever stores or
// atomics are interleaved (they only make a wait stricter).
// Measured at the prefill workload: 3.71 ms against 4.02 ms for the same
// eight-wave split with per-row-block code paths and a drained pipeline
// between tiles.
__global__ __launch_bounds__(NTHR8, 1) void down8_kernel(PParams p) {
  constexpr int TM = 256;
  constexpr int SLOT = TM * BK;  // bf16 per ring slot (32 KB)
  constexpr int AW = 4;          // A copies per wave per slab
  constexpr int V = AW + 4;      // loads per wave per slab
  constexpr int OUTN = 256;
  constexpr int HR = 128;        // rows per staging half
  // ring slots 0..3, then 32 KB: staging = slot 3 + that (HR x OUTN bf16,
  // 160 KB in all); s_next (the next tile, written by thread 0 four slabs
  // before a tile's end and read by every wave after that slab's barrier)
  // sits inside the staging, which is only written in the epilogue
  __shared__ __align__(16) bf16_t lds[5 * SLOT];
  bf16_t* const ring = lds;
  bf16_t* const stage = lds + 3 * SLOT;
  int32_t* const s_next = reinterpret_cast<int32_t*>(lds + 4 * SLOT);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = p.ncols / OUTN;
  const int64_t total = static_cast<int64_t>(ld_scalar(p.mt_off + p.N)) * NT;
  const int G = gridDim.x;
  const int C = G / 8;
  const int nk = p.K / BK;
  const int kblk = p.K / 16;
  const int64_t mat = static_cast<int64_t>(p.ncols) * p.K;
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.A), (short)0, p.a_bytes, 0x00020000);
  const int s7 = (lane >> 1) & 7;
  const int khalf = lane >> 5;
  const int frag_lane = (lane & 31) * BK;

  // ---- tile claims (thread 0 only): per-XCD counters, then the other XCDs'
  int cx = blockIdx.x % 8;
  int hops = 0;
  auto resolve = [&](int32_t n) -> int32_t {
    int64_t L = static_cast<int64_t>(n / C) * 8 * C + cx * C + n % C;
    while (L >= total) {
      if (++hops >= 8) return -1;
      cx = (cx + 1) & 7;
      const int32_t m = atomicAdd(p.sched + cx, 1);
      L = static_cast<int64_t>(m / C) * 8 * C + cx * C + m % C;
    }
    return static_cast<int32_t>(L);
  };

  // ---- a tile: its rows and columns (wave-uniform, scalar registers)
  struct Tile {
    int m0, mcount, n0;
    uint32_t abase;                // byte offset of row m0 in A
    __amdgpu_buffer_rsrc_t brsrc;  // this wave's packed weight column group
  };
  auto locate = [&](int32_t L, Tile& t) {
    const int lmt = L / NT;
    const int e = ld_scalar(p.tile_exp + lmt);
    const int mt_e = ld_scalar(p.mt_off + e);
    const int mte = ld_scalar(p.mt_off + e + 1) - mt_e;
    const int q = L - mt_e * NT;
    const int grp = q / (GMV * NT);
    const int fm = grp * GMV;
    const int gsz = min(GMV, mte - fm);
    const int rr = q - grp * GMV * NT;
    const int mt = fm + rr % gsz;
    const int nt = rr / gsz;
    const int seg0 = ld_scalar(p.offsets + e), seg1 = ld_scalar(p.offsets + e + 1);
    const int nbe = (seg1 - seg0 + 31) >> 5;
    const int blo = nbe * mt / mte, bhi = nbe * (mt + 1) / mte;
    t.m0 = seg0 + 32 * blo;
    t.mcount = min(seg0 + 32 * bhi, seg1) - t.m0;
    t.n0 = nt * OUTN;
    t.abase = static_cast<uint32_t>(t.m0) * static_cast<uint32_t>(p.K) * 2u;
    const bf16_t* bw = p.B + e * mat + static_cast<int64_t>(t.n0 / 32 + wave) * kblk * 512;
    t.brsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(bw), (short)0,
                                                static_cast<uint32_t>(kblk) * 1024u, 0x00020000);
  };
  // this lane's A copies: copy i of wave w covers rows 8 (4 w + i) + lane/8
  // of the tile, 16 bytes at chunk (lane%8) ^ ((4 (4 w + i) + lane/16) % 8);
  // that chunk depends on i only through i % 2.  A copy past the tile's rows
  // loads from outside the buffer (no data).
  const int lrow = lane >> 3;
  uint32_t achunk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    achunk[j] = (static_cast<uint32_t>(lrow) * static_cast<uint32_t>(p.K) +
                 (((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) * 8)) * 2u;
  const uint32_t blane = lane * 16;  // byte offset of this lane's piece of a 1 KB block

  bf16x8_t bq[NST][4];  // B fragments of the slabs in flight
  auto issue = [&](const Tile& t, int kt, int slot, bf16x8_t (&bf)[4]) {
#pragma unroll
    for (int i = 0; i < AW; ++i) {
      const int b = AW * wave + i;
      lds_void* dst = (lds_void*)(ring + slot * SLOT + b * 8 * BK);
      const uint32_t off = lrow < t.mcount - 8 * b
                               ? t.abase + static_cast<uint32_t>(8 * b) * static_cast<uint32_t>(p.K) * 2u + achunk[i & 1]
                               : p.a_bytes;
      lds_dma16(arsrc, dst, off, kt * BK * 2);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      bf[u] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(t.brsrc, blane, (4 * kt + u) * 1024, 0));
  };

  // ---- first tile, and the claim of the second
  int32_t pend = 0;
  if (tid == 0) {
    const int32_t L0 = resolve(atomicAdd(p.sched + cx, 1));
    if (L0 >= 0) pend = atomicAdd(p.sched + cx, 1);
    s_next[0] = L0;
  }
  __syncthreads();
  int32_t Lc = __builtin_amdgcn_readfirstlane(s_next[0]);
  if (Lc < 0) return;
  Tile tc;
  locate(Lc, tc);
  __builtin_amdgcn_sched_barrier(0);
  issue(tc, 0, 0, bq[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue(tc, 1, 1, bq[1]);
  __builtin_amdgcn_sched_barrier(0);
  issue(tc, 2, 2, bq[2]);
  __builtin_amdgcn_sched_barrier(0);

  for (;;) {
    int32_t Ln = -1;
    Tile tn;
    {
      constexpr int NRB = 8;  // every row block: rows past the tile's end are zeros
      f32x16_t acc[NRB];
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
      auto compute = [&](int slot, const bf16x8_t (&bf)[4]) {
        const bf16_t* a_s = ring + slot * SLOT + frag_lane;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int co = ((2 * t + khalf) ^ s7) << 3;
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(a_s + rb * 32 * BK + co);
            acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[t], acc[rb], 0, 0, 0);
          }
        }
      };
      constexpr int NDS = 4 * NRB;
      constexpr int DS0 = NDS < DSDEPTH ? NDS : DSDEPTH;
      auto sched = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, DS0, 0);
#pragma unroll
        for (int g = 0; g < NDS - DS0; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, DS0, 0);
      };
      int kt = 0;
      for (; kt < nk - 4; kt += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
          __builtin_amdgcn_s_barrier();
          issue(tc, kt + u + 3, (u + 3) & 3, bq[(u + 3) & 3]);
          compute(u, bq[u]);
          sched();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // slab nk-4: the next tile is named (its claim was issued a whole tile
      // ago) and located
      if (tid == 0) s_next[0] = pend < 0 ? -1 : resolve(pend);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      issue(tc, kt + 3, 3, bq[3]);
      __builtin_amdgcn_sched_barrier(0);
      Ln = __builtin_amdgcn_readfirstlane(s_next[0]);
      if (Ln >= 0) {
        locate(Ln, tn);
      } else {
        tn = tc;  // no next tile: the drain re-reads this tile's first slabs, unused
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(0, bq[0]);
      __builtin_amdgcn_sched_barrier(0);
      // slabs nk-3 .. nk-1, each with one of the next tile's first three
      // slabs in flight; the claim of the tile after it goes out first
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      if (tid == 0) pend = Ln >= 0 ? atomicAdd(p.sched + cx, 1) : -1;
      issue(tn, 0, 0, bq[0]);
      compute(1, bq[1]);
      sched();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      issue(tn, 1, 1, bq[1]);
      compute(2, bq[2]);
      sched();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      issue(tn, 2, 2, bq[2]);
      compute(3, bq[3]);
      sched();
      __builtin_amdgcn_sched_barrier(0);

      // ---- epilogue: lane holds column lane%32 of its group and rows
      // 32 rb + 8 (v/4) + 4 (lane/32) + v%4; two halves of 128 rows, each
      // staged (bf16) and written with 16-byte row-contiguous stores.  The
      // stores go through a buffer resource ending at the tile's last row,
      // so rows past it are dropped by the range check, without branches.
      const int rbase = 4 * khalf;
      constexpr int RC = OUTN / 8;  // 16-byte chunks per row
      const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
          p.C + static_cast<int64_t>(tc.m0) * p.ncols, (short)0,
          static_cast<uint32_t>(tc.mcount) * static_cast<uint32_t>(p.ncols) * 2u, 0x00020000);
      const int srow = tid / RC, scol = (tid % RC) * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h * HR >= tc.mcount) break;
        lds_barrier();  // slot 3 read by every wave / the first half stored
#pragma unroll
        for (int rb = 4 * h; rb < 4 * h + 4; ++rb) {
          if (rb < NRB) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rl = rbase + 32 * (rb - 4 * h) + 8 * (v >> 2) + (v & 3);
              stage[rl * OUTN + 32 * wave + (lane & 31)] =
                  __builtin_bit_cast(bf16_t, static_cast<__bf16>(acc[rb][v]));
            }
          }
        }
        lds_barrier();
        const uint32_t obase =
            (static_cast<uint32_t>(h * HR + srow) * static_cast<uint32_t>(p.ncols) +
             static_cast<uint32_t>(tc.n0 + scol)) * 2u;
        const uint32_t ostep = static_cast<uint32_t>(NTHR8 / RC) * static_cast<uint32_t>(p.ncols) * 2u;
#pragma unroll
        for (int i = 0; i < HR * RC / NTHR8; ++i) {
          const u32x4_t vv =
              *reinterpret_cast<const u32x4_t*>(stage + (srow + i * (NTHR8 / RC)) * OUTN + scol);
          __builtin_amdgcn_raw_buffer_store_b128(vv, crsrc, obase + i * ostep, 0, 0);
        }
      }
      // with fewer than eight slabs the next tile writes s_next (in the
      // staging) before its first barrier: every wave has read the staging
      if (nk < 8) lds_barrier();
    }
    if (Ln < 0) break;
    tc = tn;
  }
  // the unused slabs of the drain land in LDS before the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// SwiGLU backward of the FFN picks in dispatch order, from dh = g (dout W_d)
// and the a, u, h the forward saved (all fp32, [P][I]):
//   da = dh u silu'(a), du = dh silu(a), silu'(a) = s (1 + a (1 - s)), s = sigmoid(a),
// and g h (the down projection's weight-gradient operand), each written as an
// exact bf16 pair (hi, lo = bf16(v - hi)): hilo [P][4I] = da_hi, da_lo, du_hi,
// du_lo; ghlo [P][2I] = (g h)_hi, (g h)_lo.  One thread per 8 consecutive
// columns of a row: 16-byte loads and stores.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const float* __restrict__ dh, const float* __restrict__ gs, const float* __restrict__ sa,
    const float* __restrict__ su, const float* __restrict__ sh, const int32_t* __restrict__ offsets,
    int N, int I, bf16_t* __restrict__ hilo, bf16_t* __restrict__ ghlo) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const int64_t P = offsets[N];
  const int cpr = I / 8;
  auto pack = [](float x0, float x1) -> uint32_t {
    return static_cast<uint32_t>(f2bf(x0)) | (static_cast<uint32_t>(f2bf(x1)) << 16);
  };
  for (int64_t q = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; q < P * cpr;
       q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = q / cpr;
    const int c = static_cast<int>(q - row * cpr) * 8;
    const int64_t o = row * I + c;
    const float g = gs[row];
    float va[8], vu[8], vg[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(dh + o + 4 * h);
      const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(sa + o + 4 * h);
      const f32x4_t u4 = *reinterpret_cast<const f32x4_t*>(su + o + 4 * h);
      const f32x4_t h4 = *reinterpret_cast<const f32x4_t*>(sh + o + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = a4[j];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
        va[4 * h + j] = d4[j] * u4[j] * (sg * (1.0f + a * (1.0f - sg)));
        vu[4 * h + j] = d4[j] * (a * sg);
        vg[4 * h + j] = g * h4[j];
      }
    }
    // hi parts, then lo parts = the rounding residue of each
    u32x4_t w[6];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x[3][2] = {{va[2 * j], va[2 * j + 1]}, {vu[2 * j], vu[2 * j + 1]},
                             {vg[2 * j], vg[2 * j + 1]}};
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float h0 = bf2f(f2bf(x[k][0])), h1 = bf2f(f2bf(x[k][1]));
        w[2 * k][j] = pack(h0, h1);
        w[2 * k + 1][j] = pack(x[k][0] - h0, x[k][1] - h1);
      }
    }
    bf16_t* hl = hilo + row * 4 * I + c;
    *reinterpret_cast<u32x4_t*>(hl) = w[0];
    *reinterpret_cast<u32x4_t*>(hl + I) = w[1];
    *reinterpret_cast<u32x4_t*>(hl + 2 * I) = w[2];
    *reinterpret_cast<u32x4_t*>(hl + 3 * I) = w[3];
    bf16_t* gl = ghlo + row * 2 * I + c;
    *reinterpret_cast<u32x4_t*>(gl) = w[4];
    *reinterpret_cast<u32x4_t*>(gl + I) = w[5];
  }
}

// Packed layout of one [R][C] weight matrix (R output columns, C reduction
// steps): element (r, c) sits at
//   ((r / 32) * (C / 16) + c / 16) * 512 + (r % 32 + 32 * ((c / 8) % 2)) * 8 + c % 8.
// One thread writes one 16-byte chunk (8 consecutive c of one r).
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ src,
                                                   bf16_t* __restrict__ dst, int64_t nchunks,
                                                   int R, int C) {
  const int64_t per_mat = static_cast<int64_t>(R) * C / 8;
  const int kb = C / 16;
  for (int64_t q = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; q < nchunks;
       q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t m = q / per_mat;
    const int64_t o = q - m * per_mat;
    const int64_t blk = o >> 6;
    const int l = static_cast<int>(o & 63);
    const int64_t r = (blk / kb) * 32 + (l & 31);
    const int64_t c = (blk % kb) * 16 + (l >> 5) * 8;
    const int64_t base = m * R * static_cast<int64_t>(C);
    *reinterpret_cast<u32x4_t*>(dst + base + o * 8) =
        *reinterpret_cast<const u32x4_t*>(src + base + r * C + c);
  }
}

// Kernel of each (epilogue, tile height); tiles of up to 64 rows leave room
// for two workgroups per CU.  The 256-row down projection runs the
// eight-wave down8_kernel (launch_tm).
typedef void (*fwdp_fn)(PParams);
fwdp_fn pick_kernel(int epi, int tm, int* per_cu) {
  *per_cu = tm <= 64 ? 2 : 1;
  if (epi == P_SWIGLU) {
    switch (tm) {
      case 32: return fwdp_kernel<P_SWIGLU, 32>;
      case 64: return fwdp_kernel<P_SWIGLU, 64>;
      case 128: return fwdp_kernel<P_SWIGLU, 128>;
      case 256: return fwdp_kernel<P_SWIGLU, 256>;
    }
  } else {
    switch (tm) {
      case 32: return fwdp_kernel<P_STORE, 32>;
      case 64: return fwdp_kernel<P_STORE, 64>;
      case 128: return fwdp_kernel<P_STORE, 128>;

    }
  }
  return nullptr;
}

hipError_t launch_tm(int epi, int tm, const PParams& p, int cu, hipStream_t s) {
  if (tm == 256 && epi == P_STORE) {
    hipLaunchKernelGGL(down8_kernel, dim3(cu), dim3(NTHR8), 0, s, p);
    return hipGetLastError();
  }
  int per_cu = 1;
  fwdp_fn k = pick_kernel(epi, tm, &per_cu);
  if (!k) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, dim3(per_cu * cu), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Rows per tile for a layer whose FFN experts average `avg_rows` rows: the
// smallest of 32, 64, 128, 256 that covers the average (few rows: the GEMMs
// only stream weights, so padding rows cost matrix-core time and power for
// nothing; many rows: 256-row tiles read each weight panel least often).
int fwdp_rows_per_tile(int64_t avg_rows) {
  if (avg_rows <= 32) return 32;
  if (avg_rows <= 64) return 64;
  if (avg_rows <= 128) return 128;
  return 256;
}

hipError_t launch_fwdp_gateup(const bf16_t* x, int64_t x_elems, const bf16_t* wg_p,
                              const bf16_t* wu_p, const int32_t* offsets, const int32_t* perm,
                              const int32_t* mt_off, const int32_t* tile_exp, int32_t* sched,
                              int tm, int N, int I, int d, int K, bf16_t* h, int cu,
                              hipStream_t s) {
  PParams p{};
  p.N = N; p.ncols = I; p.K = d;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = x; p.a_bytes = static_cast<uint32_t>(x_elems * 2); p.perm = perm; p.kdiv = K;
  p.B = wg_p; p.B2 = wu_p; p.C = h;
  return launch_tm(P_SWIGLU, tm, p, cu, s);
}

hipError_t launch_fwdp_down(const bf16_t* h, int64_t h_elems, const bf16_t* wd_p,
                            const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                            int32_t* sched, int tm, int N, int I, int d, bf16_t* y, int cu,
                            hipStream_t s) {
  PParams p{};
  p.N = N; p.ncols = d; p.K = I;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = h; p.a_bytes = static_cast<uint32_t>(h_elems * 2);
  p.B = wd_p; p.C = y;
  return launch_tm(P_STORE, tm, p, cu, s);
}

hipError_t launch_swiglu_bwd(const float* dh, const float* gs, const float* sa, const float* su,
                             const float* sh, const int32_t* offsets, int N, int I,
                             int64_t max_rows, bf16_t* hilo, bf16_t* ghlo, hipStream_t s) {
  const int64_t want = (max_rows * (I / 8) + 255) / 256;
  const int grid = static_cast<int>(want < 1 ? 1 : (want > 16384 ? 16384 : want));
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid), dim3(256), 0, s, dh, gs, sa, su, sh, offsets,
                     N, I, hilo, ghlo);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const bf16_t* src, bf16_t* dst, int64_t nmat, int R, int C,
                               hipStream_t s) {
  const int64_t nchunks = nmat * R * static_cast<int64_t>(C) / 8;
  if (nchunks == 0) return hipSuccess;
  const int64_t want = (nchunks + 255) / 256;
  const int grid = static_cast<int>(want < 16384 ? want : 16384);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, src, dst, nchunks, R, C);
  return hipGetLastError();
}

}  // namespace zc

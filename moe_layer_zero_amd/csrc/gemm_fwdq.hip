// Forward expert GEMMs with FP8 blockwise-quantized operands (MXFP8).
//
// The LongCat deployment quantizes the expert GEMMs blockwise to FP8 and
// keeps sensitive parts in higher precision ("LongCat-Flash Technical
// Report" series blog, deployment notes).  On gfx950 the matrix cores take
// blockwise FP8 natively: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E4M3
// operands and applies one power-of-two scale (E8M0) per 32 reduction
// steps of every row and column, the OCP Microscaling format MXFP8.  So the
// blocks here are 32 values along the reduction dimension with an E8M0
// scale; weights are quantized once at load time, the gathered activations
// x once per call, and h inside the gate/up epilogue.  The router, the
// gates, the combine and the zero-computation experts (which return the
// unquantized x) stay in bf16 / fp32.
//
// Quantization of a block of 32 values v (the same rule everywhere):
//   S = biased exponent of max|v| minus 8, at least 0 (E8M0 of
//       2^(floor(log2 max|v|) - 8), 0 for an all-zero block);
//   code_i = E4M3 of v_i * 2^(127 - S), nearest with ties to even, after
//            clamping to +-448 (the conversion instruction rounds to nearest
//            even; without the clamp it returns NaN past 464).
//
// Matrix-core operand layout of one 32x32x64 step (measured on MI355X):
// lane l feeds row (or column) l % 32; with h = l / 32, its bytes 0..15 are
// reduction steps 16h .. 16h+15 and its bytes 16..31 are steps 32+16h ..
// 32+16h+15; the scale operand of lane l is the E8M0 of its row and of the
// 32-step block l / 32 of the step.
//
// Storage:
//  - activations (x', h'): codes row-major [rows][K]; scales [rows][K/32]
//    with each group of 4 blocks (one 128-step slab) stored in the order
//    (0, 2, 1, 3), so that lane half h finds the scales of both 64-step
//    MFMA steps of a slab in one 16-bit word at byte 2h of the group;
//  - weights [R][C] (R output columns, C reduction steps): codes in 1 KB
//    pieces [R/32][C/128][step 2][half 2][lane 64][16], lane l = column
//    32g + l%32 with h = l/32, piece "half" holding bytes 16*half .. of the
//    lane's 32-byte operand; then scales [R/32][C/128][lane 64] 16-bit words
//    (block 4t + h, block 4t + 2 + h) of column 32g + l%32.  A quantized
//    weight set is the N experts' codes followed by their scales.
#include <type_traits>

#include "zc_common.h"

namespace zc {
namespace {

constexpr int BKQ = 128;      // reduction steps per slab (128 bytes per row)
constexpr int NST = 4;        // LDS ring slots
constexpr int NTHR = 256;
constexpr int GMV = 8;        // row tiles per group inside an expert
// per-slot scale area: activation scales of 256 rows (1 KB), then weight
// scales of each wave's two column groups (4 waves x 2 x 256 B)
constexpr int SC_A = 1024;
constexpr int SC_BYTES = SC_A + 2048;

enum { Q_SWIGLU = 0, Q_STORE = 1 };

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct QParams {
  int N;                     // experts
  int ncols;                 // output columns (I for gate/up, d for down)
  int K;                     // reduction length (d for gate/up, I for down)
  const int32_t* offsets;    // [N+1] rows of each expert in dispatch order
  const int32_t* mt_off;     // [N+1] prefix of ceil(rows / TM)
  const int32_t* tile_exp;   // [mt_off[N]] expert of each row tile
  int32_t* sched;            // [8] per-XCD tile counters, zero at launch
  const uint8_t* A;          // codes: x' [T][d] gathered through perm, or h' [P][I]
  uint32_t a_bytes;
  const uint8_t* As;         // activation scales [rows][K/32]
  uint32_t as_bytes;
  const int32_t* perm;       // gate/up only
  int kdiv;                  // K of the layer (slot -> token)
  const uint8_t* B;          // quantized W_g or W_d (codes, then scales)
  const uint8_t* B2;         // quantized W_u (gate/up)
  uint8_t* Cq;               // gate/up: h' codes [P][I]
  uint8_t* Cs;               // gate/up: h' scales [P][I/32]
  bf16_t* Cb;                // down: y [P][d]
};

// silu(a) = a / (1 + e^-a) with the hardware reciprocal (about 1 ulp) in
// place of an IEEE division: the result is rounded to bf16 (or quantized to
// FP8) right after, and the division's ten-instruction sequence per element
// is the larger part of the gate/up epilogue.
__device__ __forceinline__ float silu_f(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Only for values the compiler has moved out of AGPR accumulators (its
// own, hazard-checked moves): an MFMA result still in a VGPR, read by inline
// asm, is outside the compiler's hazard tracking.
__device__ __forceinline__ bf16_t cvt_bf16(float f) {
  uint32_t r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, 0" : "=v"(r) : "v"(f));
  return static_cast<bf16_t>(r);
}

// E8M0 scale of a block whose largest magnitude is amax (finite, >= 0).
__device__ __forceinline__ int mx_scale(float amax) {
  const int be = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  return be > 8 ? be - 8 : 0;
}

// E4M3 code of v at scale S.
__device__ __forceinline__ uint32_t mx_code(float v, int S) {
  float q = __builtin_ldexpf(v, 127 - S);
  q = fminf(fmaxf(q, -448.f), 448.f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.f, 0, false)) & 0xffu;
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff,
                                          int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, lds_void* dst, uint32_t voff,
                                         int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, soff, 0, 0);
}

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// TM rows x 256 MFMA columns per workgroup (gate/up: 128 gate + 128 up
// columns), wave w owning all TM rows and 64 columns, as in the bf16 kernel;
// one slab = 128 reduction steps = two MFMA steps.
template <int EPI, int TM>
__global__ __launch_bounds__(NTHR, 1) void fwdq_kernel(QParams p) {
  constexpr int RB = TM / 32;
  constexpr int SLOT = TM * BKQ + SC_BYTES;  // bytes per ring slot: codes, then scales
  constexpr int V = RB + 11;                 // loads per wave per slab
  static_assert(TM == 32 || TM == 64 || TM == 128 || TM == 256, "tile height");
  __shared__ __align__(16) uint8_t ring[NST * SLOT + 16];
  int32_t* const s_claim = reinterpret_cast<int32_t*>(ring + NST * SLOT);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  constexpr int OUTN = EPI == Q_SWIGLU ? 128 : 256;
  const int NT = p.ncols / OUTN;
  const int64_t total = static_cast<int64_t>(ld_scalar(p.mt_off + p.N)) * NT;
  const int G = gridDim.x;
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
  const int nk = p.K / BKQ;
  const int kb32 = p.K / 32;

  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), (short)0, p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.As), (short)0, p.as_bytes, 0x00020000);

  const int s7 = (lane >> 1) & 7;
  const int khalf = lane >> 5;
  const int frag_lane = (lane & 31) * BKQ;

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

    // ---- A code pieces (RB per wave per slab) and this wave's scale rows.
    // The gathered rows' slots are loaded all at once and without a branch
    // (rows past the tile read its last row's slot, unused), so the loads
    // wait once together instead of one round trip each.
    constexpr bool GATHER = EPI == Q_SWIGLU;
    int src[RB + 1];
#pragma unroll
    for (int i = 0; i <= RB; ++i) {
      const int row = i < RB ? 8 * (RB * wave + i) + (lane >> 3) : 64 * wave + lane;
      const int gm = m0 + min(row, mcount - 1);
      src[i] = GATHER ? p.perm[gm] : gm;
    }
    uint32_t aoff[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int b = RB * wave + i;
      const int row = 8 * b + (lane >> 3);
      const int chunk = (lane & 7) ^ ((4 * b + (lane >> 4)) & 7);
      const int tok = GATHER ? src[i] / p.kdiv : src[i];
      aoff[i] = row < mcount ? static_cast<uint32_t>(tok) * static_cast<uint32_t>(p.K) + chunk * 16
                             : p.a_bytes;
    }
    uint32_t soff;
    {
      const int row = 64 * wave + lane;
      const int tok = GATHER ? src[RB] / p.kdiv : src[RB];
      soff = row < mcount ? static_cast<uint32_t>(tok) * static_cast<uint32_t>(kb32) : p.as_bytes;
    }
    // ---- quantized B: this wave's two column groups of 32
    const int64_t mat = static_cast<int64_t>(p.ncols) * p.K;
    const int gA = EPI == Q_SWIGLU ? n0 / 32 + wave : n0 / 32 + 2 * wave;
    const int gB = EPI == Q_SWIGLU ? gA : gA + 1;
    const uint8_t* Bsrc1 = EPI == Q_SWIGLU ? p.B2 : p.B;
    const uint8_t* b0 = p.B + e * mat + static_cast<int64_t>(gA) * nk * 4096 + lane * 16;
    const uint8_t* b1 = Bsrc1 + e * mat + static_cast<int64_t>(gB) * nk * 4096 + lane * 16;
    // weight scales: one 4-byte-per-lane copy per column group and slab into
    // LDS (lanes 0..31 carry the group's 128 bytes, lanes 32..63 read nothing)
    const int64_t nexp = static_cast<int64_t>(p.N) * mat;  // scales follow all codes
    const uint32_t sbytes = static_cast<uint32_t>(nexp / 32);
    const __amdgpu_buffer_rsrc_t bsr0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + nexp), (short)0, sbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t bsr1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(Bsrc1 + nexp), (short)0, sbytes, 0x00020000);
    const uint32_t ebase = static_cast<uint32_t>(e) * static_cast<uint32_t>(mat / 32);
    const uint32_t bso0 = lane < 32 ? ebase + static_cast<uint32_t>(gA * nk * 128 + 4 * lane)
                                    : sbytes;
    const uint32_t bso1 = lane < 32 ? ebase + static_cast<uint32_t>(gB * nk * 128 + 4 * lane)
                                    : sbytes;

    const int nrb = (mcount + 31) >> 5;
    auto run = [&](auto nrb_c) {
      constexpr int NRB = decltype(nrb_c)::value;
      // weight operands: each byte is used by one expert's tiles only, so
      // the loads carry the non-temporal hint (as in the bf16 kernels)
      auto ldw = [](const uint8_t* q) {
        return __builtin_nontemporal_load(reinterpret_cast<const i32x4_t*>(q));
      };
      i32x8_t bq[NST][2][2];   // B operands in flight: [slot][column group][step]
      auto issue = [&](int kt, int slot) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          lds_void* dst = (lds_void*)(ring + slot * SLOT + (RB * wave + i) * 8 * BKQ);
          lds_dma16(arsrc, dst, aoff[i], kt * BKQ);
        }
        lds_dma4(srsrc, (lds_void*)(ring + slot * SLOT + TM * BKQ + 256 * wave), soff, kt * 4);
        uint8_t* const bsd = ring + slot * SLOT + TM * BKQ + SC_A + 512 * wave;
        lds_dma4(bsr0, (lds_void*)bsd, bso0, kt * 128);
        lds_dma4(bsr1, (lds_void*)(bsd + 256), bso1, kt * 128);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bq[slot][0][st].lo = ldw(b0 + (4 * kt + 2 * st) * 1024);
          bq[slot][0][st].hi = ldw(b0 + (4 * kt + 2 * st + 1) * 1024);
          bq[slot][1][st].lo = ldw(b1 + (4 * kt + 2 * st) * 1024);
          bq[slot][1][st].hi = ldw(b1 + (4 * kt + 2 * st + 1) * 1024);
        }
      };

      f32x16_t acc[NRB][2];
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

      auto compute = [&](int slot) {
        const uint8_t* a_s = ring + slot * SLOT + frag_lane;
        const uint8_t* a_sc = ring + slot * SLOT + TM * BKQ + (lane & 31) * 4 + 2 * khalf;
        const uint8_t* bsl = ring + slot * SLOT + TM * BKQ + SC_A + 512 * wave + 2 * lane;
        const uint32_t sb0 = *reinterpret_cast<const uint16_t*>(bsl);
        const uint32_t sb1 = *reinterpret_cast<const uint16_t*>(bsl + 256);
        // fragment f = s NRB + rb (64-step half s, row block rb): two code
        // reads and one scale read, issued two fragments ahead of the
        // fragment's MFMAs in program order as well as in the groups below
        constexpr int NF = 2 * NRB;
        auto frag = [&](int f, i32x8_t& a, uint32_t& asw) {
          const int s = f / NRB, rb = f % NRB;
          a.lo = *reinterpret_cast<const i32x4_t*>(a_s + rb * 32 * BKQ + (((4 * s + khalf) ^ s7) << 4));
          a.hi = *reinterpret_cast<const i32x4_t*>(a_s + rb * 32 * BKQ + (((4 * s + 2 + khalf) ^ s7) << 4));
          asw = *reinterpret_cast<const uint16_t*>(a_sc + rb * 32 * 4);
        };
        i32x8_t af[3];
        uint32_t aw[3];
#pragma unroll
        for (int f = 0; f < 2 && f < NF; ++f) frag(f, af[f], aw[f]);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + 2 < NF) frag(f + 2, af[(f + 2) % 3], aw[(f + 2) % 3]);
          const int s = f / NRB, rb = f % NRB;
          const uint32_t b0s = s == 0 ? (sb0 & 0xffu) : (sb0 >> 8);
          const uint32_t b1s = s == 0 ? (sb1 & 0xffu) : (sb1 >> 8);
          const uint32_t as = s == 0 ? (aw[f % 3] & 0xffu) : (aw[f % 3] >> 8);
          acc[rb][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[f % 3], bq[slot][0][s], acc[rb][0], 0, 0, 0, static_cast<int>(as), 0,
              static_cast<int>(b0s));
          acc[rb][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af[f % 3], bq[slot][1][s], acc[rb][1], 0, 0, 0, static_cast<int>(as), 0,
              static_cast<int>(b1s));
        }
      };

      // Issue order inside a slab: the slab's loads first (with_loads), then
      // fragment reads (two 16-byte code reads and one scale read per 32
      // rows and MFMA step) one fragment ahead of its two MFMAs.
      constexpr int NFR = 2 * NRB;  // fragments per slab
      auto sched = [&](bool with_loads) {
        if (with_loads) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int g = 0; g < NFR - 1; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      };

      // same slab pipeline as the bf16 kernel: three slabs in flight, the
      // wait before slab kt leaves the loads of the two younger slabs
      // outstanding (V per slab per wave, never interleaved across slabs)
      __builtin_amdgcn_sched_barrier(0);
      issue(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      issue(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(2, 2);
      __builtin_amdgcn_sched_barrier(0);
      int kt = 0;
      for (; kt < nk - 4; kt += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
          __builtin_amdgcn_s_barrier();
          issue(kt + u + 3, (u + 3) & 3);
          compute(u);
          sched(true);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      issue(kt + 3, 3);
      compute(0);
      sched(true);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V));
      __builtin_amdgcn_s_barrier();
      compute(1);
      sched(false);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(V));
      __builtin_amdgcn_s_barrier();
      compute(2);
      sched(false);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_s_barrier();
      compute(3);
      sched(false);
      __builtin_amdgcn_sched_barrier(0);

      // ---- epilogue.  Lane: column lane%32 of its group, rows
      // 32 rb + 8 (v/4) + 4 (lane/32) + v%4.
      __syncthreads();
      const int rbase = 4 * khalf;
      if constexpr (EPI == Q_SWIGLU) {
        // h = silu(gate) * up staged as fp32 rows of 132 (128 columns + 4 of
        // padding against bank conflicts); then one thread per (row, block
        // of 32 columns) takes the block's scale and writes its 32 codes and
        // its scale byte (slab order 0, 2, 1, 3).
        constexpr int HS = 132;
        float* sth = reinterpret_cast<float*>(ring);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
            sth[rl * HS + 32 * wave + (lane & 31)] = silu_f(acc[rb][0][v]) * acc[rb][1][v];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        for (int c = tid; c < mcount * 4; c += NTHR) {
          const int rl = c >> 2, j = c & 3;
          const float* src = sth + rl * HS + 32 * j;
          float v[32];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(src + 4 * i);
            v[4 * i] = w4[0];
            v[4 * i + 1] = w4[1];
            v[4 * i + 2] = w4[2];
            v[4 * i + 3] = w4[3];
          }
          float m = 0.f;
#pragma unroll
          for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
          const int S = mx_scale(m);
          u32x4_t q0, q1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            q0[i] = mx_code(v[4 * i], S) | (mx_code(v[4 * i + 1], S) << 8) |
                    (mx_code(v[4 * i + 2], S) << 16) | (mx_code(v[4 * i + 3], S) << 24);
            q1[i] = mx_code(v[16 + 4 * i], S) | (mx_code(v[16 + 4 * i + 1], S) << 8) |
                    (mx_code(v[16 + 4 * i + 2], S) << 16) | (mx_code(v[16 + 4 * i + 3], S) << 24);
          }
          uint8_t* dq = p.Cq + static_cast<int64_t>(m0 + rl) * p.ncols + n0 + 32 * j;
          *reinterpret_cast<u32x4_t*>(dq) = q0;
          *reinterpret_cast<u32x4_t*>(dq + 16) = q1;
          p.Cs[static_cast<int64_t>(m0 + rl) * (p.ncols / 32) + n0 / 32 + 2 * (j & 1) + (j >> 1)] =
              static_cast<uint8_t>(S);
        }
      } else {
        bf16_t* st = reinterpret_cast<bf16_t*>(ring);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = rbase + 32 * rb + 8 * (v >> 2) + (v & 3);
            st[rl * OUTN + 64 * wave + (lane & 31)] = cvt_bf16(acc[rb][0][v]);
            st[rl * OUTN + 64 * wave + 32 + (lane & 31)] = cvt_bf16(acc[rb][1][v]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        constexpr int RC = OUTN / 8;
#pragma unroll 4
        for (int c = tid; c < mcount * RC; c += NTHR) {
          const int rl = c / RC, cc = (c % RC) * 8;
          *reinterpret_cast<u32x4_t*>(p.Cb + static_cast<int64_t>(m0 + rl) * p.ncols + n0 + cc) =
              *reinterpret_cast<const u32x4_t*>(st + rl * OUTN + cc);
        }
      }
      if (tid == 0) s_claim[0] = next_n;
      __syncthreads();
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

// LDS-only barrier: this wave's LDS accesses are complete, then the
// workgroup meets.  (A workgroup fence would also wait for every vector
// memory access in flight, i.e. drain the slab pipeline.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The FP8 down projection of 256-row tiles (the prefill shape) with no
// bubble between tiles: the next tile's first three slabs are loaded under
// this tile's last three slabs and its epilogue, so the weight stream does
// not stop at tile boundaries.  With reductions of 2048 steps a tile is
// only 16 slabs long, and a pipeline drained and refilled at every tile
// boundary idles the memory path for about a quarter of each tile.
//
// Same operands, fragments and MFMA order as fwdq_kernel<Q_STORE, 256>
// (bit-identical results); what differs:
//  - one code path for every tile: all eight row blocks are multiplied
//    (rows past the tile's end are loaded as zeros), so the registers that
//    carry the next tile's slabs are the same whatever the tile's height;
//  - the next tile is known four slabs before the end (its claim went out
//    during the previous tile's drain) and located then; every per-tile
//    value is a scalar except one lane offset;
//  - weight codes and scales are read through per-tile buffer resources;
//  - the epilogue stages 64 rows at a time in ring slot 3 (slots 0..2 are
//    receiving the next tile), all four quarters whatever the tile's
//    height, so every thread issues 32 row-piece stores per tile, those
//    past the tile's rows dropped by the buffer range check.
//    With that fixed count the first three slabs of a tile wait for
//    "vmcnt <= 62": issued after each of them are two slabs of V loads and
//    the 32 stores, 2V + 32 >= 62 operations, so the bound covers it (the
//    counter has six bits, and at 62 the compiler also sees the slab's
//    weight registers as loaded); from the fourth slab on, "vmcnt <= 2V"
//    as in the steady state.  (Loads return in issue order; stores and atomics in
//    between only make a wait stricter.)  The prologue issues 32 stores
//    that write nothing, so the first tile starts from the same count.
template <bool NT_W>
__global__ __launch_bounds__(NTHR, 1) void downq_kernel(QParams p) {
  constexpr int TM = 256;
  constexpr int RB = TM / 32;                // A copies per wave per slab
  constexpr int SLOT = TM * BKQ + SC_BYTES;  // bytes per ring slot
  constexpr int V = RB + 11;                 // loads per wave per slab
  constexpr int NRB = 8;
  constexpr int OUTN = 256;
  constexpr int QR = 64;                     // rows per staging quarter
  constexpr int RC = OUTN / 8;               // 16-byte pieces per row
  constexpr int NSTORE = (TM / QR) * (QR * RC / NTHR);
  static_assert(QR * OUTN * 2 <= SLOT, "a quarter fits one ring slot");
  static_assert(2 * V + NSTORE >= 62 && 2 * V <= 62, "wait bounds");
  __shared__ __align__(16) uint8_t ring[NST * SLOT + 16];
  int32_t* const s_next = reinterpret_cast<int32_t*>(ring + NST * SLOT);
  bf16_t* const stage = reinterpret_cast<bf16_t*>(ring + 3 * SLOT);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = p.ncols / OUTN;
  const int64_t total = static_cast<int64_t>(ld_scalar(p.mt_off + p.N)) * NT;
  const int G = gridDim.x;
  const int C = G / 8;
  const int nk = p.K / BKQ;
  const int kb32 = p.K / 32;
  const int64_t mat = static_cast<int64_t>(p.ncols) * p.K;
  const int64_t nexp = static_cast<int64_t>(p.N) * mat;  // weight scales follow all codes
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.A), (short)0, p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.As), (short)0, p.as_bytes, 0x00020000);
  const int s7 = (lane >> 1) & 7;
  const int khalf = lane >> 5;
  const int frag_lane = (lane & 31) * BKQ;

  // ---- tile claims (thread 0 only): per-XCD counters, then the other XCDs'
  int cx = blockIdx.x % 8;
  int hops = 0;
  auto resolve = [&](int32_t n) __attribute__((always_inline)) -> int32_t {
    int64_t L = static_cast<int64_t>(n / C) * 8 * C + cx * C + n % C;
    while (L >= total) {
      if (++hops >= 8) return -1;
      cx = (cx + 1) & 7;
      const int32_t m = atomicAdd(p.sched + cx, 1);
      L = static_cast<int64_t>(m / C) * 8 * C + cx * C + m % C;
    }
    return static_cast<int32_t>(L);
  };

  struct Tile {
    int m0, mcount, n0;
    uint32_t abase;                 // byte offset of row m0's codes in A
    uint32_t sa;                    // this lane's activation-scale row (past the end: none)
    __amdgpu_buffer_rsrc_t brsrc;   // codes of this wave's two column groups
    __amdgpu_buffer_rsrc_t bsrsrc;  // and their scales
  };
  // field by field: a whole-struct copy goes through private memory
  auto copy = [](Tile& d, const Tile& t) __attribute__((always_inline)) {
    d.m0 = t.m0;
    d.mcount = t.mcount;
    d.n0 = t.n0;
    d.abase = t.abase;
    d.sa = t.sa;
    d.brsrc = t.brsrc;
    d.bsrsrc = t.bsrsrc;
  };
  auto locate = [&](int32_t L, Tile& t) __attribute__((always_inline)) {
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
    // the expert's 32-row blocks spread evenly over its row tiles
    const int seg0 = ld_scalar(p.offsets + e), seg1 = ld_scalar(p.offsets + e + 1);
    const int nbe = (seg1 - seg0 + 31) >> 5;
    const int blo = nbe * mt / mte, bhi = nbe * (mt + 1) / mte;
    t.m0 = seg0 + 32 * blo;
    t.mcount = min(seg0 + 32 * bhi, seg1) - t.m0;
    t.n0 = nt * OUTN;
    t.abase = static_cast<uint32_t>(t.m0) * static_cast<uint32_t>(p.K);
    const int row = 64 * wave + lane;
    t.sa = row < t.mcount ? static_cast<uint32_t>(t.m0 + row) * static_cast<uint32_t>(kb32)
                          : p.as_bytes;
    const int g = t.n0 / 32 + 2 * wave;  // the first of the wave's two column groups
    t.brsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + e * mat + static_cast<int64_t>(g) * nk * 4096), (short)0,
        static_cast<uint32_t>(nk) * 8192u, 0x00020000);
    t.bsrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + nexp + e * (mat / 32) + static_cast<int64_t>(g) * nk * 128),
        (short)0, static_cast<uint32_t>(nk) * 256u, 0x00020000);
  };

  // A copy i of wave w: rows 8 b + lane/8 (b = 8 w + i), 16 bytes at chunk
  // (lane%8) ^ ((4 b + lane/16) % 8), which depends on i only through i % 2
  const int lrow = lane >> 3;
  uint32_t achunk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    achunk[j] = static_cast<uint32_t>(lrow) * static_cast<uint32_t>(p.K) +
                static_cast<uint32_t>(((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) * 16);
  const uint32_t blane0 = lane * 16;
  const uint32_t blane1 = static_cast<uint32_t>(nk) * 4096u + lane * 16;
  // weight scales: lanes 0..31 carry a group's 128 bytes of a slab, lanes
  // 32..63 point past the resource (no data)
  const uint32_t bsl0 = lane < 32 ? 4u * lane : static_cast<uint32_t>(nk) * 256u;
  const uint32_t bsl1 = lane < 32 ? static_cast<uint32_t>(nk) * 128u + 4u * lane
                                  : static_cast<uint32_t>(nk) * 256u;
  auto ldw = [](__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) __attribute__((always_inline)) {
    return __builtin_bit_cast(i32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT_W ? 2 : 0));
  };

  i32x8_t bq[NST][2][2];  // B operands in flight: [slot][column group][step]
  // LDS destinations of a slab's copies: one scalar base per slab, made
  // opaque so that the compiler does not keep every (slot, copy) address of
  // the loop in a scalar register of its own
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  auto issue = [&](const Tile& t, int kt, int slot) __attribute__((always_inline)) {
    lds_u8* base = (lds_u8*)(ring + slot * SLOT);
    asm volatile("" : "+s"(base));
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int b = RB * wave + i;
      const uint32_t off = lrow < t.mcount - 8 * b
                               ? t.abase + static_cast<uint32_t>(8 * b) * static_cast<uint32_t>(p.K) + achunk[i & 1]
                               : p.a_bytes;
      lds_dma16(arsrc, (lds_void*)(base + b * 8 * BKQ), off, kt * BKQ);
    }
    lds_dma4(srsrc, (lds_void*)(base + TM * BKQ + 256 * wave), t.sa, kt * 4);
    lds_u8* const bsd = base + TM * BKQ + SC_A + 512 * wave;
    lds_dma4(t.bsrsrc, (lds_void*)bsd, bsl0, kt * 128);
    lds_dma4(t.bsrsrc, (lds_void*)(bsd + 256), bsl1, kt * 128);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bq[slot][0][st].lo = ldw(t.brsrc, blane0, (4 * kt + 2 * st) * 1024);
      bq[slot][0][st].hi = ldw(t.brsrc, blane0, (4 * kt + 2 * st + 1) * 1024);
      bq[slot][1][st].lo = ldw(t.brsrc, blane1, (4 * kt + 2 * st) * 1024);
      bq[slot][1][st].hi = ldw(t.brsrc, blane1, (4 * kt + 2 * st + 1) * 1024);
    }
  };

  f32x16_t acc[NRB][2];
  auto compute = [&](int slot) __attribute__((always_inline)) {
    const uint8_t* a_s = ring + slot * SLOT + frag_lane;
    const uint8_t* a_sc = ring + slot * SLOT + TM * BKQ + (lane & 31) * 4 + 2 * khalf;
    const uint8_t* bsl = ring + slot * SLOT + TM * BKQ + SC_A + 512 * wave + 2 * lane;
    const uint32_t sb0 = *reinterpret_cast<const uint16_t*>(bsl);
    const uint32_t sb1 = *reinterpret_cast<const uint16_t*>(bsl + 256);
    constexpr int NF = 2 * NRB;
    auto frag = [&](int f, i32x8_t& a, uint32_t& asw) __attribute__((always_inline)) {
      const int s = f / NRB, rb = f % NRB;
      a.lo = *reinterpret_cast<const i32x4_t*>(a_s + rb * 32 * BKQ + (((4 * s + khalf) ^ s7) << 4));
      a.hi = *reinterpret_cast<const i32x4_t*>(a_s + rb * 32 * BKQ + (((4 * s + 2 + khalf) ^ s7) << 4));
      asw = *reinterpret_cast<const uint16_t*>(a_sc + rb * 32 * 4);
    };
    i32x8_t af[3];
    uint32_t aw[3];
#pragma unroll
    for (int f = 0; f < 2; ++f) frag(f, af[f], aw[f]);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + 2 < NF) frag(f + 2, af[(f + 2) % 3], aw[(f + 2) % 3]);
      const int s = f / NRB, rb = f % NRB;
      const uint32_t b0s = s == 0 ? (sb0 & 0xffu) : (sb0 >> 8);
      const uint32_t b1s = s == 0 ? (sb1 & 0xffu) : (sb1 >> 8);
      const uint32_t as = s == 0 ? (aw[f % 3] & 0xffu) : (aw[f % 3] >> 8);
      acc[rb][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          af[f % 3], bq[slot][0][s], acc[rb][0], 0, 0, 0, static_cast<int>(as), 0,
          static_cast<int>(b0s));
      acc[rb][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          af[f % 3], bq[slot][1][s], acc[rb][1], 0, 0, 0, static_cast<int>(as), 0,
          static_cast<int>(b1s));
    }
  };
  constexpr int NFR = 2 * NRB;
  auto sched = [&](bool with_loads) __attribute__((always_inline)) {
    if (with_loads) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int g = 0; g < NFR - 1; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };
  // one slab: wait for it, meet, issue a younger slab's loads, multiply
  auto slab = [&](auto wait_c, const Tile& t_issue, int kt_issue, int slot_issue, int slot) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(decltype(wait_c)::value);
    __builtin_amdgcn_s_barrier();
    issue(t_issue, kt_issue, slot_issue);
    compute(slot);
    sched(true);
    __builtin_amdgcn_sched_barrier(0);
  };
  using W62 = std::integral_constant<int, vmcnt_imm(62)>;
  using W2V = std::integral_constant<int, vmcnt_imm(2 * V)>;

  // Later claims are one buffer atomic issued by every thread, only thread
  // 0's inside the counters' range: the result register is written on
  // every path, so nothing waits for it before it is used a tile later.
  // (Claimed under "if (tid == 0)", the result joins the other threads'
  // value after the branch, and every wave waits there for all of its
  // loads in flight.)
  const __amdgpu_buffer_rsrc_t schedr =
      __builtin_amdgcn_make_buffer_rsrc(p.sched, (short)0, 32u, 0x00020000);
  // ---- first tile, and the claim of the second (thread 0: pend, pend_ok)
  int32_t pend = 0;
  bool pend_ok = false;
  if (tid == 0) {
    const int32_t L0 = resolve(atomicAdd(p.sched + cx, 1));
    if (L0 >= 0) {
      pend = atomicAdd(p.sched + cx, 1);
      pend_ok = true;
    }
    s_next[0] = L0;
  }
  __syncthreads();
  int32_t Lc = __builtin_amdgcn_readfirstlane(s_next[0]);
  if (Lc < 0) return;
  Tile tc;
  locate(Lc, tc);
  __builtin_amdgcn_sched_barrier(0);
  issue(tc, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue(tc, 1, 1);
  __builtin_amdgcn_sched_barrier(0);
  issue(tc, 2, 2);
  __builtin_amdgcn_sched_barrier(0);
  {
    // the stores an epilogue would have issued, into an empty resource (at
    // distinct offsets, so that none of them is merged away)
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc(p.Cb, (short)0, 0u, 0x00020000);
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NSTORE; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(z, none, 16 * tid + 4096 * i, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  const int rbase = 4 * khalf;
  const int srow = tid / RC, scol = (tid % RC) * 8;
  for (;;) {
#pragma unroll
    for (int i = 0; i < NRB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // slabs 0..3: the first three behind the previous epilogue's stores
    slab(W62{}, tc, 3, 3, 0);
    slab(W62{}, tc, 4, 0, 1);
    slab(W62{}, tc, 5, 1, 2);
    slab(W2V{}, tc, 6, 2, 3);
    int kt = 4;
    for (; kt < nk - 4; kt += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) slab(W2V{}, tc, kt + u + 3, (u + 3) & 3, u);
    }
    // slab nk-4: the next tile is named (its claim was issued a whole tile
    // ago) and located, and the tile after it claimed; thread 0's note is
    // complete before the barrier.  (The drain below has no branch: the
    // compiler would sink the MFMAs of the slab before it past it.)
    int32_t Ln0 = -1;
    if (tid == 0) {
      Ln0 = pend_ok ? resolve(pend) : -1;
      s_next[0] = Ln0;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * V) & ~0x0F00);
    __builtin_amdgcn_s_barrier();
    pend_ok = Ln0 >= 0;
    pend = __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
        1, schedr, tid == 0 && pend_ok ? 4 * cx : 32, 0, 0);
    issue(tc, kt + 3, 3);
    __builtin_amdgcn_sched_barrier(0);
    const int32_t Ln = __builtin_amdgcn_readfirstlane(s_next[0]);
    // no next tile: the drain re-reads this tile's first slabs, unused (no
    // branch here: the compiler would hoist the next slab's fragment reads
    // above it and keep them in scratch across it)
    Tile tn;
    locate(Ln >= 0 ? Ln : Lc, tn);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    sched(false);
    __builtin_amdgcn_sched_barrier(0);
    // slabs nk-3 .. nk-1, each with one of the next tile's first three slabs
    // in flight
    slab(W2V{}, tn, 0, 0, 1);
    slab(W2V{}, tn, 1, 1, 2);
    slab(W2V{}, tn, 2, 2, 3);

    // ---- epilogue: lane holds column lane%32 of its group and rows
    // 32 rb + 8 (v/4) + 4 (lane/32) + v%4; quarters of 64 rows staged in
    // slot 3 (bf16) and written as 16-byte row pieces through a resource
    // that ends at the tile's last row
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.Cb + static_cast<int64_t>(tc.m0) * p.ncols, (short)0,
        static_cast<uint32_t>(tc.mcount) * static_cast<uint32_t>(p.ncols) * 2u, 0x00020000);
    const uint32_t ostep = static_cast<uint32_t>(NTHR / RC) * static_cast<uint32_t>(p.ncols) * 2u;
#pragma unroll
    for (int qq = 0; qq < TM / QR; ++qq) {
      // every quarter, also those past the tile's rows (their stores fall
      // outside the resource): results used under a branch would let the
      // compiler sink the last slab's MFMAs into it, past the barriers
      lds_barrier();  // slot 3 read by every wave / the last quarter stored
#pragma unroll
      for (int rb = 2 * qq; rb < 2 * qq + 2; ++rb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = rbase + 32 * (rb - 2 * qq) + 8 * (v >> 2) + (v & 3);
          stage[rl * OUTN + 64 * wave + (lane & 31)] =
              __builtin_bit_cast(bf16_t, static_cast<__bf16>(acc[rb][0][v]));
          stage[rl * OUTN + 64 * wave + 32 + (lane & 31)] =
              __builtin_bit_cast(bf16_t, static_cast<__bf16>(acc[rb][1][v]));
        }
      }
      lds_barrier();
      const uint32_t obase =
          (static_cast<uint32_t>(qq * QR + srow) * static_cast<uint32_t>(p.ncols) +
           static_cast<uint32_t>(tc.n0 + scol)) * 2u;
#pragma unroll
      for (int i = 0; i < QR * RC / NTHR; ++i) {
        const u32x4_t vv =
            *reinterpret_cast<const u32x4_t*>(stage + (srow + i * (NTHR / RC)) * OUTN + scol);
        __builtin_amdgcn_raw_buffer_store_b128(vv, crsrc, obase + i * ostep, 0, 0);
      }
    }
    if (Ln < 0) break;
    copy(tc, tn);
    Lc = Ln;
  }
  // the unused slabs of the drain land in LDS before the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Activation quantizer: rows x K bf16 (row-major, rows gathered by nothing)
// -> codes [rows][K] and scales [rows][K/32] in slab order (0, 2, 1, 3).
// Four lanes per block, eight values per lane.
__global__ __launch_bounds__(256) void mxq_rows_kernel(const bf16_t* __restrict__ src,
                                                       int64_t nblocks, int K,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int kb = K / 32;
  for (int64_t g = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
       g < nblocks * 4; g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t blk = g >> 2;           // block index = row * kb + j
    const int part = static_cast<int>(g & 3);
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + blk * 32 + part * 8);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int S = mx_scale(m);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= mx_code(v[i], S) << (8 * i);
      hi |= mx_code(v[4 + i], S) << (8 * i);
    }
    *reinterpret_cast<uint2*>(codes + blk * 32 + part * 8) = make_uint2(lo, hi);
    if (part == 0) {
      const int64_t row = blk / kb;
      const int j = static_cast<int>(blk - row * kb);
      const int pos = (j & ~3) + 2 * (j & 1) + ((j >> 1) & 1);
      scales[row * kb + pos] = static_cast<uint8_t>(S);
    }
  }
}

// Weight quantizer + packer: nmat matrices [R][C] bf16 -> codes in the
// packed layout, then scales (see the header comment).
__global__ __launch_bounds__(256) void mxq_weights_kernel(const bf16_t* __restrict__ src,
                                                          int64_t nblocks, int R, int C,
                                                          uint8_t* __restrict__ dst,
                                                          int64_t nmat) {
  const int kb = C / 32;
  const int nk = C / 128;
  const int64_t per_mat = static_cast<int64_t>(R) * C;
  uint16_t* const sdst = reinterpret_cast<uint16_t*>(dst + nmat * per_mat);
  for (int64_t g = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
       g < nblocks * 4; g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t blk = g >> 2;
    const int part = static_cast<int>(g & 3);
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + blk * 32 + part * 8);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int S = mx_scale(m);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= mx_code(v[i], S) << (8 * i);
      hi |= mx_code(v[4 + i], S) << (8 * i);
    }
    const int64_t mi = blk / (static_cast<int64_t>(R) * kb);
    const int64_t rem = blk - mi * R * kb;
    const int r = static_cast<int>(rem / kb);
    const int jb = static_cast<int>(rem - static_cast<int64_t>(r) * kb);  // block along C
    const int t = jb >> 2;               // slab
    const int step = (jb >> 1) & 1;      // MFMA step in the slab
    const int half = jb & 1;             // operand half (bytes 16 half ..)
    const int h = part >> 1;             // lane half: values 16h .. 16h+15 of the block
    const int lanei = (r & 31) + 32 * h;
    const int64_t piece = ((static_cast<int64_t>(r >> 5) * nk + t) * 2 + step) * 2 + half;
    uint8_t* o = dst + mi * per_mat + piece * 1024 + lanei * 16 + (part & 1) * 8;
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    if (part == 0) {
      // 16-bit word (block 4t + hh, block 4t + 2 + hh) of lane (r%32) + 32 hh
      const int j = jb & 3;
      const int hh = j & 1, byte = j >> 1;
      const int64_t wi = (static_cast<int64_t>(r >> 5) * nk + t) * 64 + (r & 31) + 32 * hh;
      reinterpret_cast<uint8_t*>(sdst + mi * (per_mat / 64))[wi * 2 + byte] =
          static_cast<uint8_t>(S);
    }
  }
}

typedef void (*fwdq_fn)(QParams);
// Tile heights 32 .. 256.  The 256-row down projection runs downq_kernel
// when the reduction has at least eight slabs (launch_q); below that the
// four-wave kernel's 256-row variant, which spills a few registers in its
// tile setup and epilogue, none inside the k loop.
fwdq_fn pick_q(int epi, int tm, int* per_cu) {
  *per_cu = tm <= 64 ? 2 : 1;
  if (epi == Q_SWIGLU) {
    switch (tm) {
      case 32: return fwdq_kernel<Q_SWIGLU, 32>;
      case 64: return fwdq_kernel<Q_SWIGLU, 64>;
      case 128: return fwdq_kernel<Q_SWIGLU, 128>;
      case 256: return fwdq_kernel<Q_SWIGLU, 256>;
    }
  } else {
    switch (tm) {
      case 32: return fwdq_kernel<Q_STORE, 32>;
      case 64: return fwdq_kernel<Q_STORE, 64>;
      case 128: return fwdq_kernel<Q_STORE, 128>;
      case 256: return fwdq_kernel<Q_STORE, 256>;
    }
  }
  return nullptr;
}

hipError_t launch_q(int epi, int tm, const QParams& p, int cu, hipStream_t s) {
  if (epi == Q_STORE && tm == 256 && p.K >= 8 * BKQ) {
    hipLaunchKernelGGL(downq_kernel<true>, dim3(cu), dim3(NTHR), 0, s, p);
    return hipGetLastError();
  }
  int per_cu = 1;
  fwdq_fn k = pick_q(epi, tm, &per_cu);
  if (!k) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, dim3(per_cu * cu), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

int grid_for(int64_t threads) {
  const int64_t want = (threads + 255) / 256;
  return static_cast<int>(want < 16384 ? want : 16384);
}

}  // namespace

hipError_t launch_mxq_rows(const bf16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                           hipStream_t s) {
  const int64_t nblocks = rows * (K / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxq_rows_kernel, dim3(grid_for(nblocks * 4)), dim3(256), 0, s, src, nblocks,
                     K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mxq_weights(const bf16_t* src, uint8_t* dst, int64_t nmat, int R, int C,
                              hipStream_t s) {
  const int64_t nblocks = nmat * R * static_cast<int64_t>(C / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxq_weights_kernel, dim3(grid_for(nblocks * 4)), dim3(256), 0, s, src,
                     nblocks, R, C, dst, nmat);
  return hipGetLastError();
}

hipError_t launch_fwdq_gateup(const uint8_t* xq, const uint8_t* xs, int64_t T, const uint8_t* wg_q,
                              const uint8_t* wu_q, const int32_t* offsets, const int32_t* perm,
                              const int32_t* mt_off, const int32_t* tile_exp, int32_t* sched,
                              int tm, int N, int I, int d, int K, uint8_t* hq, uint8_t* hs, int cu,
                              hipStream_t s) {
  QParams p{};
  p.N = N; p.ncols = I; p.K = d;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = xq; p.a_bytes = static_cast<uint32_t>(T * d);
  p.As = xs; p.as_bytes = static_cast<uint32_t>(T * (d / 32));
  p.perm = perm; p.kdiv = K;
  p.B = wg_q; p.B2 = wu_q; p.Cq = hq; p.Cs = hs;
  return launch_q(Q_SWIGLU, tm, p, cu, s);
}

hipError_t launch_fwdq_down(const uint8_t* hq, const uint8_t* hs, int64_t rows,
                            const uint8_t* wd_q, const int32_t* offsets, const int32_t* mt_off,
                            const int32_t* tile_exp, int32_t* sched, int tm, int N, int I, int d,
                            bf16_t* y, int cu, hipStream_t s) {
  QParams p{};
  p.N = N; p.ncols = d; p.K = I;
  p.offsets = offsets; p.mt_off = mt_off; p.tile_exp = tile_exp; p.sched = sched;
  p.A = hq; p.a_bytes = static_cast<uint32_t>(rows * I);
  p.As = hs; p.as_bytes = static_cast<uint32_t>(rows * (I / 32));
  p.B = wd_q; p.Cb = y;
  return launch_q(Q_STORE, tm, p, cu, s);
}

}  // namespace zc

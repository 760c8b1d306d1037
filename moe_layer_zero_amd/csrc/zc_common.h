// Internal declarations shared by the HIP translation units of libzcmoe.
// Device helpers (bf16 <-> fp32, MFMA operand types) and the host-side
// launcher interfaces that api.hip sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zc {

// ---------------------------------------------------------------- types
typedef uint16_t bf16_t;  // storage of a bfloat16 (upper half of an fp32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<bf16_t>((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// A wave-uniform read of a table that no kernel writes while the reading one
// runs (tile and segment prefixes), as a scalar load: scalar loads are counted
// apart from the vector memory operations, so the reader does not wait on
// loads, stores or atomics it has in flight.
template <typename T>
__device__ __forceinline__ T ld_scalar(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)ptr;
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static constexpr int kVec = 4;  // elements per 16-byte chunk
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
  static constexpr int kVec = 8;
};

// Row-tile height of the grouped GEMMs; the dispatch step publishes the
// per-expert prefix of ceil(rows / kGemmBM) tiles for them.
constexpr int kGemmBM = 128;
// Most experts a layer may have (E = N + Z <= 1024, checked by the host API).
constexpr int kMaxExperts = 1024;
// Row-tile height of the bf16 forward expert GEMMs (gemm_fwd.hip).
constexpr int kFwdBM = 256;

// ---------------------------------------------------------------- launchers
// Every launcher queues work on `s` and returns the hipError_t of the launch.

// Router scores: logits[T][E] = x[T][d] * wr[E][d]^T (fp32 out).  With
// router_gemm_splits(T, E, d) > 1 the hidden dimension is cut into that many
// chunks whose fp32 partials (part: splits * T * E floats) are added in
// chunk order.
int router_gemm_splits(int64_t Tn, int64_t E, int64_t d);
template <typename T>
hipError_t launch_router_gemm(const T* x, const T* wr, float* logits, int Tn, int E, int d,
                              float* part, int cu_count, hipStream_t s);

// Routing keys, biased top-K, gates (one wavefront per token).
hipError_t launch_topk(const float* logits, const float* bias, int Tn, int E, int K,
                       int gate_norm, int32_t* topk_idx, float* topk_gate, hipStream_t s);

// Device-level load-balance loss of section 2.1.2 (Eq.(4)-(5)) from the
// scores and the per-expert pick counts: out = [L, f_1..f_{D+1},
// P_1..P_{D+1}] (binary64).  Scratch: lb_scratch_bytes(T, E).
size_t lb_scratch_bytes(int64_t Tn, int64_t E);
hipError_t launch_lb_loss(const float* logits, const int32_t* counts, int Tn, int N, int E, int K,
                          int D, double K_e, double alpha, double* out, void* scratch,
                          hipStream_t s);
// coef[j] = alpha * f_{g(j)} / T (fp32, [E]): the loss's score gradient is
// R_j (coef_j - sum_k R_k coef_k) for each token.
hipError_t launch_lb_coef(const int32_t* counts, int Tn, int N, int E, int K, int D, double K_e,
                          double alpha, float* coef, hipStream_t s);

// Dispatch: per-expert counts, offsets, canonical permutation and its inverse.
// Scratch: dispatch_scratch_bytes(T, E, N).  Also writes the per-expert
// row-tile prefixes tile_off[N+1] and tile_off2[N+1] for the grouped GEMMs
// (tile heights bm and bm2), if tile_exp / tile_exp1 are not NULL the
// expert of each of the tile_off2[N] bm2-row / tile_off[N] bm-row tiles,
// and if sched is not NULL zeroes its kSchedInts tile counters (for the
// packed-weight GEMMs of the same call).
size_t dispatch_scratch_bytes(int64_t Tn, int64_t E, int64_t N);
hipError_t launch_dispatch(const int32_t* topk_idx, int Tn, int E, int N, int K, int bm, int bm2,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                           int32_t* tile_off, int32_t* tile_off2, int32_t* tile_exp,
                           int32_t* tile_exp1, int32_t* sched, void* scratch, hipStream_t s);
constexpr int kSchedInts = 16;  // 8 XCD counters for gate/up, 8 for down

// FFN picks per token (budget-control telemetry): hist[K+1] and moments
// [mean, population std], from topk_idx.  Scratch: stats_scratch_bytes(T, K).
size_t stats_scratch_bytes(int64_t Tn, int64_t K);
hipError_t launch_route_stats(const int32_t* topk_idx, int Tn, int N, int K, int32_t* hist,
                              double* moments, void* scratch, hipStream_t s);
// acc[i] += counts[i] for i < E (int32).
hipError_t launch_accumulate_counts(const int32_t* counts, int E, int32_t* acc, hipStream_t s);

// tile_off[N+1] from offsets[N+1] (for a backward call that only has the
// routing of its forward call).
hipError_t launch_tile_offsets(const int32_t* offsets, int N, int bm, int32_t* tile_off,
                               hipStream_t s);
// ... and also the bm2-row prefix with the expert of each of its tiles, and
// zeroed tile counters (for the packed-weight backward GEMMs).
hipError_t launch_tile_offsets2(const int32_t* offsets, int N, int bm, int32_t* tile_off, int bm2,
                                int32_t* tile_off2, int32_t* tile_exp2, int32_t* sched, int nsched,
                                hipStream_t s);

// Grouped / dense GEMMs (gemm.hip); the backward's fp32 intermediates enter
// bf16 GEMMs as exact hi+lo bf16 pairs.
template <typename T>
hipError_t launch_ffn_gateup(const T* x, const T* wg, const T* wu, const int32_t* offsets,
                             const int32_t* perm, const int32_t* tile_off, int N, int I, int d,
                             int K, int64_t max_rows, T* h, float* save_a, float* save_u,
                             float* save_h, int cu_count, hipStream_t s);
template <typename T>
hipError_t launch_ffn_down(const T* h, const T* wd, const int32_t* offsets,
                           const int32_t* tile_off, int N, int I, int d, int64_t max_rows, T* y,
                           int cu_count, hipStream_t s);
template <typename T>
hipError_t launch_bwd_down_dh(const T* dout, const int32_t* perm, int K, const float* gs,
                              const T* wd, const float* sa, const float* su,
                              const int32_t* offsets, const int32_t* tile_off, int N, int I,
                              int d, int64_t max_rows, float* dadu, int cu_count, hipStream_t s);
template <typename T>
hipError_t launch_bwd_down_dw(const T* dout, const int32_t* perm, int K, const float* hsave,
                              const float* gs, const int32_t* offsets, int N, int I, int d,
                              T* dwd, int cu_count, hipStream_t s);
template <typename T>
hipError_t launch_bwd_gateup_dx(const float* dadu, const T* wg, const T* wu,
                                const int32_t* offsets, const int32_t* tile_off, int N, int I,
                                int d, int64_t max_rows, float* dxp, int cu_count, hipStream_t s);
template <typename T>
hipError_t launch_bwd_gateup_dw(const float* dadu, const T* x, const int32_t* offsets,
                                const int32_t* perm, int N, int I, int d, int K, T* dwg, T* dwu,
                                int cu_count, hipStream_t s);
template <typename T>
hipError_t launch_router_dw(const float* dl, int ldl, const T* x, int Tn, int E, int d, T* dwr,
                            float* part, int cu_count, hipStream_t s);
// Token chunks of the router weight gradient (1: no split); part of
// launch_router_dw needs splits * E * d floats when splits > 1.
int router_dw_splits(int64_t Tn, int64_t E, int64_t d);
template <typename T>
hipError_t launch_router_dx(const float* dl, int ldl, const T* wr, int Tn, int E, int d,
                            float* dxr, int cu_count, hipStream_t s);

// bf16 forward expert GEMMs with 256 x 256 tiles (gemm_fwd.hip); mt_off is
// the kFwdBM row-tile prefix from the dispatch step.
hipError_t launch_fwd_gateup(const bf16_t* x, const bf16_t* wg, const bf16_t* wu,
                             const int32_t* offsets, const int32_t* perm, const int32_t* mt_off,
                             int N, int I, int d, int K, bf16_t* h, float* save_a, float* save_u,
                             float* save_h, int cu, hipStream_t s);
hipError_t launch_fwd_down(const bf16_t* h, const bf16_t* wd, const int32_t* offsets,
                           const int32_t* mt_off, int N, int I, int d, bf16_t* y, int cu,
                           hipStream_t s);

// bf16 forward expert GEMMs on packed weights (gemm_fwdp.hip): x_elems /
// h_elems bound the activation buffer (loads past it read nothing); tm is
// the row-tile height, fwdp_rows_per_tile(T*K/N), mt_off the prefix of
// ceil(rows / tm) and tile_exp the expert of each tile from the dispatch
// step; sched: 8 tile counters, zero at launch (the dispatch zeroes them).
int fwdp_rows_per_tile(int64_t avg_rows);
hipError_t launch_fwdp_gateup(const bf16_t* x, int64_t x_elems, const bf16_t* wg_p,
                              const bf16_t* wu_p, const int32_t* offsets, const int32_t* perm,
                              const int32_t* mt_off, const int32_t* tile_exp, int32_t* sched,
                              int tm, int N, int I, int d, int K, bf16_t* h, int cu,
                              hipStream_t s);
hipError_t launch_fwdp_down(const bf16_t* h, int64_t h_elems, const bf16_t* wd_p,
                            const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                            int32_t* sched, int tm, int N, int I, int d, bf16_t* y, int cu,
                            hipStream_t s);
// nmat row-major [R][C] bf16 matrices -> packed layout (R % 32 == 0, C % 16 == 0).
hipError_t launch_pack_weights(const bf16_t* src, bf16_t* dst, int64_t nmat, int R, int C,
                               hipStream_t s);
// SwiGLU backward from dh and the saved a, u, h ([P][I] fp32 each): hilo
// [P][4I] = exact bf16 hi/lo pairs of da and du, ghlo [P][2I] = those of
// gs * h; I a multiple of 8.
hipError_t launch_swiglu_bwd(const float* dh, const float* gs, const float* sa, const float* su,
                             const float* sh, const int32_t* offsets, int N, int I,
                             int64_t max_rows, bf16_t* hilo, bf16_t* ghlo, hipStream_t s);
// Expert weight gradients (gemm_dw.hip): per expert e, the [M][Ncol]
// product sum over its rows p of X[p]^T Y[p], X given as an exact bf16
// hi/lo pair (X, XL: columns 0..M of rows of pitch ldx), Y exact bf16;
// stored [M][Ncol] bf16 per expert, or [Ncol][M] when transposed; sched: 8
// counters, zero at launch.
hipError_t launch_dw(bool transposed, int N, int M, int Ncol, const int32_t* offsets,
                     int32_t* sched, const bf16_t* X, const bf16_t* XL, int64_t ldx, const bf16_t* Y,
                     int64_t ldy, int64_t rows, bf16_t* C, int cu, hipStream_t s);
// dst[p] = src[perm[p] / K] (rows of width w) for the FFN picks in dispatch order.
hipError_t launch_gather_rows(const bf16_t* src, const int32_t* perm, const int32_t* offsets,
                              int N, int K, int w, int64_t max_rows, bf16_t* dst, hipStream_t s);

// Grouped GEMMs on row-major weights (gemm_rmw.hip): the forward (with
// sa, su, sh given it also keeps a, u, h in fp32; all three null: h only),
// and the backward's dh = gs * (dout
// W_d) and expert dx = [da_hi | da_lo | du_hi | du_lo] [W_g; W_g; W_u; W_u]
// (fp32, [P][I] and [P][d]) reading the row-major weights directly.  Tile
// tables as for the packed-weight kernels: the tm-row prefix mt_off, the
// expert of each tile, 8 per-XCD counters zeroed before the launch (tm = 64,
// 128 or 256; dh and dx take 64 or 128).  rmw_fwd_supported (forward) and
// rmw_supported (forward and backward): d and I multiples of 256 and every
// byte offset the kernels take within 31 bits.
bool rmw_fwd_supported(int64_t rows, int64_t Tn, int64_t d, int64_t I);
bool rmw_supported(int64_t rows, int64_t Tn, int64_t d, int64_t I);
hipError_t launch_rmw_gateup(const bf16_t* x, int64_t Tn, const bf16_t* wg, const bf16_t* wu,
                             const int32_t* offsets, const int32_t* perm, const int32_t* mt_off,
                             const int32_t* tile_exp, int32_t* sched, int tm, int N, int I, int d,
                             int K, bf16_t* h, float* sa, float* su, float* sh, int cu,
                             hipStream_t s);
hipError_t launch_rmw_down(const bf16_t* h, int64_t rows, const bf16_t* wd,
                           const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                           int32_t* sched, int tm, int N, int I, int d, bf16_t* y, int cu,
                           hipStream_t s);
hipError_t launch_rmw_dh(const bf16_t* doutd, int64_t rows, const bf16_t* wd,
                         const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                         int32_t* sched, int tm, int N, int I, int d, const float* gs, float* dh,
                         int cu, hipStream_t s);
// Dense c[M][n] = a[M][K] b[n][K]^T in fp32 on the same kernel (the router
// scores of large batches): n a multiple of 256, K of 32, byte offsets
// within 31 bits (rmw_dense_supported).
bool rmw_dense_supported(int64_t M, int64_t n, int64_t K);
hipError_t launch_rmw_dense(const bf16_t* a, int64_t M, const bf16_t* b, int n, int K, float* c,
                            int cu, hipStream_t s);
hipError_t launch_rmw_dx(const bf16_t* hilo, int64_t rows, const bf16_t* wg, const bf16_t* wu,
                         const int32_t* offsets, const int32_t* mt_off, const int32_t* tile_exp,
                         int32_t* sched, int tm, int N, int I, int d, float* dxp, int cu,
                         hipStream_t s);

// MXFP8 expert GEMMs (gemm_fwdq.hip): E4M3 codes with one E8M0 scale per
// 32 reduction steps.  Activation quantizer (rows x K bf16 -> codes and
// slab-ordered scales), weight quantizer + packer (nmat [R][C] matrices ->
// packed codes followed by packed scales), and the two grouped GEMMs (tile
// bookkeeping as for the packed bf16 GEMMs).
hipError_t launch_mxq_rows(const bf16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                           hipStream_t s);
hipError_t launch_mxq_weights(const bf16_t* src, uint8_t* dst, int64_t nmat, int R, int C,
                              hipStream_t s);
hipError_t launch_fwdq_gateup(const uint8_t* xq, const uint8_t* xs, int64_t T, const uint8_t* wg_q,
                              const uint8_t* wu_q, const int32_t* offsets, const int32_t* perm,
                              const int32_t* mt_off, const int32_t* tile_exp, int32_t* sched,
                              int tm, int N, int I, int d, int K, uint8_t* hq, uint8_t* hs, int cu,
                              hipStream_t s);
hipError_t launch_fwdq_down(const uint8_t* hq, const uint8_t* hs, int64_t rows,
                            const uint8_t* wd_q, const int32_t* offsets, const int32_t* mt_off,
                            const int32_t* tile_exp, int32_t* sched, int tm, int N, int I, int d,
                            bf16_t* y, int cu, hipStream_t s);

// Combine: out = out_scale * (c_t x_t + sum_r g_r y[inv]).
template <typename T>
hipError_t launch_combine(const T* x, const T* y, const int32_t* topk_idx, const float* gate,
                          const int32_t* inv, int Tn, int d, int N, int K, float out_scale,
                          T* out, hipStream_t s);

// Combine backward: dg per slot, out_scale * gate of every FFN pick in
// dispatch order (gs), and the router-score gradient dl [T][ldl] (fp32);
// with lb_coef (from launch_lb_coef, else NULL) dl also takes the
// load-balance loss's score gradient.
template <typename T>
hipError_t launch_combine_bwd(const T* x, const T* y, const T* dout, const float* logits,
                              const int32_t* topk_idx, const float* gate, const int32_t* inv,
                              int Tn, int d, int N, int E, int K, int gate_norm, float out_scale,
                              const float* lb_coef, float* gs, float* dg, float* dl, int ldl,
                              hipStream_t s);

// dx gather: dx = out_scale * c_t * dout_t + sum_r dxp[inv] + dxr_t.
template <typename T>
hipError_t launch_dx_gather(const T* dout, const float* dxp, const float* dxr, const int32_t* topk_idx,
                            const float* gate, const int32_t* inv, int Tn, int d, int N, int K,
                            float out_scale, T* dx, hipStream_t s);

// Bias update, Eq.(2) of section 2.1.1.
hipError_t launch_pid(int N, int K, const int32_t* counts, int64_t T_all, double mu, double K_e,
                      float* bias, hipStream_t s);

}  // namespace zc

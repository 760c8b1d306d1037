/*
 * zc_moe.h -- C ABI of the MI355X (gfx950) MoE layer with zero-computation
 * experts.
 *
 * The layer is the one of "LongCat-Flash Technical Report", section 2.1
 * ("Zero-computation experts"), Eq.(1): a softmax router over N FFN experts
 * plus Z zero-computation experts, a per-expert bias b_i that only shifts
 * which K experts are picked, gates taken from the unbiased softmax, FFN
 * experts evaluated on the tokens routed to them, and zero-computation
 * experts returning their input x_t.  The bias follows Eq.(2) of section
 * 2.1.1 ("Computation budget control").  The device-level load-balance
 * loss is the one of section 2.1.2 ("Load balance control").
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *    owns every buffer; the library never allocates or frees device memory
 *    and never synchronises with the host.  Scratch memory comes in through
 *    (ws, ws_bytes); its required size is zc_moe_workspace_size().
 *  - All work is queued on `stream` (a hipStream_t, passed as void*; NULL is
 *    the default stream).  Outputs are valid once the stream has reached
 *    that point; they are undefined after an error status.
 *  - Arguments are checked on the host before anything is queued.  A bad
 *    argument returns ZC_ERR_INVALID / ZC_ERR_UNSUPPORTED / ZC_ERR_WORKSPACE
 *    and writes nothing.  A failed launch returns ZC_ERR_HIP.  The detail of
 *    the last non-OK status of the calling thread is in zc_last_error().
 *  - Every reduction has a fixed order: for fixed inputs and shapes, results
 *    are bitwise reproducible from run to run.
 *  - Row-major layouts, "out x in" for weights (like a linear layer's
 *    weight), so every GEMM reads its reduction dimension contiguously:
 *      x, out, dout, dx      [T][d]
 *      w_router, dw_router   [E][d]          E = N + Z
 *      w_gate, w_up (+ grads)[N][I][d]
 *      w_down, dw_down       [N][d][I]
 *    Expert indices 0..N-1 are FFN experts, N..E-1 zero-computation experts.
 *  - Data pointers must be 16-byte aligned.  bf16 layers need d and I to be
 *    multiples of 64, fp32 layers multiples of 32 (else ZC_ERR_UNSUPPORTED).
 *  - Non-finite inputs: a NaN or infinite router score makes every routing
 *    key of its token NaN (through the softmax), and NaN keys rank below
 *    every number, so the selection stays total: such a token picks experts
 *    0..K-1 (valid indices) and NaN flows on through its gates or its x
 *    row; no index leaves its range.  T*K < 2^31 is required (checked).
 */
#ifndef ZC_MOE_H
#define ZC_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZC_OK = 0,
  ZC_ERR_INVALID = 1,     /* null pointer, bad size, bad enum value      */
  ZC_ERR_UNSUPPORTED = 2, /* valid layer outside the supported shapes    */
  ZC_ERR_WORKSPACE = 3,   /* ws too small (or NULL with ws_bytes needed) */
  ZC_ERR_HIP = 4          /* a HIP launch or runtime call failed         */
} zc_status;

typedef enum { ZC_F32 = 0, ZC_BF16 = 1 } zc_dtype;

/* Layer description (host struct, passed by pointer). */
typedef struct {
  int64_t T;         /* tokens in the batch (0 allowed: nothing is done)      */
  int64_t d;         /* hidden size                                           */
  int64_t N;         /* FFN experts (>= 0)                                    */
  int64_t Z;         /* zero-computation experts (>= 0), E = N + Z in 1..1024 */
  int64_t I;         /* FFN inner size                                        */
  int64_t K;         /* experts per token, 1 <= K <= min(E, 32)               */
  int32_t dtype;     /* zc_dtype of x, weights, out, dx and weight gradients; */
                     /* logits, gates and bias are always fp32; bf16 math     */
                     /* accumulates in fp32                                   */
  int32_t gate_norm; /* 1: gates renormalised over the K picks (softmax of    */
                     /*    the picked scores; the picked R_i rescaled to sum  */
                     /*    to 1);  0: gate = R_i exactly as Eq.(1) prints it  */
  float out_scale;   /* scalar on the layer output (1.0 = none)               */
  int32_t weight_layout; /* zc_weight_layout of w_gate, w_up and w_down       */
  int32_t cu_limit;  /* 0: the GEMMs' persistent grids fill every compute    */
                     /* unit; n > 0, a multiple of 8 (the grids deal tiles to */
                     /* the 8 XCDs): they are sized as for min(n, CUs) units. */
                     /* Results do not depend on it (every sum has a fixed    */
                     /* order, whichever workgroup computes it); it leaves    */
                     /* compute units to concurrent work and lets a test      */
                     /* check that claim.  Other values: ZC_ERR_INVALID.      */
} zc_moe_desc;

/* Layouts of the FFN expert weights.
 *  ZC_WEIGHTS_ROWMAJOR: the row-major layouts listed above.
 *  ZC_WEIGHTS_PACKED:   the output of zc_moe_pack_weights.  Accepted by
 *      zc_moe_forward for bf16 layers with d and I multiples of 256, when no
 *      activations are saved (saved == NULL): the inference forward.  The
 *      backward and the saving forward need row-major weights.
 *  ZC_WEIGHTS_MXFP8:    the output of zc_moe_quantize_weights: FP8
 *      blockwise-quantized expert weights (see there).  Accepted by
 *      zc_moe_forward for bf16 layers with d and I multiples of 512 and no
 *      saved buffer: the FP8 inference forward. */
typedef enum {
  ZC_WEIGHTS_ROWMAJOR = 0, ZC_WEIGHTS_PACKED = 1, ZC_WEIGHTS_MXFP8 = 2
} zc_weight_layout;

/* Routing state: written by zc_moe_route / zc_moe_forward, read by
 * zc_moe_backward.  All device buffers owned by the caller. */
typedef struct {
  float* logits;     /* [T][E] router scores x W_r^T (fp32)                   */
  int32_t* topk_idx; /* [T][K] picked expert per slot; slot 0 = largest key   */
  float* topk_gate;  /* [T][K] gate per slot                                  */
  int32_t* counts;   /* [E]    tokens per expert (the T_i of Eq.(2))          */
  int32_t* offsets;  /* [N+1]  exclusive prefix sum of counts[0..N)           */
  int32_t* perm;     /* [T*K]  first offsets[N] entries: the flat slots t*K+r */
                     /*        of FFN picks sorted by (expert, token)         */
  int32_t* inv;      /* [T*K]  position of slot t*K+r in perm, -1 for a       */
                     /*        zero-computation pick                          */
} zc_route_buf;

enum {
  ZC_OP_ROUTE = 0, ZC_OP_FORWARD = 1, ZC_OP_BACKWARD = 2, ZC_OP_LB_LOSS = 3,
  ZC_OP_ROUTE_STATS = 4
};

/* Device-level load-balance loss settings ("LongCat-Flash Technical
 * Report", section 2.1.2; host struct, passed by pointer).  The N FFN
 * experts form D groups of G = N/D consecutive indices (group j holds
 * experts (j-1)G .. jG-1: the experts one device holds under expert
 * parallelism); every zero-computation expert is in the extra group D+1. */
typedef struct {
  int64_t D;    /* groups, 1 <= D <= N, N % D == 0                          */
  double K_e;   /* expected FFN experts per token: 0 < K_e <= K, and        */
                /* K_e < K when Z > 0                                       */
  double alpha; /* balance factor (finite)                                  */
} zc_lb_cfg;

/* Bytes of scratch memory `op` needs for this layer (0 for an invalid
 * description).  The bound depends only on the description, never on the
 * routing, so it can be sized before the first call. */
size_t zc_moe_workspace_size(const zc_moe_desc* desc, int op);

/* Bytes of the activation buffer `saved` that zc_moe_forward fills for
 * zc_moe_backward (pre-activations, hidden and expert outputs of every FFN
 * pick, sized for the worst case T*K picks).  Layout, each piece starting
 * at a multiple of 256 bytes: a = x W_g^T, u = x W_u^T and h = silu(a) * u
 * in fp32, [T*K][I] each, row p = the p-th FFN pick in dispatch order (the
 * route's perm; rows from offsets[N] on are unused), then the expert
 * outputs y, [T*K][d] in the layer dtype. */
size_t zc_moe_saved_size(const zc_moe_desc* desc);

/* Router and dispatch: Eq.(1)'s scores, biased top-K and gates, then the
 * per-expert token counts and the (expert, token) dispatch order.
 *   logits = x W_r^T (fp32 accumulation);
 *   key_j  = p_j + b_j with p the softmax of the token's logits, computed in
 *            binary64 (max subtraction, Cody-Waite + degree-13 Taylor
 *            exponential, 64 partial sums combined pairwise at xor distance
 *            32..1, one division per key);
 *   picks  = the K largest keys, ties to the lower expert index (a NaN
 *            key ranks below every number);
 *   gates  = e_j / (sum of the picked e) (gate_norm 1) or p_j (gate_norm 0),
 *            with e_j the exponentials above, rounded to fp32.
 * If x and w_router are both NULL the scores already in r->logits are used
 * as given (routing of scores computed elsewhere).  bias: [E] fp32. */
zc_status zc_moe_route(const zc_moe_desc* desc, const void* x,
                       const void* w_router, const float* bias,
                       zc_route_buf* r, void* ws, size_t ws_bytes,
                       void* stream);

/* Full layer forward: route as above, then for every FFN pick
 * h = silu(x W_g^T) * (x W_u^T) and y = h W_d^T on the tokens routed to that
 * expert (grouped bf16 MFMA GEMMs, fp32 accumulation, h and y stored in the
 * layer dtype), then
 *   out_t = out_scale * ( (sum of gates on zero-computation picks) * x_t
 *                         + sum over FFN picks r ascending of g_r * y_r ),
 * accumulated in fp32.  Zero-computation experts cost one scalar per token.
 * saved (nullable, zc_moe_saved_size bytes) receives what zc_moe_backward
 * needs.  w_gate/w_up/w_down may be NULL only when N == 0. */
zc_status zc_moe_forward(const zc_moe_desc* desc, const void* x,
                         const void* w_router, const float* bias,
                         const void* w_gate, const void* w_up,
                         const void* w_down, void* out, zc_route_buf* r,
                         void* saved, void* ws, size_t ws_bytes, void* stream);

/* The inference forward of zc_moe_forward (saved = NULL) without a
 * workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It allocates nothing: its scratch is a device array inside
 * the library, ZC_NOALLOC_SCRATCH_BYTES per GPU, held by every GPU the
 * library runs on until the process ends (looked up once per device, on
 * the first call with that device current).  Layers whose
 * zc_moe_workspace_size(desc, ZC_OP_FORWARD) exceeds it are rejected with
 * ZC_ERR_WORKSPACE before anything is queued; the LongCat-Flash layer at a
 * 256-token decode batch (57 MB) fits.  The caller still owns x, the
 * weights, out and r, with the same contract as zc_moe_forward.  Every call
 * on a GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, other threads) race and give undefined results; calls queued on
 * one stream are ordered and safe.  Each call rewrites what it reads of the
 * scratch before reading it.  Kernel timing events are not recorded. */
#define ZC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
zc_status zc_moe_forward_noalloc(const zc_moe_desc* desc, const void* x,
                                 const void* w_router, const float* bias,
                                 const void* w_gate, const void* w_up,
                                 const void* w_down, void* out, zc_route_buf* r,
                                 void* stream);

/* Backward of zc_moe_forward with the routing held fixed (the picked set is
 * piecewise constant in the inputs; the bias gets no gradient, it is
 * decoupled from the training objective).  Given dout [T][d]:
 *   dg_r  = <out_scale*dout_t, y_r> (FFN pick) or <out_scale*dout_t, x_t>;
 *   expert gradients through y = W_d(silu(W_g x) * W_u x);
 *   router: dl_j = g_j (dg_j - sum_picks g dg) on the picks (gate_norm 1),
 *           dl_j = p_j (dg_j [pick] - sum_picks p dg) (gate_norm 0);
 *   dx = out_scale*(identity gates)*dout + expert dx + dl W_r.
 * With lb (host, nullable) the objective also holds the device-level
 * load-balance loss of zc_moe_lb_loss on the same routing, and dl above
 * takes its score gradient (f held fixed, it counts discrete picks):
 *   dl_j += p_j (c_j - sum_k p_k c_k),  c_j = alpha f_{g(j)} / T,
 * with p the fp32 softmax of the token's scores and g(j) the group of j.
 * Every gradient buffer is overwritten (not accumulated): with T == 0 the
 * weight gradients are zeros, and x, saved, dout and dx may be NULL.  r and
 * saved must come from the zc_moe_forward call being differentiated. */
zc_status zc_moe_backward(const zc_moe_desc* desc, const void* x,
                          const void* w_router, const void* w_gate,
                          const void* w_up, const void* w_down,
                          const zc_route_buf* r, const void* saved,
                          const void* dout, void* dx, void* dw_router,
                          void* dw_gate, void* dw_up, void* dw_down,
                          const zc_lb_cfg* lb, void* ws, size_t ws_bytes,
                          void* stream);

/* Device-level load-balance loss, section 2.1.2 of the report:
 *   L = alpha * sum_{j=1}^{D+1} f_j P_j,
 *   P_j = (1/T) sum over i in group j and all tokens t of R_{t,i}  (Eq.(4)),
 *   f_j = D/(K_e T) * (picks of all tokens in group j),  j <= D    (Eq.(5)),
 *   f_{D+1} = 1/((K-K_e) T) * (zero-computation picks)             (Eq.(5)),
 * a pick counting once for each expert of the group it lands on, so every
 * f_j is 1 when the FFN picks spread evenly and K_e FFN experts are picked
 * per token on average; with Z = 0 the extra group's term is left out.
 * R is the unbiased softmax of r->logits, computed in binary64 exactly as
 * for the routing keys (see zc_moe_route); the picks come from r->counts.
 * r is the route buffer of the zc_moe_route / zc_moe_forward call of this
 * micro-batch (only logits and counts are read).  out (device, 1 + 2(D+1)
 * doubles): L, then f_1..f_{D+1}, then P_1..P_{D+1} (the extra group's
 * slots 0 when Z = 0); all zero when T = 0.  Sums run in a fixed order.
 * Scratch: zc_moe_workspace_size(desc, ZC_OP_LB_LOSS) bytes. */
zc_status zc_moe_lb_loss(const zc_moe_desc* desc, const zc_lb_cfg* lb,
                         const zc_route_buf* r, double* out, void* ws,
                         size_t ws_bytes, void* stream);

/* Eq.(2) bias update, in place on bias [N+Z] (fp32), for FFN experts i < N:
 *   b_i += mu * ( K_e/(K*N) - T_i/(K*T_all) ),  T_i = counts[i],
 * in binary64 with exactly the operations
 *   tgt = K_e/((double)K*N); obs = (double)T_i/((double)K*T_all);
 *   b_i = (float)((double)b_i + mu*(tgt - obs));
 * zero-computation experts keep their bias.  counts [N+Z] int32 (device).
 * Needs T_all >= 1, K >= 1, N >= 0. */
zc_status zc_moe_pid_update(int64_t N, int64_t Z, int64_t K,
                            const int32_t* counts, int64_t T_all, double mu,
                            double K_e, float* bias, void* stream);

/* Budget-control telemetry ("LongCat-Flash Technical Report", section
 * 2.1.1, which tracks the mean and the spread of the FFN experts each token
 * activates, Fig.3b/3c).  From r->topk_idx of a routed batch:
 *   n_t      = number of token t's K picks that are FFN experts (< N);
 *   hist[k]  = tokens with n_t = k, k = 0..K   (device, K+1 int32);
 *   moments  = [mean of n_t, population standard deviation of n_t]
 *              (device, 2 doubles; mean from the exact integer sum; both 0
 *              when T = 0).
 * Scratch: zc_moe_workspace_size(desc, ZC_OP_ROUTE_STATS) bytes. */
zc_status zc_moe_route_stats(const zc_moe_desc* desc, const zc_route_buf* r,
                             int32_t* hist, double* moments, void* ws,
                             size_t ws_bytes, void* stream);

/* acc[i] += counts[i] for i < E (device int32 arrays, distinct): sums the
 * per-expert counts T_i of several micro-batches (or steps), so that one
 * zc_moe_pid_update over acc with T_all = their total tokens applies
 * Eq.(2) over a global batch, or at a lower update frequency, as section
 * 2.1.1 advises for small batches.  The caller zeroes acc before the first
 * micro-batch and keeps the total below 2^31 picks per expert. */
zc_status zc_moe_accumulate_counts(int64_t E, const int32_t* counts,
                                   int32_t* acc, void* stream);

/* Rearranges one set of FFN expert weights (bf16) from the row-major layout
 * into ZC_WEIGHTS_PACKED, for the bf16 inference forward, which then streams
 * every weight panel from HBM in whole 1 KB pieces straight into the matrix
 * cores' operand registers ("LongCat-Flash Technical Report", section 2.1:
 * the FFN experts' weights are the bulk of the layer's memory traffic).
 *   which = ZC_PACK_GATE_UP: src is w_gate or w_up, [N][I][d];
 *   which = ZC_PACK_DOWN:    src is w_down, [N][d][I].
 * Each expert's [R][C] matrix (R output columns, C reduction length) is
 * stored as consecutive 1 KB blocks, block (r/32, c/16) at index
 * (r/32)*(C/16) + c/16, and inside a block element (r, c) at
 * (r%32 + 32*((c/8)%2))*8 + c%8: the B operand of one 32x32x16 MFMA step for
 * 32 output columns, lane by lane.  dst has src's size and must not overlap
 * it.  Needs dtype bf16 and d, I multiples of 256 (the desc's weight_layout
 * is ignored).  Queued on `stream` like every call. */
enum { ZC_PACK_GATE_UP = 0, ZC_PACK_DOWN = 1 };
zc_status zc_moe_pack_weights(const zc_moe_desc* desc, int which, const void* src, void* dst,
                              void* stream);

/* FP8 blockwise quantization of one set of FFN expert weights (bf16) for
 * the FP8 inference forward (the LongCat deployment runs its expert GEMMs
 * blockwise in FP8, keeping sensitive parts in higher precision).  Format:
 * OCP Microscaling MXFP8 -- each run of 32 consecutive values along a
 * weight row's reduction dimension shares one power-of-two scale
 * 2^(S-127), S an 8-bit exponent (E8M0), and each value is stored as an
 * FP8 E4M3 code of value / 2^(S-127):
 *   S = floor(log2 max|v|) - 8 + 127 (at least 0; 0 for an all-zero run);
 *   code = nearest E4M3 value, ties to even, magnitudes above 448 clamped.
 * A forward with desc->weight_layout = ZC_WEIGHTS_MXFP8 quantizes x the
 * same way per token (runs of 32 along d) and h per pick (runs of 32 along
 * I, from h rounded to fp32), multiplies on the scaled FP8 matrix cores with
 * fp32 accumulation, and keeps the router, gates, combine and the
 * zero-computation experts (which return the unquantized x) in bf16/fp32.
 *   which = ZC_PACK_GATE_UP: src is w_gate or w_up, [N][I][d];
 *   which = ZC_PACK_DOWN:    src is w_down, [N][d][I].
 * dst (zc_moe_quantized_weight_bytes(desc) bytes, not overlapping src)
 * receives the codes of all N experts in the matrix cores' operand order,
 * then their scales; its layout is private to this library.  Needs dtype
 * bf16 and d, I multiples of 512 (desc->weight_layout is ignored). */
size_t zc_moe_quantized_weight_bytes(const zc_moe_desc* desc);
zc_status zc_moe_quantize_weights(const zc_moe_desc* desc, int which,
                                  const void* src, void* dst, void* stream);

/* Kernel timing for benchmarks.  While profiling is on, every entry point
 * brackets each of its kernel launches with a pair of HIP events recorded on
 * the call's own stream, tagged with one of the phases below.  The events
 * are host-side objects created by the library; no device memory is
 * allocated.  zc_moe_profile_read waits for every recorded event, adds each
 * duration (ms) to total_ms[phase] and one to count[phase] (both host
 * arrays of ZC_NUM_PHASES entries, zeroed first), then forgets the events.
 * Turning profiling off discards events not read yet. */
enum {
  ZC_PH_ROUTER_GEMM = 0, ZC_PH_TOPK, ZC_PH_DISPATCH, ZC_PH_GATE_UP, ZC_PH_DOWN, ZC_PH_COMBINE,
  ZC_PH_BWD_COMBINE, ZC_PH_BWD_DOWN_DH, ZC_PH_BWD_DOWN_DW, ZC_PH_BWD_GATE_UP_DX,
  ZC_PH_BWD_GATE_UP_DW, ZC_PH_BWD_ROUTER_DW, ZC_PH_BWD_ROUTER_DX, ZC_PH_BWD_DX_GATHER,
  ZC_PH_BIAS_UPDATE, ZC_PH_TILE_OFFSETS, ZC_PH_LB_LOSS, ZC_PH_LB_COEF, ZC_PH_ROUTE_STATS,
  ZC_PH_ACCUMULATE, ZC_PH_QUANTIZE, ZC_PH_BWD_GATHER, ZC_NUM_PHASES
};
zc_status zc_moe_profile(int on);
zc_status zc_moe_profile_read(double* total_ms, int32_t* count);
const char* zc_moe_phase_name(int phase); /* static text, "" if out of range */

/* Static text for a status code (never NULL). */
const char* zc_status_string(zc_status s);

/* Detail of the calling thread's last non-OK status ("" if none). */
const char* zc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZC_MOE_H */

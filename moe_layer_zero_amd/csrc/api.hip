// C ABI of libzcmoe: argument checks, workspace carving and the launch
// sequence of each entry point.  See include/zc_moe.h for the contract.
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/zc_moe.h"
#include "zc_common.h"

using zc::bf16_t;

namespace {

thread_local std::string g_last_error;

zc_status fail(zc_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
zc_status fail(zc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

zc_status hip_fail(hipError_t e, const char* what) {
  return fail(ZC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define ZC_HIP(call, what)                           \
  do {                                               \
    hipError_t e_ = (call);                          \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// ---- optional per-phase kernel timing (zc_moe_profile)
struct PhaseRec {
  int phase;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<PhaseRec> g_prof_recs;

// Set while the calling thread runs the allocation-free forward: its
// launches record no timing events (creating an event may allocate).
thread_local bool t_no_events = false;

// Records a start event on construction and an end event in done(), on the
// stream of the launch, when profiling is on.
class PhaseScope {
 public:
  PhaseScope(int phase, hipStream_t s) : phase_(phase), s_(s) {
    if (!t_no_events && g_prof_on.load(std::memory_order_relaxed) &&
        hipEventCreate(&a_) == hipSuccess)
      (void)hipEventRecord(a_, s_);
    else
      a_ = nullptr;
  }
  void done() {
    if (!a_) return;
    hipEvent_t b = nullptr;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a_);
      return;
    }
    (void)hipEventRecord(b, s_);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_recs.push_back(PhaseRec{phase_, a_, b});
  }

 private:
  int phase_;
  hipStream_t s_;
  hipEvent_t a_;
};

#define ZC_LAUNCH(phase, call, what)                 \
  do {                                               \
    PhaseScope ps_((phase), s);                      \
    hipError_t e_ = (call);                          \
    ps_.done();                                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

void drop_records() {
  for (auto& r : g_prof_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof_recs.clear();
}

// Compute-unit count of the current device, cached per device.
std::atomic<int> g_cu[64];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    int v = g_cu[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  // the persistent grids deal their tiles to the 8 XCDs in equal shares
  n = n < 8 ? 8 : n / 8 * 8;
  if (dev < 64) g_cu[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Compute units the persistent grids of a call are sized for.
int cus(const zc_moe_desc* d) {
  const int n = cu_count();
  return d->cu_limit > 0 && d->cu_limit < n ? d->cu_limit : n;
}

int64_t a256(int64_t b) { return (b + 255) & ~int64_t(255); }
int64_t esize(const zc_moe_desc* d) { return d->dtype == ZC_F32 ? 4 : 2; }
int64_t ldl_of(int64_t E) { return (E + 7) / 8 * 8; }

#define ZC_CHECK(x)                   \
  do {                                \
    zc_status s_ = (x);               \
    if (s_ != ZC_OK) return s_;       \
  } while (0)

// Shapes the packed layout and its forward kernels handle: bf16, d and I
// multiples of 256, activation buffers (x [T][d], h [T*K][I]) addressable
// with 32-bit byte offsets.
zc_status check_packable(const zc_moe_desc* d) {
  if (d->dtype != ZC_BF16) return fail(ZC_ERR_UNSUPPORTED, "packed weights need a bf16 layer");
  if (d->d % 256 || d->I % 256)
    return fail(ZC_ERR_UNSUPPORTED, "packed weights need d and I multiples of 256 (d=%lld I=%lld)",
                (long long)d->d, (long long)d->I);
  if (d->T * d->d * 2 >= (int64_t(1) << 31) || d->T * d->K * d->I * 2 >= (int64_t(1) << 31))
    return fail(ZC_ERR_UNSUPPORTED, "packed-weight forward needs T*d and T*K*I below 2^30");
  return ZC_OK;
}

// Shapes the MXFP8 forward handles: bf16 layer, d and I multiples of 512
// (whole groups of four 128-step slabs), 32-bit byte offsets into x' and h'.
zc_status check_mxfp8(const zc_moe_desc* d) {
  if (d->dtype != ZC_BF16) return fail(ZC_ERR_UNSUPPORTED, "MXFP8 weights need a bf16 layer");
  if (d->d % 512 || d->I % 512)
    return fail(ZC_ERR_UNSUPPORTED, "MXFP8 weights need d and I multiples of 512 (d=%lld I=%lld)",
                (long long)d->d, (long long)d->I);
  if (d->T * d->d >= (int64_t(1) << 31) || d->T * d->K * d->I >= (int64_t(1) << 31))
    return fail(ZC_ERR_UNSUPPORTED, "MXFP8 forward needs T*d and T*K*I below 2^31");
  return ZC_OK;
}

zc_status check_desc(const zc_moe_desc* d) {
  if (!d) return fail(ZC_ERR_INVALID, "desc is NULL");
  const int64_t E = d->N + d->Z;
  if (d->T < 0 || d->d < 1 || d->N < 0 || d->Z < 0 || d->I < 1)
    return fail(ZC_ERR_INVALID, "bad sizes T=%lld d=%lld N=%lld Z=%lld I=%lld", (long long)d->T,
                (long long)d->d, (long long)d->N, (long long)d->Z, (long long)d->I);
  if (E < 1 || E > 1024) return fail(ZC_ERR_INVALID, "N+Z=%lld outside 1..1024", (long long)E);
  if (d->K < 1 || d->K > E || d->K > 32)
    return fail(ZC_ERR_INVALID, "K=%lld outside 1..min(N+Z, 32)", (long long)d->K);
  if (d->dtype != ZC_F32 && d->dtype != ZC_BF16)
    return fail(ZC_ERR_INVALID, "dtype %d is neither ZC_F32 nor ZC_BF16", d->dtype);
  if (d->gate_norm != 0 && d->gate_norm != 1)
    return fail(ZC_ERR_INVALID, "gate_norm %d is neither 0 nor 1", d->gate_norm);
  if (!std::isfinite(d->out_scale)) return fail(ZC_ERR_INVALID, "out_scale is not finite");
  if (d->weight_layout != ZC_WEIGHTS_ROWMAJOR && d->weight_layout != ZC_WEIGHTS_PACKED &&
      d->weight_layout != ZC_WEIGHTS_MXFP8)
    return fail(ZC_ERR_INVALID, "weight_layout %d is not ROWMAJOR, PACKED or MXFP8",
                d->weight_layout);
  if (d->cu_limit < 0 || d->cu_limit % 8)
    return fail(ZC_ERR_INVALID, "cu_limit %d is neither 0 nor a positive multiple of 8",
                d->cu_limit);
  if (d->T * d->K >= (int64_t(1) << 31) || d->d >= (int64_t(1) << 24) || d->I >= (int64_t(1) << 24))
    return fail(ZC_ERR_UNSUPPORTED, "T*K, d or I too large for 32-bit indexing");
  const int64_t mult = d->dtype == ZC_BF16 ? 64 : 32;
  if (d->d % mult || d->I % mult)
    return fail(ZC_ERR_UNSUPPORTED, "%s layers need d and I multiples of %lld (d=%lld I=%lld)",
                d->dtype == ZC_BF16 ? "bf16" : "fp32", (long long)mult, (long long)d->d,
                (long long)d->I);
  if (d->weight_layout == ZC_WEIGHTS_PACKED) ZC_CHECK(check_packable(d));
  if (d->weight_layout == ZC_WEIGHTS_MXFP8) ZC_CHECK(check_mxfp8(d));
  return ZC_OK;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

zc_status check_ptr(const void* p, const char* name, bool nullable = false) {
  if (!p) return nullable ? ZC_OK : fail(ZC_ERR_INVALID, "%s is NULL", name);
  if (!aligned(p)) return fail(ZC_ERR_INVALID, "%s is not 16-byte aligned", name);
  return ZC_OK;
}

// Per-token buffers may be NULL when there are no tokens (T == 0).
zc_status check_route(const zc_route_buf* r, bool no_tokens) {
  if (!r) return fail(ZC_ERR_INVALID, "route buffer is NULL");
  ZC_CHECK(check_ptr(r->logits, "r->logits", no_tokens));
  ZC_CHECK(check_ptr(r->topk_idx, "r->topk_idx", no_tokens));
  ZC_CHECK(check_ptr(r->topk_gate, "r->topk_gate", no_tokens));
  ZC_CHECK(check_ptr(r->counts, "r->counts"));
  ZC_CHECK(check_ptr(r->offsets, "r->offsets"));
  ZC_CHECK(check_ptr(r->perm, "r->perm", no_tokens));
  ZC_CHECK(check_ptr(r->inv, "r->inv", no_tokens));
  return ZC_OK;
}

// ---- workspace layouts (all pieces 256-byte aligned)
struct RouteWs {
  int32_t* tile_off;   // row-tile prefix for the generic grouped GEMM
  int32_t* tile_off2;  // row-tile prefix for the bf16 forward expert GEMMs
  int32_t* tile_exp;   // expert of each of those row tiles
  int32_t* tile_exp1;  // expert of each row tile of the first prefix
  int32_t* sched;      // tile counters of the packed-weight GEMMs
  float* rpart;        // fp32 partials of a split router GEMM (nullptr: unsplit)
  void* dispatch;
};
// Row tiles of the second prefix, at most: every FFN pick in a tile of its
// own expert, tiles at least 32 rows high.
int64_t max_tiles2(const zc_moe_desc* d) { return d->T * d->K / 32 + d->N + 1; }
int64_t rpart_bytes(const zc_moe_desc* d) {
  const int64_t E = d->N + d->Z;
  const int s = zc::router_gemm_splits(d->T, E, d->d);
  return s > 1 ? 4 * s * d->T * E : 0;
}
int64_t route_ws_bytes(const zc_moe_desc* d) {
  return 2 * a256(4 * (d->N + 1)) + 2 * a256(4 * max_tiles2(d)) + a256(4 * zc::kSchedInts) +
         a256(rpart_bytes(d)) + a256(zc::dispatch_scratch_bytes(d->T, d->N + d->Z, d->N));
}
RouteWs carve_route(char* p, const zc_moe_desc* d) {
  RouteWs w;
  w.tile_off = reinterpret_cast<int32_t*>(p);
  w.tile_off2 = reinterpret_cast<int32_t*>(p + a256(4 * (d->N + 1)));
  char* q = p + 2 * a256(4 * (d->N + 1));
  w.tile_exp = reinterpret_cast<int32_t*>(q);
  q += a256(4 * max_tiles2(d));
  w.tile_exp1 = reinterpret_cast<int32_t*>(q);
  q += a256(4 * max_tiles2(d));
  w.sched = reinterpret_cast<int32_t*>(q);
  q += a256(4 * zc::kSchedInts);
  w.rpart = rpart_bytes(d) > 0 ? reinterpret_cast<float*>(q) : nullptr;
  q += a256(rpart_bytes(d));
  w.dispatch = q;
  return w;
}

// Saved activations: a, u, h of every FFN pick in fp32 (what the backward
// differentiates through, unrounded) and the expert outputs y in the layer
// dtype (what the combine used).
struct Saved {
  float *a, *u, *h;
  void* y;
};
int64_t saved_bytes(const zc_moe_desc* d) {
  const int64_t rows = d->T * d->K, es = esize(d);
  return 3 * a256(rows * d->I * 4) + a256(rows * d->d * es);
}
Saved carve_saved(char* p, const zc_moe_desc* d) {
  const int64_t rows = d->T * d->K;
  const int64_t hi = a256(rows * d->I * 4);
  return Saved{reinterpret_cast<float*>(p), reinterpret_cast<float*>(p + hi),
               reinterpret_cast<float*>(p + 2 * hi), p + 3 * hi};
}

// Forward scratch: routing scratch, h in the layer dtype (operand of the
// down GEMM) and y when no saved buffer takes it.
// MXFP8 layers add x' (codes T*d, scales T*d/32); h' (codes and scales)
// fits in the h piece.
int64_t fwd_ws_bytes(const zc_moe_desc* d) {
  const int64_t rows = d->T * d->K, es = esize(d);
  int64_t b = route_ws_bytes(d) + a256(rows * d->I * es) + a256(rows * d->d * es);
  if (d->weight_layout == ZC_WEIGHTS_MXFP8) b += a256(d->T * d->d) + a256(d->T * d->d / 32);
  return b;
}

struct BwdWs {
  int32_t* tile_off;
  // dadu: da, du [P][2I] on the generic path; dh [P][I] on the packed-weight
  // path (its SwiGLU backward then writes the hi/lo pairs below)
  float *gs, *dg, *dl, *dadu, *dxp, *dxr, *rdw, *lbc;
  // matrix-core backward (use_bwdp): tile prefix and experts, counters,
  // exact bf16 hi/lo pairs of da, du and g h, and x and dout rows in
  // dispatch order
  int32_t *mt2, *texp2, *sched;
  bf16_t *hilo, *ghlo, *xd, *doutd;
};
constexpr int kBwdSched = 48;  // dh, dx, dW_d, dW_g, dW_u: 8 counters each
// The backward's dh and expert-dx GEMMs read the row-major weights directly
// (gemm_rmw.hip), and its expert weight gradients run on operands gathered
// into dispatch order, for bf16 layers with d and I multiples of 256 whose
// byte offsets into dout, x, the hi/lo pairs and the weights fit 31 bits
// (the weight-gradient loads run up to 64 rows past an expert's).
bool use_bwdp(const zc_moe_desc* d) {
  if (d->dtype != ZC_BF16 || d->N == 0 || d->d % 256 || d->I % 256) return false;
  return zc::rmw_supported(d->T * d->K, d->T, d->d, d->I);
}
// Row-tile height of the dh and dx GEMMs: the average rows per FFN expert
// rounded up to 64 or 128.
int bwdp_rows_per_tile(const zc_moe_desc* d) {
  return d->T * d->K / d->N <= 64 ? 64 : zc::kGemmBM;
}
int64_t bwdp_bytes(const zc_moe_desc* d) {
  if (!use_bwdp(d)) return 0;
  const int64_t rows = d->T * d->K;
  return a256(4 * (d->N + 1)) + a256(4 * max_tiles2(d)) + a256(4 * kBwdSched) +
         a256(rows * 4 * d->I * 2) + a256(rows * 2 * d->I * 2) + 2 * a256(rows * d->d * 2);
}
// fp32 partials of the router weight gradient (token chunks), 0 when unsplit
int64_t rdw_bytes(const zc_moe_desc* d) {
  const int64_t E = d->N + d->Z;
  const int s = zc::router_dw_splits(d->T, E, d->d);
  return s > 1 ? 4 * s * E * d->d : 0;
}
int64_t bwd_ws_bytes(const zc_moe_desc* d) {
  const int64_t rows = d->T * d->K, E = d->N + d->Z;
  return a256(4 * (d->N + 1)) + a256(4 * rows) + a256(4 * d->T * d->K) +
         a256(4 * d->T * ldl_of(E)) + a256(4 * rows * 2 * d->I) + a256(4 * rows * d->d) +
         a256(4 * d->T * d->d) + a256(rdw_bytes(d)) + a256(4 * E) + bwdp_bytes(d);
}
BwdWs carve_bwd(char* p, const zc_moe_desc* d) {
  const int64_t rows = d->T * d->K, E = d->N + d->Z;
  BwdWs w;
  w.tile_off = reinterpret_cast<int32_t*>(p);
  p += a256(4 * (d->N + 1));
  auto take = [&p](int64_t bytes) {
    float* q = reinterpret_cast<float*>(p);
    p += a256(bytes);
    return q;
  };
  w.gs = take(4 * rows);
  w.dg = take(4 * d->T * d->K);
  w.dl = take(4 * d->T * ldl_of(E));
  w.dadu = take(4 * rows * 2 * d->I);
  w.dxp = take(4 * rows * d->d);
  w.dxr = take(4 * d->T * d->d);
  w.rdw = rdw_bytes(d) > 0 ? take(rdw_bytes(d)) : nullptr;
  w.lbc = take(4 * E);
  w.mt2 = w.texp2 = w.sched = nullptr;
  w.hilo = w.ghlo = w.xd = w.doutd = nullptr;
  if (use_bwdp(d)) {
    auto takeb = [&p](int64_t bytes) {
      char* q = p;
      p += a256(bytes);
      return q;
    };
    w.mt2 = reinterpret_cast<int32_t*>(takeb(4 * (d->N + 1)));
    w.texp2 = reinterpret_cast<int32_t*>(takeb(4 * max_tiles2(d)));
    w.sched = reinterpret_cast<int32_t*>(takeb(4 * kBwdSched));
    w.hilo = reinterpret_cast<bf16_t*>(takeb(rows * 4 * d->I * 2));
    w.ghlo = reinterpret_cast<bf16_t*>(takeb(rows * 2 * d->I * 2));
    w.xd = reinterpret_cast<bf16_t*>(takeb(rows * d->d * 2));
    w.doutd = reinterpret_cast<bf16_t*>(takeb(rows * d->d * 2));
  }
  return w;
}

zc_status check_ws(const void* ws, size_t ws_bytes, int64_t need) {
  if (need > 0 && (!ws || ws_bytes < static_cast<size_t>(need)))
    return fail(ZC_ERR_WORKSPACE, "workspace of %zu bytes at %p, %lld needed", ws_bytes, ws,
                (long long)need);
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(ZC_ERR_INVALID, "workspace is not 256-byte aligned");
  return ZC_OK;
}

// Load-balance loss settings against the layer: D groups of N/D FFN
// experts, 0 < K_e <= K (K_e < K when there are zero-computation experts,
// whose pick frequency divides by K - K_e), finite alpha.
zc_status check_lb(const zc_moe_desc* d, const zc_lb_cfg* lb) {
  if (!lb) return fail(ZC_ERR_INVALID, "load-balance settings are NULL");
  if (d->N < 1) return fail(ZC_ERR_INVALID, "the load-balance loss needs FFN experts (N >= 1)");
  if (lb->D < 1 || lb->D > d->N || d->N % lb->D)
    return fail(ZC_ERR_INVALID, "D=%lld does not split N=%lld into equal groups",
                (long long)lb->D, (long long)d->N);
  if (!std::isfinite(lb->K_e) || !(lb->K_e > 0.0) || lb->K_e > static_cast<double>(d->K) ||
      (d->Z > 0 && !(lb->K_e < static_cast<double>(d->K))))
    return fail(ZC_ERR_INVALID, "K_e=%g outside (0, K=%lld%s", lb->K_e, (long long)d->K,
                d->Z > 0 ? ")" : "]");
  if (!std::isfinite(lb->alpha)) return fail(ZC_ERR_INVALID, "alpha is not finite");
  return ZC_OK;
}
int64_t stats_ws_bytes(const zc_moe_desc* d) {
  return a256(static_cast<int64_t>(zc::stats_scratch_bytes(d->T, d->K)));
}
int64_t lb_ws_bytes(const zc_moe_desc* d) {
  return a256(static_cast<int64_t>(zc::lb_scratch_bytes(d->T, d->N + d->Z)));
}

// The 256 x 256 forward kernels: bf16 layers with row-major weights (with a
// saved buffer the gate/up epilogue also writes a, u, h in fp32 for the
// backward), 32-bit element offsets (rows * columns < 2^31), and on
// average at least 64 rows per FFN expert (T*K/N, known on the host without
// reading the counts back); decode-sized batches keep the 128 x 128 kernel,
// whose larger grid streams a few rows' worth of weights per expert better.
template <typename T>
bool use_fwd_kernels(const zc_moe_desc* d) {
  if (!std::is_same<T, bf16_t>::value) return false;
  if (d->N == 0 || d->T * d->K < 64 * d->N) return false;
  const int64_t rows = d->T * d->K, cols = d->I > d->d ? d->I : d->d;
  return rows * cols < (int64_t(1) << 31) && d->T * d->d < (int64_t(1) << 31);
}

// The row-major weight kernels of gemm_rmw.hip (forward, with or without
// saved activations): bf16 layers with d and I multiples of 256 whose byte
// offsets fit 31 bits.
bool rmw_layer(const zc_moe_desc* d) {
  return d->dtype == ZC_BF16 && d->N > 0 && d->weight_layout == ZC_WEIGHTS_ROWMAJOR &&
         zc::rmw_fwd_supported(d->T * d->K, d->T, d->d, d->I);
}
template <typename T>
bool use_rmw(const zc_moe_desc* d) {
  return std::is_same<T, bf16_t>::value && rmw_layer(d);
}

// Router scores on the 256 x 256-tile kernel: bf16 layers with E a multiple
// of 256 and at least 128 such tiles (T * E >= 2^23); smaller batches keep
// the generic kernel, which splits the hidden dimension to fill the GPU.
template <typename T>
bool use_dense_router(const zc_moe_desc* d) {
  const int64_t E = d->N + d->Z;
  return std::is_same<T, bf16_t>::value && d->T * E >= (int64_t(1) << 23) &&
         zc::rmw_dense_supported(d->T, E, d->d);
}

// Router + dispatch on an already validated call.
// Row-tile height of the second tile prefix (tile_off2): the packed-weight
// forward picks it from the average rows per FFN expert, the row-major
// kernels of gemm_rmw.hip likewise but at least 64 rows, the other row-major
// bf16 forward kernels use 256.
int fwd_rows_per_tile(const zc_moe_desc* d) {
  if (d->N == 0) return zc::kFwdBM;
  const int tm = zc::fwdp_rows_per_tile(d->T * d->K / d->N);
  if (d->weight_layout != ZC_WEIGHTS_ROWMAJOR) return tm;
  return rmw_layer(d) ? (tm < 64 ? 64 : tm) : zc::kFwdBM;
}

template <typename T>
zc_status do_route(const zc_moe_desc* d, const T* x, const T* wr, const float* bias,
                   zc_route_buf* r, const RouteWs& w, hipStream_t s) {
  const int Tn = static_cast<int>(d->T), E = static_cast<int>(d->N + d->Z);
  const int N = static_cast<int>(d->N), K = static_cast<int>(d->K);
  if (x && Tn > 0) {
    if (use_dense_router<T>(d))
      ZC_LAUNCH(ZC_PH_ROUTER_GEMM,
                zc::launch_rmw_dense(reinterpret_cast<const bf16_t*>(x), Tn,
                                     reinterpret_cast<const bf16_t*>(wr), E,
                                     static_cast<int>(d->d), r->logits, cus(d), s),
                "router GEMM launch");
    else
      ZC_LAUNCH(ZC_PH_ROUTER_GEMM,
                zc::launch_router_gemm<T>(x, wr, r->logits, Tn, E, static_cast<int>(d->d),
                                          w.rpart, cus(d), s),
                "router GEMM launch");
  }
  ZC_LAUNCH(ZC_PH_TOPK, zc::launch_topk(r->logits, bias, Tn, E, K, d->gate_norm, r->topk_idx, r->topk_gate, s),
         "top-K launch");
  ZC_LAUNCH(ZC_PH_DISPATCH, zc::launch_dispatch(r->topk_idx, Tn, E, N, K, zc::kGemmBM,
                                                fwd_rows_per_tile(d),
                                                r->counts, r->offsets, r->perm, r->inv, w.tile_off,
                                                w.tile_off2, w.tile_exp, w.tile_exp1, w.sched,
                                                w.dispatch, s),
         "dispatch launch");
  return ZC_OK;
}

template <typename T>
zc_status do_forward(const zc_moe_desc* d, const T* x, const T* wr, const float* bias,
                     const T* wg, const T* wu, const T* wd, T* out, zc_route_buf* r, void* saved,
                     char* ws, hipStream_t s) {
  RouteWs rw = carve_route(ws, d);
  ZC_CHECK(do_route<T>(d, x, wr, bias, r, rw, s));
  const int Tn = static_cast<int>(d->T), N = static_cast<int>(d->N), K = static_cast<int>(d->K);
  const int dd = static_cast<int>(d->d), I = static_cast<int>(d->I);
  const int64_t rows = d->T * d->K;
  char* p = ws + route_ws_bytes(d);
  T* h = reinterpret_cast<T*>(p);
  T* y = reinterpret_cast<T*>(p + a256(rows * d->I * esize(d)));
  float *sa = nullptr, *su = nullptr, *sh = nullptr;
  if (saved) {
    Saved sv = carve_saved(static_cast<char*>(saved), d);
    sa = sv.a;
    su = sv.u;
    sh = sv.h;
    y = static_cast<T*>(sv.y);
  }
  if (N > 0 && Tn > 0) {
    const int cu = cus(d);
    if (d->weight_layout == ZC_WEIGHTS_MXFP8) {
      // MXFP8 inference: x quantized once, h quantized in the gate/up
      // epilogue (validated: bf16, no saved buffer)
      uint8_t* xq = reinterpret_cast<uint8_t*>(ws + fwd_ws_bytes(d) - a256(d->T * d->d) -
                                               a256(d->T * d->d / 32));
      uint8_t* xs = xq + a256(d->T * d->d);
      uint8_t* hq = reinterpret_cast<uint8_t*>(h);
      uint8_t* hs = hq + a256(rows * d->I);
      ZC_LAUNCH(ZC_PH_QUANTIZE,
                zc::launch_mxq_rows(reinterpret_cast<const bf16_t*>(x), d->T, dd, xq, xs, s),
                "activation quantization launch");
      ZC_LAUNCH(ZC_PH_GATE_UP,
                zc::launch_fwdq_gateup(xq, xs, d->T, reinterpret_cast<const uint8_t*>(wg),
                                       reinterpret_cast<const uint8_t*>(wu), r->offsets, r->perm,
                                       rw.tile_off2, rw.tile_exp, rw.sched, fwd_rows_per_tile(d), N,
                                       I, dd, K, hq, hs, cu, s),
                "gate/up GEMM launch");
      ZC_LAUNCH(ZC_PH_DOWN,
                zc::launch_fwdq_down(hq, hs, rows, reinterpret_cast<const uint8_t*>(wd), r->offsets,
                                     rw.tile_off2, rw.tile_exp, rw.sched + 8,
                                     fwd_rows_per_tile(d), N, I, dd,
                                     reinterpret_cast<bf16_t*>(y), cu, s),
                "down GEMM launch");
    } else if (d->weight_layout == ZC_WEIGHTS_PACKED) {
      // bf16 inference on packed weights (validated: bf16, no saved buffer)
      const bf16_t* hx = reinterpret_cast<const bf16_t*>(x);
      bf16_t* hh = reinterpret_cast<bf16_t*>(h);
      ZC_LAUNCH(ZC_PH_GATE_UP,
                zc::launch_fwdp_gateup(hx, d->T * d->d, reinterpret_cast<const bf16_t*>(wg),
                                       reinterpret_cast<const bf16_t*>(wu), r->offsets, r->perm,
                                       rw.tile_off2, rw.tile_exp, rw.sched, fwd_rows_per_tile(d), N,
                                       I, dd, K, hh, cu, s),
                "gate/up GEMM launch");
      ZC_LAUNCH(ZC_PH_DOWN,
                zc::launch_fwdp_down(hh, rows * d->I, reinterpret_cast<const bf16_t*>(wd),
                                     r->offsets, rw.tile_off2, rw.tile_exp, rw.sched + 8,
                                     fwd_rows_per_tile(d), N, I, dd, reinterpret_cast<bf16_t*>(y),
                                     cu, s),
                "down GEMM launch");
    } else if (use_rmw<T>(d)) {
      // bf16 on row-major weights; with a saved buffer (training) a, u, h
      // are also kept in fp32
      ZC_LAUNCH(ZC_PH_GATE_UP,
                zc::launch_rmw_gateup(reinterpret_cast<const bf16_t*>(x), d->T,
                                      reinterpret_cast<const bf16_t*>(wg),
                                      reinterpret_cast<const bf16_t*>(wu), r->offsets, r->perm,
                                      rw.tile_off2, rw.tile_exp, rw.sched, fwd_rows_per_tile(d), N,
                                      I, dd, K, reinterpret_cast<bf16_t*>(h), sa, su, sh, cu, s),
                "gate/up GEMM launch");
      ZC_LAUNCH(ZC_PH_DOWN,
                zc::launch_rmw_down(reinterpret_cast<const bf16_t*>(h), rows,
                                    reinterpret_cast<const bf16_t*>(wd), r->offsets, rw.tile_off2,
                                    rw.tile_exp, rw.sched + 8, fwd_rows_per_tile(d), N, I, dd,
                                    reinterpret_cast<bf16_t*>(y), cu, s),
                "down GEMM launch");
    } else if (use_fwd_kernels<T>(d)) {
      // bf16 on row-major weights whose d or I is not a multiple of 256:
      // 256 x 256 tiles, weights streamed once per expert; with a saved
      // buffer the gate/up epilogue also keeps a, u, h
      ZC_LAUNCH(ZC_PH_GATE_UP,
                zc::launch_fwd_gateup(reinterpret_cast<const bf16_t*>(x),
                                      reinterpret_cast<const bf16_t*>(wg),
                                      reinterpret_cast<const bf16_t*>(wu), r->offsets, r->perm,
                                      rw.tile_off2, N, I, dd, K, reinterpret_cast<bf16_t*>(h),
                                      sa, su, sh, cu, s),
                "gate/up GEMM launch");
      ZC_LAUNCH(ZC_PH_DOWN,
                zc::launch_fwd_down(reinterpret_cast<const bf16_t*>(h),
                                    reinterpret_cast<const bf16_t*>(wd), r->offsets, rw.tile_off2, N,
                                    I, dd, reinterpret_cast<bf16_t*>(y), cu, s),
                "down GEMM launch");
    } else {
      ZC_LAUNCH(ZC_PH_GATE_UP, zc::launch_ffn_gateup<T>(x, wg, wu, r->offsets, r->perm, rw.tile_off,
                                                        N, I, dd, K, rows, h, sa, su, sh, cu, s),
                "gate/up GEMM launch");
      ZC_LAUNCH(ZC_PH_DOWN, zc::launch_ffn_down<T>(h, wd, r->offsets, rw.tile_off, N, I, dd, rows,
                                                   y, cu, s),
                "down GEMM launch");
    }
  }
  ZC_LAUNCH(ZC_PH_COMBINE, zc::launch_combine<T>(x, y, r->topk_idx, r->topk_gate, r->inv, Tn, dd, N, K, d->out_scale,
                               out, s),
         "combine launch");
  return ZC_OK;
}

template <typename T>
zc_status do_backward(const zc_moe_desc* d, const T* x, const T* wr, const T* wg, const T* wu,
                      const T* wd, const zc_route_buf* r, const void* saved, const T* dout, T* dx,
                      T* dwr, T* dwg, T* dwu, T* dwd, const zc_lb_cfg* lb, char* ws,
                      hipStream_t s) {
  const int Tn = static_cast<int>(d->T), N = static_cast<int>(d->N), K = static_cast<int>(d->K);
  const int E = static_cast<int>(d->N + d->Z), dd = static_cast<int>(d->d);
  const int I = static_cast<int>(d->I), ldl = static_cast<int>(ldl_of(E));
  const int64_t rows = d->T * d->K;
  const int cu = cus(d);
  BwdWs w = carve_bwd(ws, d);
  Saved sv = carve_saved(const_cast<char*>(static_cast<const char*>(saved)), d);
  const T* y = static_cast<const T*>(sv.y);
  const bool bwdp = std::is_same<T, bf16_t>::value && use_bwdp(d);
  const int tmb = bwdp ? bwdp_rows_per_tile(d) : 0;
  if (N > 0) {
    if (bwdp) {
      ZC_LAUNCH(ZC_PH_TILE_OFFSETS,
                zc::launch_tile_offsets2(r->offsets, N, zc::kGemmBM, w.tile_off, tmb, w.mt2,
                                         w.texp2, w.sched, kBwdSched, s),
                "tile offsets");
    } else {
      ZC_LAUNCH(ZC_PH_TILE_OFFSETS,
                zc::launch_tile_offsets(r->offsets, N, zc::kGemmBM, w.tile_off, s), "tile offsets");
    }
  }
  if (lb)
    ZC_LAUNCH(ZC_PH_LB_COEF,
              zc::launch_lb_coef(r->counts, Tn, N, E, K, static_cast<int>(lb->D), lb->K_e,
                                 lb->alpha, w.lbc, s),
              "load-balance coefficient launch");
  ZC_LAUNCH(ZC_PH_BWD_COMBINE,
            zc::launch_combine_bwd<T>(x, y, dout, r->logits, r->topk_idx, r->topk_gate, r->inv, Tn,
                                      dd, N, E, K, d->gate_norm, d->out_scale,
                                      lb ? w.lbc : nullptr, w.gs, w.dg, w.dl, ldl, s),
            "combine backward launch");
  if (N > 0) {
    if (Tn > 0 && bwdp) {
      ZC_LAUNCH(ZC_PH_BWD_GATHER,
                zc::launch_gather_rows(reinterpret_cast<const bf16_t*>(dout), r->perm, r->offsets,
                                       N, K, dd, rows, w.doutd, s),
                "row gather launch");
      ZC_LAUNCH(ZC_PH_BWD_GATHER,
                zc::launch_gather_rows(reinterpret_cast<const bf16_t*>(x), r->perm, r->offsets, N,
                                       K, dd, rows, w.xd, s),
                "row gather launch");
      ZC_LAUNCH(ZC_PH_BWD_DOWN_DH,
                zc::launch_rmw_dh(w.doutd, rows, reinterpret_cast<const bf16_t*>(wd), r->offsets,
                                  w.mt2, w.texp2, w.sched, tmb, N, I, dd, w.gs, w.dadu, cu, s),
                "down backward (dh) launch");
      ZC_LAUNCH(ZC_PH_BWD_DOWN_DH,
                zc::launch_swiglu_bwd(w.dadu, w.gs, sv.a, sv.u, sv.h, r->offsets, N, I, rows,
                                      w.hilo, w.ghlo, s),
                "SwiGLU backward launch");
    } else if (Tn > 0) {
      ZC_LAUNCH(ZC_PH_BWD_DOWN_DH,
                zc::launch_bwd_down_dh<T>(dout, r->perm, K, w.gs, wd, sv.a, sv.u, r->offsets,
                                          w.tile_off, N, I, dd, rows, w.dadu, cu, s),
                "down backward (dh) launch");
    }
    if (bwdp)
      ZC_LAUNCH(ZC_PH_BWD_DOWN_DW,
                zc::launch_dw(true, N, I, dd, r->offsets, w.sched + 16, w.ghlo, w.ghlo + I, 2 * I,
                              w.doutd, dd, rows, reinterpret_cast<bf16_t*>(dwd), cu, s),
                "down weight-gradient launch");
    else
      ZC_LAUNCH(ZC_PH_BWD_DOWN_DW,
                zc::launch_bwd_down_dw<T>(dout, r->perm, K, sv.h, w.gs, r->offsets, N, I, dd, dwd,
                                          cu, s),
                "down weight-gradient launch");
    if (Tn > 0 && bwdp) {
      ZC_LAUNCH(ZC_PH_BWD_GATE_UP_DX,
                zc::launch_rmw_dx(w.hilo, rows, reinterpret_cast<const bf16_t*>(wg),
                                  reinterpret_cast<const bf16_t*>(wu), r->offsets, w.mt2, w.texp2,
                                  w.sched + 8, tmb, N, I, dd, w.dxp, cu, s),
                "gate/up backward (dx) launch");
    } else if (Tn > 0) {
      ZC_LAUNCH(ZC_PH_BWD_GATE_UP_DX,
                zc::launch_bwd_gateup_dx<T>(w.dadu, wg, wu, r->offsets, w.tile_off, N, I, dd, rows,
                                            w.dxp, cu, s),
                "gate/up backward (dx) launch");
    }
    if (bwdp) {
      ZC_LAUNCH(ZC_PH_BWD_GATE_UP_DW,
                zc::launch_dw(false, N, I, dd, r->offsets, w.sched + 24, w.hilo, w.hilo + I, 4 * I,
                              w.xd, dd, rows, reinterpret_cast<bf16_t*>(dwg), cu, s),
                "gate/up weight-gradient launch");
      ZC_LAUNCH(ZC_PH_BWD_GATE_UP_DW,
                zc::launch_dw(false, N, I, dd, r->offsets, w.sched + 32, w.hilo + 2 * I,
                              w.hilo + 3 * I, 4 * I, w.xd, dd, rows, reinterpret_cast<bf16_t*>(dwu),
                              cu, s),
                "gate/up weight-gradient launch");
    } else {
      ZC_LAUNCH(ZC_PH_BWD_GATE_UP_DW,
                zc::launch_bwd_gateup_dw<T>(w.dadu, x, r->offsets, r->perm, N, I, dd, K, dwg, dwu,
                                            cu, s),
                "gate/up weight-gradient launch");
    }
  }
  ZC_LAUNCH(ZC_PH_BWD_ROUTER_DW, zc::launch_router_dw<T>(w.dl, ldl, x, Tn, E, dd, dwr, w.rdw, cu, s),
            "router weight-gradient launch");
  if (Tn > 0) {
    ZC_LAUNCH(ZC_PH_BWD_ROUTER_DX, zc::launch_router_dx<T>(w.dl, ldl, wr, Tn, E, dd, w.dxr, cu, s),
              "router dx launch");
    ZC_LAUNCH(ZC_PH_BWD_DX_GATHER,
              zc::launch_dx_gather<T>(dout, w.dxp, w.dxr, r->topk_idx, r->topk_gate, r->inv, Tn, dd,
                                      N, K, d->out_scale, dx, s),
              "dx gather launch");
  }
  return ZC_OK;
}

// ---- scratch of the allocation-free forward (zc_moe_forward_noalloc)
// A file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  Host code never uses
// the array's name as a device address: scratch_ptr() looks each device's
// copy up once (hipGetSymbolAddress, with that device current) and keeps it.
constexpr size_t kNoAllocScratch = size_t(64) << 20;  // ZC_NOALLOC_SCRATCH_BYTES
static __device__ __align__(256) char scratch[kNoAllocScratch];
static_assert(kNoAllocScratch == ZC_NOALLOC_SCRATCH_BYTES, "header and library disagree");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

zc_status scratch_ptr(void** out) {
  int dev = -1;
  ZC_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ZC_ERR_UNSUPPORTED, "device %d: the allocation-free forward tracks devices 0..%d",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    ZC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(ZC_ERR_HIP, "scratch of device %d at %p is not 256-byte aligned", dev, p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ZC_OK;
}

zc_status check_weights(const zc_moe_desc* d, const void* wg, const void* wu, const void* wd) {
  const bool opt = d->N == 0;
  ZC_CHECK(check_ptr(wg, "w_gate", opt));
  ZC_CHECK(check_ptr(wu, "w_up", opt));
  ZC_CHECK(check_ptr(wd, "w_down", opt));
  return ZC_OK;
}

}  // namespace

extern "C" {

size_t zc_moe_workspace_size(const zc_moe_desc* desc, int op) {
  if (check_desc(desc) != ZC_OK) return 0;
  switch (op) {
    case ZC_OP_ROUTE: return static_cast<size_t>(route_ws_bytes(desc));
    case ZC_OP_FORWARD: return static_cast<size_t>(fwd_ws_bytes(desc));
    case ZC_OP_BACKWARD: return static_cast<size_t>(bwd_ws_bytes(desc));
    case ZC_OP_LB_LOSS: return static_cast<size_t>(lb_ws_bytes(desc));
    case ZC_OP_ROUTE_STATS: return static_cast<size_t>(stats_ws_bytes(desc));
    default: return 0;
  }
}

size_t zc_moe_saved_size(const zc_moe_desc* desc) {
  if (check_desc(desc) != ZC_OK) return 0;
  return static_cast<size_t>(saved_bytes(desc));
}

zc_status zc_moe_route(const zc_moe_desc* desc, const void* x, const void* w_router,
                       const float* bias, zc_route_buf* r, void* ws, size_t ws_bytes,
                       void* stream) {
  ZC_CHECK(check_desc(desc));
  ZC_CHECK(check_route(r, desc->T == 0));
  ZC_CHECK(check_ptr(bias, "bias"));
  if ((x == nullptr) != (w_router == nullptr) && desc->T > 0)
    return fail(ZC_ERR_INVALID, "x and w_router must both be set or both be NULL");
  ZC_CHECK(check_ptr(x, "x", true));
  ZC_CHECK(check_ptr(w_router, "w_router", true));
  ZC_CHECK(check_ws(ws, ws_bytes, route_ws_bytes(desc)));
  RouteWs w = carve_route(static_cast<char*>(ws), desc);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (desc->dtype == ZC_BF16)
    return do_route<bf16_t>(desc, static_cast<const bf16_t*>(x),
                            static_cast<const bf16_t*>(w_router), bias, r, w, s);
  return do_route<float>(desc, static_cast<const float*>(x), static_cast<const float*>(w_router),
                         bias, r, w, s);
}

zc_status zc_moe_forward(const zc_moe_desc* desc, const void* x, const void* w_router,
                         const float* bias, const void* w_gate, const void* w_up,
                         const void* w_down, void* out, zc_route_buf* r, void* saved, void* ws,
                         size_t ws_bytes, void* stream) {
  ZC_CHECK(check_desc(desc));
  const bool none = desc->T == 0;
  ZC_CHECK(check_route(r, none));
  ZC_CHECK(check_ptr(x, "x", none));
  ZC_CHECK(check_ptr(w_router, "w_router"));
  ZC_CHECK(check_ptr(bias, "bias"));
  ZC_CHECK(check_weights(desc, w_gate, w_up, w_down));
  ZC_CHECK(check_ptr(out, "out", none));
  ZC_CHECK(check_ptr(saved, "saved", true));
  if (saved && desc->weight_layout != ZC_WEIGHTS_ROWMAJOR)
    return fail(ZC_ERR_UNSUPPORTED, "a forward that saves activations needs row-major weights");
  ZC_CHECK(check_ws(ws, ws_bytes, fwd_ws_bytes(desc)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (desc->dtype == ZC_BF16)
    return do_forward<bf16_t>(desc, static_cast<const bf16_t*>(x),
                              static_cast<const bf16_t*>(w_router), bias,
                              static_cast<const bf16_t*>(w_gate), static_cast<const bf16_t*>(w_up),
                              static_cast<const bf16_t*>(w_down), static_cast<bf16_t*>(out), r,
                              saved, w, s);
  return do_forward<float>(desc, static_cast<const float*>(x), static_cast<const float*>(w_router),
                           bias, static_cast<const float*>(w_gate),
                           static_cast<const float*>(w_up), static_cast<const float*>(w_down),
                           static_cast<float*>(out), r, saved, w, s);
}

zc_status zc_moe_forward_noalloc(const zc_moe_desc* desc, const void* x, const void* w_router,
                                 const float* bias, const void* w_gate, const void* w_up,
                                 const void* w_down, void* out, zc_route_buf* r, void* stream) {
  ZC_CHECK(check_desc(desc));
  const int64_t need = fwd_ws_bytes(desc);
  if (need > static_cast<int64_t>(kNoAllocScratch))
    return fail(ZC_ERR_WORKSPACE,
                "the allocation-free forward holds %zu bytes of scratch per device; this layer "
                "needs %lld (zc_moe_workspace_size(desc, ZC_OP_FORWARD))",
                kNoAllocScratch, (long long)need);
  void* ws = nullptr;
  ZC_CHECK(scratch_ptr(&ws));
  t_no_events = true;
  const zc_status st = zc_moe_forward(desc, x, w_router, bias, w_gate, w_up, w_down, out, r,
                                      nullptr, ws, kNoAllocScratch, stream);
  t_no_events = false;
  return st;
}

zc_status zc_moe_backward(const zc_moe_desc* desc, const void* x, const void* w_router,
                          const void* w_gate, const void* w_up, const void* w_down,
                          const zc_route_buf* r, const void* saved, const void* dout, void* dx,
                          void* dw_router, void* dw_gate, void* dw_up, void* dw_down,
                          const zc_lb_cfg* lb, void* ws, size_t ws_bytes, void* stream) {
  ZC_CHECK(check_desc(desc));
  if (desc->weight_layout != ZC_WEIGHTS_ROWMAJOR)
    return fail(ZC_ERR_UNSUPPORTED, "the backward needs row-major weights");
  const bool none = desc->T == 0;
  ZC_CHECK(check_route(r, none));
  ZC_CHECK(check_ptr(x, "x", none));
  ZC_CHECK(check_ptr(w_router, "w_router"));
  ZC_CHECK(check_weights(desc, w_gate, w_up, w_down));
  ZC_CHECK(check_ptr(saved, "saved", none));
  ZC_CHECK(check_ptr(dout, "dout", none));
  ZC_CHECK(check_ptr(dx, "dx", none));
  ZC_CHECK(check_ptr(dw_router, "dw_router"));
  ZC_CHECK(check_weights(desc, dw_gate, dw_up, dw_down));
  if (lb) ZC_CHECK(check_lb(desc, lb));
  ZC_CHECK(check_ws(ws, ws_bytes, bwd_ws_bytes(desc)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (desc->dtype == ZC_BF16)
    return do_backward<bf16_t>(
        desc, static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router),
        static_cast<const bf16_t*>(w_gate), static_cast<const bf16_t*>(w_up),
        static_cast<const bf16_t*>(w_down), r, saved, static_cast<const bf16_t*>(dout),
        static_cast<bf16_t*>(dx), static_cast<bf16_t*>(dw_router), static_cast<bf16_t*>(dw_gate),
        static_cast<bf16_t*>(dw_up), static_cast<bf16_t*>(dw_down), lb, w, s);
  return do_backward<float>(desc, static_cast<const float*>(x), static_cast<const float*>(w_router),
                            static_cast<const float*>(w_gate), static_cast<const float*>(w_up),
                            static_cast<const float*>(w_down), r, saved,
                            static_cast<const float*>(dout), static_cast<float*>(dx),
                            static_cast<float*>(dw_router), static_cast<float*>(dw_gate),
                            static_cast<float*>(dw_up), static_cast<float*>(dw_down), lb, w, s);
}

zc_status zc_moe_lb_loss(const zc_moe_desc* desc, const zc_lb_cfg* lb, const zc_route_buf* r,
                         double* out, void* ws, size_t ws_bytes, void* stream) {
  ZC_CHECK(check_desc(desc));
  ZC_CHECK(check_lb(desc, lb));
  if (!r) return fail(ZC_ERR_INVALID, "route buffer is NULL");
  ZC_CHECK(check_ptr(r->logits, "r->logits", desc->T == 0));
  ZC_CHECK(check_ptr(r->counts, "r->counts"));
  ZC_CHECK(check_ptr(out, "out"));
  ZC_CHECK(check_ws(ws, ws_bytes, lb_ws_bytes(desc)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = static_cast<int>(desc->N + desc->Z);
  ZC_LAUNCH(ZC_PH_LB_LOSS,
            zc::launch_lb_loss(r->logits, r->counts, static_cast<int>(desc->T),
                               static_cast<int>(desc->N), E, static_cast<int>(desc->K),
                               static_cast<int>(lb->D), lb->K_e, lb->alpha, out, ws, s),
            "load-balance loss launch");
  return ZC_OK;
}

zc_status zc_moe_route_stats(const zc_moe_desc* desc, const zc_route_buf* r, int32_t* hist,
                             double* moments, void* ws, size_t ws_bytes, void* stream) {
  ZC_CHECK(check_desc(desc));
  if (!r) return fail(ZC_ERR_INVALID, "route buffer is NULL");
  ZC_CHECK(check_ptr(r->topk_idx, "r->topk_idx", desc->T == 0));
  ZC_CHECK(check_ptr(hist, "hist"));
  ZC_CHECK(check_ptr(moments, "moments"));
  ZC_CHECK(check_ws(ws, ws_bytes, stats_ws_bytes(desc)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  ZC_LAUNCH(ZC_PH_ROUTE_STATS,
            zc::launch_route_stats(r->topk_idx, static_cast<int>(desc->T),
                                   static_cast<int>(desc->N), static_cast<int>(desc->K), hist,
                                   moments, ws, s),
            "routing statistics launch");
  return ZC_OK;
}

zc_status zc_moe_accumulate_counts(int64_t E, const int32_t* counts, int32_t* acc, void* stream) {
  if (E < 1 || E > 1024) return fail(ZC_ERR_INVALID, "E=%lld outside 1..1024", (long long)E);
  ZC_CHECK(check_ptr(counts, "counts"));
  ZC_CHECK(check_ptr(acc, "acc"));
  if (counts == acc) return fail(ZC_ERR_INVALID, "counts and acc are the same buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  ZC_LAUNCH(ZC_PH_ACCUMULATE, zc::launch_accumulate_counts(counts, static_cast<int>(E), acc, s),
            "count accumulation launch");
  return ZC_OK;
}

zc_status zc_moe_pack_weights(const zc_moe_desc* desc, int which, const void* src, void* dst,
                              void* stream) {
  ZC_CHECK(check_desc(desc));
  if (desc->dtype != ZC_BF16) return fail(ZC_ERR_UNSUPPORTED, "packed weights need a bf16 layer");
  if (desc->d % 256 || desc->I % 256)
    return fail(ZC_ERR_UNSUPPORTED, "packed weights need d and I multiples of 256 (d=%lld I=%lld)",
                (long long)desc->d, (long long)desc->I);
  if (which != ZC_PACK_GATE_UP && which != ZC_PACK_DOWN)
    return fail(ZC_ERR_INVALID, "which=%d is neither ZC_PACK_GATE_UP nor ZC_PACK_DOWN", which);
  const bool opt = desc->N == 0;
  ZC_CHECK(check_ptr(src, "src", opt));
  ZC_CHECK(check_ptr(dst, "dst", opt));
  const int64_t bytes = desc->N * desc->I * desc->d * 2;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (bytes > 0 && a < b + bytes && b < a + bytes)
    return fail(ZC_ERR_INVALID, "src and dst overlap");
  if (desc->N == 0) return ZC_OK;
  const int R = static_cast<int>(which == ZC_PACK_GATE_UP ? desc->I : desc->d);
  const int C = static_cast<int>(which == ZC_PACK_GATE_UP ? desc->d : desc->I);
  hipError_t e = zc::launch_pack_weights(static_cast<const bf16_t*>(src), static_cast<bf16_t*>(dst),
                                         desc->N, R, C, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "weight packing launch");
  return ZC_OK;
}

size_t zc_moe_quantized_weight_bytes(const zc_moe_desc* desc) {
  if (check_desc(desc) != ZC_OK) return 0;
  const int64_t n = desc->N * desc->I * desc->d;
  return static_cast<size_t>(n + n / 32);
}

zc_status zc_moe_quantize_weights(const zc_moe_desc* desc, int which, const void* src, void* dst,
                                  void* stream) {
  ZC_CHECK(check_desc(desc));
  ZC_CHECK(check_mxfp8(desc));
  if (which != ZC_PACK_GATE_UP && which != ZC_PACK_DOWN)
    return fail(ZC_ERR_INVALID, "which=%d is neither ZC_PACK_GATE_UP nor ZC_PACK_DOWN", which);
  const bool opt = desc->N == 0;
  ZC_CHECK(check_ptr(src, "src", opt));
  ZC_CHECK(check_ptr(dst, "dst", opt));
  const int64_t sbytes = desc->N * desc->I * desc->d * 2;
  const int64_t dbytes = static_cast<int64_t>(zc_moe_quantized_weight_bytes(desc));
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (sbytes > 0 && a < b + dbytes && b < a + sbytes)
    return fail(ZC_ERR_INVALID, "src and dst overlap");
  if (desc->N == 0) return ZC_OK;
  const int R = static_cast<int>(which == ZC_PACK_GATE_UP ? desc->I : desc->d);
  const int C = static_cast<int>(which == ZC_PACK_GATE_UP ? desc->d : desc->I);
  hipError_t e = zc::launch_mxq_weights(static_cast<const bf16_t*>(src), static_cast<uint8_t*>(dst),
                                        desc->N, R, C, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "weight quantization launch");
  return ZC_OK;
}

zc_status zc_moe_pid_update(int64_t N, int64_t Z, int64_t K, const int32_t* counts, int64_t T_all,
                            double mu, double K_e, float* bias, void* stream) {
  if (N < 0 || Z < 0 || N + Z < 1 || N + Z > 1024)
    return fail(ZC_ERR_INVALID, "N=%lld Z=%lld: need N, Z >= 0 and 1 <= N+Z <= 1024",
                (long long)N, (long long)Z);
  if (K < 1 || T_all < 1) return fail(ZC_ERR_INVALID, "K and T_all must be >= 1");
  if (!std::isfinite(mu) || !std::isfinite(K_e)) return fail(ZC_ERR_INVALID, "mu or K_e not finite");
  ZC_CHECK(check_ptr(counts, "counts"));
  ZC_CHECK(check_ptr(bias, "bias"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  ZC_LAUNCH(ZC_PH_BIAS_UPDATE, zc::launch_pid(static_cast<int>(N), static_cast<int>(K), counts, T_all, mu, K_e, bias, s),
         "bias update launch");
  return ZC_OK;
}

zc_status zc_moe_profile(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!on) drop_records();
  g_prof_on.store(on != 0);
  return ZC_OK;
}

zc_status zc_moe_profile_read(double* total_ms, int32_t* count) {
  if (!total_ms || !count) return fail(ZC_ERR_INVALID, "total_ms and count must be host arrays");
  for (int i = 0; i < ZC_NUM_PHASES; ++i) {
    total_ms[i] = 0.0;
    count[i] = 0;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  zc_status st = ZC_OK;
  for (auto& r : g_prof_recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      st = hip_fail(e, "reading kernel timing events");
      continue;
    }
    total_ms[r.phase] += ms;
    count[r.phase] += 1;
  }
  drop_records();
  return st;
}

const char* zc_moe_phase_name(int phase) {
  static const char* names[ZC_NUM_PHASES] = {
      "router_gemm", "topk", "dispatch", "gate_up_gemm", "down_gemm", "combine",
      "bwd_combine", "bwd_down_dh", "bwd_down_dw", "bwd_gate_up_dx", "bwd_gate_up_dw",
      "bwd_router_dw", "bwd_router_dx", "bwd_dx_gather", "bias_update", "tile_offsets",
      "lb_loss", "lb_coef", "route_stats", "accumulate_counts", "quantize", "bwd_gather"};
  return (phase >= 0 && phase < ZC_NUM_PHASES) ? names[phase] : "";
}

const char* zc_status_string(zc_status s) {
  // callers from C or Python may pass any int: read it as one, never as an
  // out-of-range value of the enum type
  int v = 0;
  static_assert(sizeof v == sizeof s, "zc_status is an int");
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case ZC_OK: return "ok";
    case ZC_ERR_INVALID: return "invalid argument";
    case ZC_ERR_UNSUPPORTED: return "unsupported shape";
    case ZC_ERR_WORKSPACE: return "workspace too small";
    case ZC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* zc_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

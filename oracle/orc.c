/*
 * orc.c -- fp64 CPU oracle for the MoE layer with zero-computation experts.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant table with the
 * HIP library; the two sides agree only through the written specification of
 * each step below.
 *
 * Source: "LongCat-Flash Technical Report" (Chinese translation on
 * 171host.com), section 2.1 "Zero-computation experts", Eq.(1) and the
 * expert definition E_i that follows it, section 2.1.1 "Computation
 * budget control", Eq.(2), and section 2.1.2 "Load balance control" (the
 * device-level loss L_LB with Eq.(4) and Eq.(5)); the routing telemetry
 * follows the statistics section 2.1.1 records (Fig.3b/3c).  The FFN expert form (SwiGLU without biases) and
 * the linear softmax router are readings of points the page leaves open.
 *
 * Every floating-point step runs in binary64 on the exact values of the
 * (fp32 or bf16) inputs, in plain loop order.  The only place where the
 * oracle follows an arithmetic recipe rather than "whatever libm does" is
 * the routing key (orc_exp + 64-way partial sums), because a float value
 * there decides an integer (the top-K set) and both sides must take that
 * decision with the same binary64 operations.  Build with
 * -ffp-contract=off so that no multiply-add is fused behind our back.
 *
 * Parity pins: every function here is pinned by the CPU tests (brute-force
 * top-K, closed forms, library special cases, finite differences); none is
 * "parity unpinned".
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Exact widening of one stored input element to binary64. */
static double ld(const void* base, int dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Routing-key exponential.
 *
 * Cody-Waite argument reduction (W. J. Cody and W. Waite, "Software Manual
 * for the Elementary Functions", 1980): z = k ln2 + r with k = rint(z/ln2)
 * and ln2 split into a 32-significant-bit head and a binary64 tail, then the
 * Taylor series of e^r to degree 13 by Horner's rule with fused
 * multiply-adds, then scaling by 2^k.  Inputs below -700 return 0 (the
 * probability is then below 1e-304 and only matters through exact ties).
 *   head = 2977044472 / 2^32                (ln 2 rounded to 32 bits)
 *   tail = ln 2 - head, rounded to binary64
 *   inv  = 1/ln 2 rounded to binary64
 */
static const double ORC_LN2_HEAD = 0x1.62e42ff000000p-1;
static const double ORC_LN2_TAIL = -0x1.718432a1b0e26p-35;
static const double ORC_INV_LN2 = 0x1.71547652b82fep+0;

double orc_exp(double z) {
  if (isnan(z)) return z;
  if (z < -700.0) return 0.0;
  double k = rint(z * ORC_INV_LN2);
  double r = (z - k * ORC_LN2_HEAD) - k * ORC_LN2_TAIL;
  /* 1/n! for n = 13 .. 0, each the correctly rounded quotient. */
  static const double inv_fact[14] = {
      1.0 / 6227020800.0, 1.0 / 479001600.0, 1.0 / 39916800.0,
      1.0 / 3628800.0,    1.0 / 362880.0,    1.0 / 40320.0,
      1.0 / 5040.0,       1.0 / 720.0,       1.0 / 120.0,
      1.0 / 24.0,         1.0 / 6.0,         1.0 / 2.0,
      1.0,                1.0};
  double p = inv_fact[0];
  for (int n = 1; n < 14; ++n) p = fma(p, r, inv_fact[n]);
  return ldexp(p, (int)k);
}

/* Sum of e[0..E) in the fixed order used for the routing denominator:
 * 64 partial sums (partial lambda takes indices j with j mod 64 == lambda,
 * ascending, starting from 0.0), then six pairwise rounds in which every
 * partial becomes itself plus its partner at xor distance 32, 16, 8, 4, 2, 1.
 * All partials end equal; return partial 0. */
static double orc_sum64(const double* e, int64_t E) {
  double part[64], nxt[64];
  for (int l = 0; l < 64; ++l) part[l] = 0.0;
  for (int64_t j = 0; j < E; ++j) part[j % 64] = part[j % 64] + e[j];
  for (int o = 32; o >= 1; o >>= 1) {
    for (int l = 0; l < 64; ++l) nxt[l] = part[l] + part[l ^ o];
    for (int l = 0; l < 64; ++l) part[l] = nxt[l];
  }
  return part[0];
}

/* Threads the OpenMP loops below will use. */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* O1 -- router logits l[t][j] = sum_k x[t][k] * Wr[j][k]  (k ascending).
 * The page calls R a softmax router and prints no formula for its scores;
 * the plain reading is a bias-free linear map of x_t, one row per expert. */
int orc_logits(int64_t T, int64_t d, int64_t E, int dt, const void* x,
               const void* wr, double* logits) {
  if (T < 0 || d <= 0 || E <= 0 || !x || !wr || !logits) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < E; ++j) {
      double s = 0.0;
      for (int64_t k = 0; k < d; ++k) s += ld(x, dt, t * d + k) * ld(wr, dt, j * d + k);
      logits[t * E + j] = s;
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O2..O5 -- Eq.(1): keys R_i + b_i, TopK, gates; then the per-expert token
 * counts T_i of Eq.(2) and the canonical dispatch order.
 *
 *  keys:   m = max_j l_j; e_j = orc_exp(l_j - m); S = orc_sum64(e);
 *          p_j = e_j / S; key_j = p_j + (double)b_j; a NaN key counts
 *          as -infinity (a NaN or infinite score makes all of a token's
 *          keys NaN; the selection below then stays total: picks 0..K-1,
 *          NaN gates).
 *  top-K:  K rounds; round r takes the unselected j with the largest key,
 *          equal keys going to the smaller j.  Slot r is the r-th pick.
 *  gates:  gate_norm = 1: g_r = e_{s_r} / (sum_{q<K} e_{s_q}, q ascending)
 *          (softmax restricted to the picks: the selected R_i rescaled to
 *          sum to one); gate_norm = 0: g_r = p_{s_r} (Eq.(1) as printed).
 *  counts: counts[j] = number of tokens whose picks include j (all E).
 *  offsets[e] = sum of counts over FFN experts e' < e, e = 0..N.
 *  perm:   for e = 0..N-1, for t ascending with e among its picks, append
 *          the flat slot t*K + r.  (expert, token) pairs are unique, so this
 *          order is the only stable one.
 *  inv:    inv[t*K + r] = position of that slot in perm, or -1 when the
 *          pick is a zero-computation expert (j >= N).
 * Any output pointer except topk_idx may be NULL. */
int orc_route(int64_t T, int64_t E, int64_t N, int64_t K, int gate_norm,
              const double* logits, const float* bias, double* keys_out,
              int32_t* topk_idx, double* gates, int32_t* counts,
              int32_t* offsets, int32_t* perm, int32_t* inv) {
  if (T < 0 || E <= 0 || N < 0 || N > E || K < 1 || K > E || !logits || !bias || !topk_idx)
    return 1;
#pragma omp parallel
  {
    double* e = (double*)malloc(sizeof(double) * (size_t)E);
    double* key = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double* l = logits + t * E;
      double m = l[0];
      for (int64_t j = 1; j < E; ++j)
        if (l[j] > m) m = l[j];
      for (int64_t j = 0; j < E; ++j) e[j] = orc_exp(l[j] - m);
      double S = orc_sum64(e, E);
      for (int64_t j = 0; j < E; ++j) {
        key[j] = e[j] / S + (double)bias[j];
        if (isnan(key[j])) key[j] = -INFINITY;
        taken[j] = 0;
      }
      if (keys_out)
        for (int64_t j = 0; j < E; ++j) keys_out[t * E + j] = key[j];
      for (int64_t r = 0; r < K; ++r) {
        int64_t best = -1;
        for (int64_t j = 0; j < E; ++j) {
          if (taken[j]) continue;
          if (best < 0 || key[j] > key[best]) best = j;
        }
        taken[best] = 1;
        topk_idx[t * K + r] = (int32_t)best;
      }
      if (gates) {
        double den = 0.0;
        for (int64_t r = 0; r < K; ++r) den = den + e[topk_idx[t * K + r]];
        for (int64_t r = 0; r < K; ++r) {
          double er = e[topk_idx[t * K + r]];
          gates[t * K + r] = gate_norm ? er / den : er / S;
        }
      }
    }
    free(e);
    free(key);
    free(taken);
  }
  if (counts || offsets || perm || inv) {
    int32_t* cnt = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int64_t i = 0; i < T * K; ++i) cnt[topk_idx[i]] += 1;
    if (counts) memcpy(counts, cnt, sizeof(int32_t) * (size_t)E);
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
    off[0] = 0;
    for (int64_t j = 0; j < N; ++j) off[j + 1] = off[j] + cnt[j];
    if (offsets) memcpy(offsets, off, sizeof(int32_t) * (size_t)(N + 1));
    if (inv)
      for (int64_t i = 0; i < T * K; ++i) inv[i] = -1;
    if (perm || inv) {
      int32_t* cur = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
      memcpy(cur, off, sizeof(int32_t) * (size_t)(N + 1));
      /* walking tokens in ascending order and appending to each expert's
       * segment yields exactly the (expert, token) order */
      for (int64_t t = 0; t < T; ++t)
        for (int64_t r = 0; r < K; ++r) {
          int32_t j = topk_idx[t * K + r];
          if (j >= N) continue;
          int32_t pos = cur[j]++;
          if (perm) perm[pos] = (int32_t)(t * K + r);
          if (inv) inv[t * K + r] = pos;
        }
      free(cur);
    }
    free(off);
    free(cnt);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O6 -- one FFN expert on one token row (SwiGLU, no biases):
 *   a = Wg x,  u = Wu x,  h = silu(a) * u,  y = Wd h,  silu(z) = z/(1+e^-z).
 * Wg, Wu are [I][d] and Wd is [d][I], row-major ("out x in"). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

static void ffn_act(int64_t d, int64_t I, int dt, const void* x, int64_t xoff,
                    const void* wg, const void* wu, double* a, double* u, double* h) {
  for (int64_t i = 0; i < I; ++i) {
    double sa = 0.0, su = 0.0;
    for (int64_t k = 0; k < d; ++k) {
      double xv = ld(x, dt, xoff + k);
      sa += ld(wg, dt, i * d + k) * xv;
      su += ld(wu, dt, i * d + k) * xv;
    }
    a[i] = sa;
    u[i] = su;
    h[i] = silu(sa) * su;
  }
}

static void ffn_row(int64_t d, int64_t I, int dt, const void* x, int64_t xoff,
                    const void* wg, const void* wu, const void* wd, double* a,
                    double* u, double* h, double* y) {
  ffn_act(d, I, dt, x, xoff, wg, wu, a, u, h);
  for (int64_t n = 0; n < d; ++n) {
    double s = 0.0;
    for (int64_t i = 0; i < I; ++i) s += ld(wd, dt, n * I + i) * h[i];
    y[n] = s;
  }
}

/* O6, first half, for a list of picks: the expert's pre-activations and
 * hidden row a = Wg x_t, u = Wu x_t, h = silu(a) * u of pick q = (token
 * tok[q], FFN expert ex[q]), written to a, u, h [n][I].  wg/wu are
 * per-expert pointer tables of length N (an entry may be NULL when no pick
 * names that expert). */
int orc_ffn_act(int64_t T, int64_t d, int64_t N, int64_t I, int dt, const void* x,
                const void* const* wg, const void* const* wu, int64_t n,
                const int64_t* tok, const int32_t* ex, double* a, double* u, double* h) {
  if (!x || !wg || !wu || !tok || !ex || !a || !u || !h) return 1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t q = 0; q < n; ++q) {
    const int64_t t = tok[q];
    const int32_t e = ex[q];
    if (t < 0 || t >= T || e < 0 || e >= N || !wg[e] || !wu[e]) {
      bad = 1;
      continue;
    }
    ffn_act(d, I, dt, x, t * d, wg[e], wu[e], a + q * I, u + q * I, h + q * I);
  }
  return bad ? 1 : 0;
}

/* O6 + O7 -- layer output for the tokens toks[0..n_tok) (all tokens when
 * toks is NULL, n_tok = T):
 *   out_t = out_scale * ( (sum of gates on zero-computation picks) * x_t
 *                         + sum over FFN picks r ascending of g_r * FFN(x_t) )
 * which is sum_i g_i E_i(x_t) with E_i(x_t) = x_t for N < i <= N+Z.
 * wg/wu/wd are per-expert pointer tables of length N; an entry may be NULL
 * when no listed token picks that expert.  y_slot (nullable) receives the
 * unscaled expert output per slot, [n_tok][K][d], zero on identity slots. */
int orc_forward(int64_t T, int64_t d, int64_t N, int64_t I, int64_t K, int dt,
                double out_scale, const void* x, const void* const* wg,
                const void* const* wu, const void* const* wd,
                const int32_t* topk_idx, const double* gates, int64_t n_tok,
                const int64_t* toks, double* out, double* y_slot) {
  if (!x || !wg || !wu || !wd || !topk_idx || !gates || !out) return 1;
  if (!toks) n_tok = T;
  int bad = 0;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    double* u = (double*)malloc(sizeof(double) * (size_t)I);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_tok; ++q) {
      int64_t t = toks ? toks[q] : q;
      if (t < 0 || t >= T) { bad = 1; continue; }
      double* o = out + q * d;
      double c = 0.0;
      for (int64_t r = 0; r < K; ++r)
        if (topk_idx[t * K + r] >= N) c += gates[t * K + r];
      for (int64_t n = 0; n < d; ++n) o[n] = c * ld(x, dt, t * d + n);
      for (int64_t r = 0; r < K; ++r) {
        int64_t e = topk_idx[t * K + r];
        double* ys = y_slot ? y_slot + (q * K + r) * d : NULL;
        if (e >= N) {
          if (ys) memset(ys, 0, sizeof(double) * (size_t)d);
          continue;
        }
        if (!wg[e] || !wu[e] || !wd[e]) { bad = 1; continue; }
        ffn_row(d, I, dt, x, t * d, wg[e], wu[e], wd[e], a, u, h, y);
        for (int64_t n = 0; n < d; ++n) o[n] += gates[t * K + r] * y[n];
        if (ys) memcpy(ys, y, sizeof(double) * (size_t)d);
      }
      for (int64_t n = 0; n < d; ++n) o[n] *= out_scale;
    }
    free(a);
    free(u);
    free(h);
    free(y);
  }
  return bad ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* O9 -- backward of O1..O7 with the routing held fixed (the top-K set is
 * piecewise constant; the bias is decoupled from the objective, so it gets
 * no gradient).  Given dY for the tokens toks[0..n_tok):
 *   dYs = out_scale * dY_t
 *   real pick r, e = s_r:  dg_r = <dYs, y_r>;  dy = g_r dYs;
 *        dh = Wd^T dy;  da = dh*u*silu'(a);  du = dh*silu(a);
 *        dx += Wg^T da + Wu^T du;  dWd[e] += dy h^T;
 *        dWg[e] += da x^T;  dWu[e] += du x^T
 *   identity pick r:       dg_r = <dYs, x_t>;  dx += g_r dYs
 *   router, gate_norm = 1: dl_j = g_j (dg_j - sum_S g dg) on the picks, 0 off
 *          gate_norm = 0:  dl_j = p_j (dg~_j - sum_S p dg) for every j, with
 *                          dg~ the pick's dg or 0
 *        (p = softmax of the logits, from orc_exp and orc_sum64 as in O2)
 *   dWr += dl x_t^T;  dx += Wr^T dl
 * silu'(z) = s (1 + z (1 - s)), s = 1/(1+e^-z).
 * Weight gradients are accumulated (+=) over the listed tokens in ascending
 * list order; expert tables dwg/dwu/dwd may hold NULL for experts whose
 * gradient is not wanted; dwr may be NULL.  dx is [n_tok][d], overwritten.
 * gates must be the gates of the same gate_norm mode.
 * dl_extra (nullable, [T][E]) is a further gradient of the objective with
 * respect to the router scores (the load-balance loss's, from
 * orc_lb_loss); it is added to dl above before dWr and the dx term.
 * dx = NULL asks for the listed experts' weight gradients alone: then dwr
 * must be NULL, and only the FFN picks of experts with a gradient table
 * entry are differentiated (the other picks and the router contribute
 * nothing to those gradients). */
int orc_backward(int64_t T, int64_t d, int64_t N, int64_t Z, int64_t I,
                 int64_t K, int dt, int gate_norm, double out_scale,
                 const void* x, const void* wr, const void* const* wg,
                 const void* const* wu, const void* const* wd,
                 const double* logits, const int32_t* topk_idx,
                 const double* gates, const void* dY, int64_t n_tok,
                 const int64_t* toks, const double* dl_extra, double* dx,
                 double* dwr, double* const* dwg, double* const* dwu,
                 double* const* dwd) {
  const int64_t E = N + Z;
  if (!x || !wr || !wg || !wu || !wd || !logits || !topk_idx || !gates || !dY ||
      (!dx && dwr))
    return 1;
  const int experts_only = dx == NULL;
  if (!toks) n_tok = T;
  for (int64_t q = 0; q < n_tok; ++q) {
    int64_t t = toks ? toks[q] : q;
    if (t < 0 || t >= T) return 1;
    for (int64_t r = 0; r < K; ++r) {
      int64_t e = topk_idx[t * K + r];
      if (e < N && (!wg[e] || !wu[e] || !wd[e]) &&
          (!experts_only || dwg[e] || dwu[e] || dwd[e]))
        return 1;
    }
  }
  /* per-slot saved quantities, needed again for the weight gradients */
  const int64_t S = n_tok * K;
  double* A = (double*)calloc((size_t)(S * I), sizeof(double));
  double* U = (double*)calloc((size_t)(S * I), sizeof(double));
  double* H = (double*)calloc((size_t)(S * I), sizeof(double));
  double* DA = (double*)calloc((size_t)(S * I), sizeof(double));
  double* DU = (double*)calloc((size_t)(S * I), sizeof(double));
  double* DY = (double*)calloc((size_t)(S * d), sizeof(double));
  double* DL = (double*)calloc((size_t)(n_tok * E), sizeof(double));
  if (!A || !U || !H || !DA || !DU || !DY || !DL) {
    free(A); free(U); free(H); free(DA); free(DU); free(DY); free(DL);
    return 2;
  }
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    double* dys = (double*)malloc(sizeof(double) * (size_t)d);
    double* dh = (double*)malloc(sizeof(double) * (size_t)I);
    double* dg = (double*)malloc(sizeof(double) * (size_t)K);
    double* ex = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_tok; ++q) {
      int64_t t = toks ? toks[q] : q;
      double* dxo = experts_only ? NULL : dx + q * d;
      for (int64_t n = 0; n < d; ++n) {
        dys[n] = out_scale * ld(dY, dt, t * d + n);
        if (dxo) dxo[n] = 0.0;
      }
      for (int64_t r = 0; r < K; ++r) {
        int64_t e = topk_idx[t * K + r];
        double g = gates[t * K + r];
        int64_t sl = q * K + r;
        if (experts_only && (e >= N || (!dwg[e] && !dwu[e] && !dwd[e]))) continue;
        if (e >= N) {
          double s = 0.0;
          for (int64_t n = 0; n < d; ++n) s += dys[n] * ld(x, dt, t * d + n);
          dg[r] = s;
          for (int64_t n = 0; n < d; ++n) dxo[n] += g * dys[n];
          continue;
        }
        double *a = A + sl * I, *u = U + sl * I, *h = H + sl * I;
        ffn_row(d, I, dt, x, t * d, wg[e], wu[e], wd[e], a, u, h, y);
        double s = 0.0;
        for (int64_t n = 0; n < d; ++n) s += dys[n] * y[n];
        dg[r] = s;
        double* dyv = DY + sl * d;
        for (int64_t n = 0; n < d; ++n) dyv[n] = g * dys[n];
        for (int64_t i = 0; i < I; ++i) {
          double acc = 0.0;
          for (int64_t n = 0; n < d; ++n) acc += ld(wd[e], dt, n * I + i) * dyv[n];
          dh[i] = acc;
        }
        double *da = DA + sl * I, *du = DU + sl * I;
        for (int64_t i = 0; i < I; ++i) {
          double sg = 1.0 / (1.0 + exp(-a[i]));
          da[i] = dh[i] * u[i] * (sg * (1.0 + a[i] * (1.0 - sg)));
          du[i] = dh[i] * (a[i] * sg);
        }
        if (experts_only) continue;
        for (int64_t k = 0; k < d; ++k) {
          double acc = 0.0;
          for (int64_t i = 0; i < I; ++i)
            acc += ld(wg[e], dt, i * d + k) * da[i] + ld(wu[e], dt, i * d + k) * du[i];
          dxo[k] += acc;
        }
      }
      if (experts_only) continue;
      /* router: softmax Jacobian restricted as the gate mode dictates */
      double* dl = DL + q * E;
      if (gate_norm) {
        double sgd = 0.0;
        for (int64_t r = 0; r < K; ++r) sgd += gates[t * K + r] * dg[r];
        for (int64_t r = 0; r < K; ++r) {
          int64_t j = topk_idx[t * K + r];
          dl[j] = gates[t * K + r] * (dg[r] - sgd);
        }
      } else {
        const double* l = logits + t * E;
        double m = l[0];
        for (int64_t j = 1; j < E; ++j)
          if (l[j] > m) m = l[j];
        for (int64_t j = 0; j < E; ++j) ex[j] = orc_exp(l[j] - m);
        double Ssum = orc_sum64(ex, E);
        double spd = 0.0;
        for (int64_t r = 0; r < K; ++r) spd += gates[t * K + r] * dg[r];
        for (int64_t j = 0; j < E; ++j) dl[j] = -(ex[j] / Ssum) * spd;
        for (int64_t r = 0; r < K; ++r) {
          int64_t j = topk_idx[t * K + r];
          dl[j] += (ex[j] / Ssum) * dg[r];
        }
      }
      if (dl_extra)
        for (int64_t j = 0; j < E; ++j) dl[j] += dl_extra[t * E + j];
      for (int64_t k = 0; k < d; ++k) {
        double acc = 0.0;
        for (int64_t j = 0; j < E; ++j) acc += dl[j] * ld(wr, dt, j * d + k);
        dxo[k] += acc;
      }
    }
    free(y); free(dys); free(dh); free(dg); free(ex);
  }
  /* weight gradients: one expert (or router row) per thread, tokens in list
   * order, so every sum has a fixed order */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t e = 0; e < N; ++e) {
    if (!dwg[e] && !dwu[e] && !dwd[e]) continue;
    for (int64_t q = 0; q < n_tok; ++q) {
      int64_t t = toks ? toks[q] : q;
      for (int64_t r = 0; r < K; ++r) {
        if (topk_idx[t * K + r] != e) continue;
        int64_t sl = q * K + r;
        if (dwd[e])
          for (int64_t n = 0; n < d; ++n)
            for (int64_t i = 0; i < I; ++i) dwd[e][n * I + i] += DY[sl * d + n] * H[sl * I + i];
        for (int64_t i = 0; i < I; ++i)
          for (int64_t k = 0; k < d; ++k) {
            double xv = ld(x, dt, t * d + k);
            if (dwg[e]) dwg[e][i * d + k] += DA[sl * I + i] * xv;
            if (dwu[e]) dwu[e][i * d + k] += DU[sl * I + i] * xv;
          }
      }
    }
  }
  if (dwr) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < E; ++j)
      for (int64_t q = 0; q < n_tok; ++q) {
        int64_t t = toks ? toks[q] : q;
        double v = DL[q * E + j];
        if (v == 0.0) continue;
        for (int64_t k = 0; k < d; ++k) dwr[j * d + k] += v * ld(x, dt, t * d + k);
      }
  }
  free(A); free(U); free(H); free(DA); free(DU); free(DY); free(DL);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O8 -- Eq.(2), the per-step bias increment, for FFN experts i < N:
 *   b_i <- fp32( b_i + mu * ( K_e/(K*N) - T_i/(K*T_all) ) )
 * in binary64 with exactly these operations:
 *   tgt = K_e / ((double)K * N);  obs = (double)T_i / ((double)K * T_all);
 *   b_i = (float)((double)b_i + mu * (tgt - obs)).
 * Zero-computation experts (i >= N) keep their bias. */
int orc_pid_update(int64_t N, int64_t Z, int64_t K, const int32_t* counts,
                   int64_t T_all, double mu, double K_e, float* bias) {
  (void)Z;
  if (N < 0 || K < 1 || T_all < 1 || !counts || !bias) return 1;
  double tgt = K_e / ((double)K * (double)N);
  for (int64_t i = 0; i < N; ++i) {
    double obs = (double)counts[i] / ((double)K * (double)T_all);
    bias[i] = (float)((double)bias[i] + mu * (tgt - obs));
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O10 -- device-level load-balance loss of section 2.1.2 ("Load balance
 * control"): the L_LB formula there with P_j of Eq.(4) and f_j of Eq.(5):
 *   L = alpha * sum_{j=1}^{D+1} f_j P_j.
 * Groups: the N FFN experts split into D groups of G = N/D consecutive
 * indices (Group_j = experts (j-1)G .. jG-1, the experts one device holds
 * under expert parallelism); every zero-computation expert belongs to the
 * extra group D+1.
 *   P_j = (1/T) sum over i in Group_j, t of R_{t,i}, with R the unbiased
 *         softmax of the token's scores (orc_exp, orc_sum64 as in O2);
 *   f_j = D/(K_e T) * (picks of all tokens that fall in Group_j), j <= D;
 *   f_{D+1} = 1/((K-K_e) T) * (picks of zero-computation experts).
 * The indicator counts picks: a token with two picks in one group counts
 * twice, so that every f_j is 1 when the FFN picks spread evenly over the
 * groups and the layer takes K_e FFN experts per token on average.  With
 * Z = 0 the extra group is empty and its term is left out.
 * Gradient with respect to the scores (f is a count of discrete picks and
 * is held constant): with c_j = alpha f_{g(j)} / T for the group g(j) of j,
 *   dL/dl_{t,i} = R_{t,i} ( c_{g(i)} - sum_k R_{t,k} c_{g(k)} ).
 * out: [1 + 2(D+1)] = L, f_1..f_{D+1}, P_1..P_{D+1} (slots of the extra
 * group are 0 when Z = 0); dlogits: [T][E] or NULL.  T = 0 gives zeros.
 * Needs N >= 1, 1 <= D <= N, N % D == 0, 0 < K_e <= K, and K_e < K when
 * Z > 0. */
int orc_lb_loss(int64_t T, int64_t E, int64_t N, int64_t K, int64_t D,
                double K_e, double alpha, const double* logits,
                const int32_t* topk_idx, double* out, double* dlogits) {
  const int64_t Z = E - N;
  if (T < 0 || N < 1 || Z < 0 || K < 1 || K > E || D < 1 || D > N || N % D != 0 ||
      !(K_e > 0.0) || K_e > (double)K || (Z > 0 && !(K_e < (double)K)) || !out ||
      (T > 0 && (!logits || !topk_idx)))
    return 1;
  const int64_t G = N / D, ng = D + 1;
  for (int64_t j = 0; j < 1 + 2 * ng; ++j) out[j] = 0.0;
  if (T == 0) return 0;
  /* f from the picks */
  double* picks = (double*)calloc((size_t)ng, sizeof(double));
  for (int64_t i = 0; i < T * K; ++i) {
    int32_t e = topk_idx[i];
    if (e < 0 || e >= E) { free(picks); return 1; }
    picks[e < N ? e / G : D] += 1.0;
  }
  double* f = out + 1;
  double* P = out + 1 + ng;
  for (int64_t j = 0; j < D; ++j) f[j] = (double)D / (K_e * (double)T) * picks[j];
  if (Z > 0) f[D] = 1.0 / (((double)K - K_e) * (double)T) * picks[D];
  free(picks);
  /* R per token, then P_j as the group sum of the per-expert token sums */
  double* R = (double*)malloc(sizeof(double) * (size_t)(T * E));
#pragma omp parallel
  {
    double* e = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double* l = logits + t * E;
      double m = l[0];
      for (int64_t j = 1; j < E; ++j)
        if (l[j] > m) m = l[j];
      for (int64_t j = 0; j < E; ++j) e[j] = orc_exp(l[j] - m);
      double S = orc_sum64(e, E);
      for (int64_t j = 0; j < E; ++j) R[t * E + j] = e[j] / S;
    }
    free(e);
  }
  for (int64_t i = 0; i < E; ++i) {
    double col = 0.0;
    for (int64_t t = 0; t < T; ++t) col += R[t * E + i];
    P[i < N ? i / G : D] += col;
  }
  for (int64_t j = 0; j < ng; ++j) P[j] /= (double)T;
  double L = 0.0;
  for (int64_t j = 0; j < ng; ++j) L += f[j] * P[j];
  out[0] = alpha * L;
  if (dlogits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const double* r = R + t * E;
      double mean = 0.0;
      for (int64_t k = 0; k < E; ++k) mean += r[k] * (alpha * f[k < N ? k / G : D] / (double)T);
      for (int64_t i = 0; i < E; ++i) {
        double ci = alpha * f[i < N ? i / G : D] / (double)T;
        dlogits[t * E + i] = r[i] * (ci - mean);
      }
    }
  }
  free(R);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O11 -- budget-control telemetry of section 2.1.1 (the mean and the
 * standard deviation of the FFN experts each token activates, plotted in
 * Fig.3b/3c):
 *   n_t = number of the token's K picks that are FFN experts (index < N);
 *   hist[k] = number of tokens with n_t = k, k = 0..K;
 *   mean = (1/T) sum_t n_t;  std = sqrt((1/T) sum_t (n_t - mean)^2)
 * (the population deviation over the batch's tokens, t ascending).
 * T = 0 gives an all-zero histogram and mean = std = 0. */
int orc_route_stats(int64_t T, int64_t N, int64_t K, const int32_t* topk_idx,
                    int32_t* hist, double* mean, double* std) {
  if (T < 0 || N < 0 || K < 1 || !hist || !mean || !std || (T > 0 && !topk_idx)) return 1;
  for (int64_t k = 0; k <= K; ++k) hist[k] = 0;
  *mean = 0.0;
  *std = 0.0;
  if (T == 0) return 0;
  int32_t* n = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  for (int64_t t = 0; t < T; ++t) {
    int32_t c = 0;
    for (int64_t r = 0; r < K; ++r) c += topk_idx[t * K + r] < N ? 1 : 0;
    n[t] = c;
    hist[c] += 1;
  }
  double s = 0.0;
  for (int64_t t = 0; t < T; ++t) s += (double)n[t];
  double m = s / (double)T;
  double v = 0.0;
  for (int64_t t = 0; t < T; ++t) v += ((double)n[t] - m) * ((double)n[t] - m);
  *mean = m;
  *std = sqrt(v / (double)T);
  free(n);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O12 -- FP8 blockwise quantization of expert operands (the deployment path
 * of the LongCat pages quantizes blockwise to FP8 and keeps sensitive parts
 * in higher precision).  Block format: the OCP Microscaling (MX) format
 * MXFP8-E4M3, i.e. 32 consecutive values along the reduction dimension
 * share one power-of-two scale X = 2^(S-127) stored as an 8-bit exponent S
 * (E8M0), and each value is stored as an FP8 E4M3 code of v / X.
 *
 * E4M3 (OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 holds subnormals m/8 * 2^-6; the largest finite magnitude is 448
 * (field 1111, mantissa 110); 1111/111 is NaN; no infinities.
 *
 * Scale of a block: amax = max |v_i|; if amax = 0, S = 0; otherwise
 * S = floor(log2 amax) - 8 + 127 (8 = exponent of the largest E4M3 power of
 * two), clamped to 0..254.  Codes: v_i / X rounded to the nearest E4M3
 * value, ties to the even mantissa code, magnitudes above 448 saturated to
 * 448.  Dequantized value: decode(code) * X. */
double orc_e4m3_value(int code) {
  code &= 0xff;
  const double s = (code & 0x80) ? -1.0 : 1.0;
  const int e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) return s * ldexp((double)m, -9);          /* m/8 * 2^-6 */
  return s * ldexp((double)(8 + m), e - 10);             /* (1 + m/8) 2^(e-7) */
}

/* Nearest E4M3 code of a finite v (exact binary64 arithmetic: v times a
 * power of two is exact, rint rounds ties to even). */
int orc_e4m3_encode(double v) {
  const int neg = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return neg | 0x7e;
  int ex;
  frexp(a, &ex);                      /* a = f 2^ex, f in [0.5, 1) */
  int E = ex - 1;                     /* floor(log2 a) for a > 0 */
  if (a == 0.0 || E < -6) E = -6;     /* subnormal quantum 2^-9 */
  double q = rint(ldexp(a, 3 - E));   /* units of 2^(E-3) */
  if (q == 16.0) {                    /* rounded up into the next binade */
    q = 8.0;
    E += 1;
  }
  if (E > 8 || (E == 8 && q > 14.0)) return neg | 0x7e;
  if (q < 8.0) return neg | (int)q;   /* subnormal (E = -6) or zero */
  return neg | ((E + 7) << 3) | ((int)q - 8);
}

/* Quantize rows x cols values (dt: ORC_F32 / ORC_BF16 storage, or 2 for
 * binary64) in blocks of 32 along each row: codes [rows][cols], scales
 * [rows][cols/32] (E8M0, plain block order).  cols % 32 == 0. */
int orc_mx_quantize(int64_t rows, int64_t cols, int dt, const void* src, uint8_t* codes,
                    uint8_t* scales) {
  if (rows < 0 || cols <= 0 || cols % 32 || !src || !codes || !scales) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 32; ++b) {
      double v[32], amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const int64_t o = r * cols + b * 32 + i;
        v[i] = dt == 2 ? ((const double*)src)[o] : ld(src, dt, o);
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
      }
      int S = 0;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex);
        S = (ex - 1) - 8 + 127;
        if (S < 0) S = 0;
        if (S > 254) S = 254;
      }
      scales[r * (cols / 32) + b] = (uint8_t)S;
      for (int i = 0; i < 32; ++i)
        codes[r * cols + b * 32 + i] = (uint8_t)orc_e4m3_encode(ldexp(v[i], 127 - S));
    }
  }
  return 0;
}

/* Dequantized values decode(code) * 2^(S-127), binary64. */
int orc_mx_dequantize(int64_t rows, int64_t cols, const uint8_t* codes, const uint8_t* scales,
                      double* out) {
  if (rows < 0 || cols <= 0 || cols % 32 || !codes || !scales || !out) return 1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      out[r * cols + c] = ldexp(orc_e4m3_value(codes[r * cols + c]),
                                (int)scales[r * (cols / 32) + c / 32] - 127);
  return 0;
}

/* O13 -- the layer forward with MXFP8 expert operands (O12):
 *   x'  = MX(x_t) along d (per token);  W' = MX(W) along each weight's
 *         reduction dimension (given as codes + scales per expert, the
 *         output of orc_mx_quantize on [I][d] or [d][I]);
 *   a = W'_g x',  u = W'_u x',  h = silu(a) * u  (binary64);
 *   h' = MX(h) along I;  y = W'_d h';
 *   out_t = out_scale * ( c_t x_t + sum over FFN picks of g_r y_r ), with
 *         the zero-computation term on the unquantized x_t.
 * Weight tables: per expert e, codes (wgc/wuc [I][d], wdc [d][I]) and
 * scales (wgs/wus [I][d/32], wds [d][I/32]); NULL for experts no listed
 * token picks.  y_out (nullable) receives y per listed (token, slot)
 * [n_tok*K][d] (0 for identity picks). */
static int mx_tables_ok(int64_t T, int64_t N, int64_t K, const uint8_t* const* wgc,
                        const uint8_t* const* wgs, const uint8_t* const* wuc,
                        const uint8_t* const* wus, const uint8_t* const* wdc,
                        const uint8_t* const* wds, const int32_t* topk_idx, int64_t n_tok,
                        const int64_t* toks) {
  for (int64_t q = 0; q < n_tok; ++q) {
    const int64_t t = toks ? toks[q] : q;
    if (t < 0 || t >= T) return 0;
    for (int64_t r = 0; r < K; ++r) {
      const int64_t e = topk_idx[t * K + r];
      if (e < N && (!wgc[e] || !wgs[e] || !wuc[e] || !wus[e] || !wdc[e] || !wds[e])) return 0;
    }
  }
  return 1;
}

/* Row n of an MXFP8 matrix [R][C] (codes + scales), dequantized:
 * decode(code) * 2^(S-127).  pow2[S] = 2^(S-127) (exact), so each product is
 * exact too: E4M3 values times 2^-127 .. 2^127 stay normal binary64. */
static double mx_pow2[256];
static void mx_row(const double* val, const uint8_t* codes, const uint8_t* scales, int64_t n,
                   int64_t C, double* row) {
  for (int64_t k = 0; k < C; ++k)
    row[k] = val[codes[n * C + k]] * mx_pow2[scales[(n * C + k) / 32]];
}
static void mx_tables(double* val) {
  for (int c = 0; c < 256; ++c) {
    val[c] = orc_e4m3_value(c);
    mx_pow2[c] = ldexp(1.0, c - 127);
  }
}

int orc_forward_mx(int64_t T, int64_t d, int64_t N, int64_t I, int64_t K, int dt,
                   double out_scale, const void* x, const uint8_t* const* wgc,
                   const uint8_t* const* wgs, const uint8_t* const* wuc,
                   const uint8_t* const* wus, const uint8_t* const* wdc,
                   const uint8_t* const* wds, const int32_t* topk_idx, const double* gates,
                   int64_t n_tok, const int64_t* toks, double* out, double* y_out) {
  if (T < 0 || d <= 0 || d % 32 || I <= 0 || I % 32 || K < 1 || !x || !wgc || !wgs || !wuc ||
      !wus || !wdc || !wds || !topk_idx || !gates || !out)
    return 1;
  if (!toks) n_tok = T;
  if (!mx_tables_ok(T, N, K, wgc, wgs, wuc, wus, wdc, wds, topk_idx, n_tok, toks)) return 1;
  double val[256];
  mx_tables(val);
  const int64_t wmax = d > I ? d : I;
#pragma omp parallel
  {
    double* xq = (double*)malloc(sizeof(double) * (size_t)d);
    uint8_t* qc = (uint8_t*)malloc((size_t)wmax);
    uint8_t* qs = (uint8_t*)malloc((size_t)wmax / 32);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* hq = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    double* wrow = (double*)malloc(sizeof(double) * (size_t)wmax);
    double* urow = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_tok; ++q) {
      const int64_t t = toks ? toks[q] : q;
      orc_mx_quantize(1, d, dt, dt == ORC_BF16 ? (const void*)((const uint16_t*)x + t * d)
                                              : (const void*)((const float*)x + t * d),
                      qc, qs);
      orc_mx_dequantize(1, d, qc, qs, xq);
      double* o = out + q * d;
      double c = 0.0;
      for (int64_t n = 0; n < d; ++n) o[n] = 0.0;
      for (int64_t r = 0; r < K; ++r) {
        const int64_t e = topk_idx[t * K + r];
        const double g = gates[t * K + r];
        double* yo = y_out ? y_out + (q * K + r) * d : NULL;
        if (e >= N) {
          c += g;
          if (yo)
            for (int64_t n = 0; n < d; ++n) yo[n] = 0.0;
          continue;
        }
        for (int64_t i = 0; i < I; ++i) {
          mx_row(val, wgc[e], wgs[e], i, d, wrow);
          mx_row(val, wuc[e], wus[e], i, d, urow);
          double a = 0.0, u = 0.0;
          for (int64_t k = 0; k < d; ++k) {
            a += wrow[k] * xq[k];
            u += urow[k] * xq[k];
          }
          h[i] = silu(a) * u;
        }
        orc_mx_quantize(1, I, 2, h, qc, qs);
        orc_mx_dequantize(1, I, qc, qs, hq);
        for (int64_t n = 0; n < d; ++n) {
          mx_row(val, wdc[e], wds[e], n, I, wrow);
          double acc = 0.0;
          for (int64_t i = 0; i < I; ++i) acc += wrow[i] * hq[i];
          y[n] = acc;
          if (yo) yo[n] = acc;
        }
        for (int64_t n = 0; n < d; ++n) o[n] += g * y[n];
      }
      for (int64_t n = 0; n < d; ++n) o[n] = out_scale * (c * ld(x, dt, t * d + n) + o[n]);
    }
    free(xq); free(qc); free(qs); free(h); free(hq); free(y); free(wrow); free(urow);
  }
  return 0;
}

/* TOLERANCE HELPER for comparisons against O13 -- not part of the layer.
 * h' is a quantization decision taken on a computed value (h), and any
 * implementation that sums the dot products a, u in fp32 (and evaluates silu
 * and the product in fp32) holds an h that differs from the binary64 h of
 * O13 in its last bits.  With a and u known to within eps times the sum of
 * their absolute products (Sa, Su), h_i is known to within
 *   tol_i = eps (|silu'(a) u| Sa + |silu(a)| Su) + 2^-21 |h_i|,
 * so an h_i within tol_i of a rounding boundary of its code (or a block
 * whose amax is that close to a power of two, which moves its scale) may
 * legitimately come out one code apart.  flip [n_tok][d] receives, per
 * output element, the largest change such code changes can cause:
 *   out_scale * sum over FFN picks of |g| * sum over the affected i of
 *   |W'_d[n][i]| * (largest distance between the dequantized candidates).
 * Same arguments as orc_forward_mx. */
static void mx_candidates(const double* h, const double* tol, int64_t I, const uint8_t* qs,
                          const double* hq, double* delta);
int orc_mx_flip_bound(int64_t T, int64_t d, int64_t N, int64_t I, int64_t K, int dt,
                      double out_scale, const void* x, const uint8_t* const* wgc,
                      const uint8_t* const* wgs, const uint8_t* const* wuc,
                      const uint8_t* const* wus, const uint8_t* const* wdc,
                      const uint8_t* const* wds, const int32_t* topk_idx, const double* gates,
                      int64_t n_tok, const int64_t* toks, double eps, double* flip) {
  if (T < 0 || d <= 0 || d % 32 || I <= 0 || I % 32 || K < 1 || !x || !wgc || !wgs || !wuc ||
      !wus || !wdc || !wds || !topk_idx || !gates || !flip || !(eps >= 0.0))
    return 1;
  if (!toks) n_tok = T;
  if (!mx_tables_ok(T, N, K, wgc, wgs, wuc, wus, wdc, wds, topk_idx, n_tok, toks)) return 1;
  double val[256];
  mx_tables(val);
  const int64_t wmax = d > I ? d : I;
#pragma omp parallel
  {
    double* xq = (double*)malloc(sizeof(double) * (size_t)d);
    uint8_t* qc = (uint8_t*)malloc((size_t)wmax);
    uint8_t* qs = (uint8_t*)malloc((size_t)wmax / 32);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* hq = (double*)malloc(sizeof(double) * (size_t)I);
    double* wrow = (double*)malloc(sizeof(double) * (size_t)wmax);
    double* urow = (double*)malloc(sizeof(double) * (size_t)d);
    double* dlt = (double*)malloc(sizeof(double) * (size_t)I);
    double* tl = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_tok; ++q) {
      const int64_t t = toks ? toks[q] : q;
      orc_mx_quantize(1, d, dt, dt == ORC_BF16 ? (const void*)((const uint16_t*)x + t * d)
                                              : (const void*)((const float*)x + t * d),
                      qc, qs);
      orc_mx_dequantize(1, d, qc, qs, xq);
      double* fo = flip + q * d;
      for (int64_t n = 0; n < d; ++n) fo[n] = 0.0;
      for (int64_t r = 0; r < K; ++r) {
        const int64_t e = topk_idx[t * K + r];
        const double g = gates[t * K + r];
        if (e >= N) continue;
        for (int64_t i = 0; i < I; ++i) {
          mx_row(val, wgc[e], wgs[e], i, d, wrow);
          mx_row(val, wuc[e], wus[e], i, d, urow);
          double a = 0.0, u = 0.0, sa = 0.0, su = 0.0;
          for (int64_t k = 0; k < d; ++k) {
            a += wrow[k] * xq[k];
            u += urow[k] * xq[k];
            sa += fabs(wrow[k] * xq[k]);
            su += fabs(urow[k] * xq[k]);
          }
          h[i] = silu(a) * u;
          const double sg = 1.0 / (1.0 + exp(-a));
          tl[i] = eps * (fabs(sg * (1.0 + a * (1.0 - sg)) * u) * sa + fabs(a * sg) * su) +
                  ldexp(fabs(h[i]), -21);
        }
        orc_mx_quantize(1, I, 2, h, qc, qs);
        orc_mx_dequantize(1, I, qc, qs, hq);
        mx_candidates(h, tl, I, qs, hq, dlt);
        for (int64_t n = 0; n < d; ++n) {
          mx_row(val, wdc[e], wds[e], n, I, wrow);
          double fl = 0.0;
          for (int64_t i = 0; i < I; ++i)
            if (dlt[i] > 0.0) fl += fabs(wrow[i]) * dlt[i];
          fo[n] += fabs(out_scale * g) * fl;
        }
      }
    }
    free(xq); free(qc); free(qs); free(h); free(hq); free(wrow); free(urow); free(dlt); free(tl);
  }
  return 0;
}

/* For each h_i: 0 when its code and scale are the same for every value in
 * [h_i - tol_i, h_i + tol_i] (and for the block's amax moved the same way);
 * otherwise the largest distance between hq_i and the dequantized value of
 * any of those alternatives. */
static void mx_candidates(const double* h, const double* tol, int64_t I, const uint8_t* qs,
                          const double* hq, double* delta) {
  for (int64_t b = 0; b < I / 32; ++b) {
    double lo = 0.0, hi = 0.0;  /* range of the block's amax */
    for (int i = 0; i < 32; ++i) {
      const double m = fabs(h[b * 32 + i]), t = tol[b * 32 + i];
      if (m + t > hi) hi = m + t;
      if (m - t > lo) lo = m - t;
    }
    int Ss[3], ns = 0;
    Ss[ns++] = qs[b];
    const double ends[2] = {lo, hi};
    for (int w = 0; w < 2; ++w) {
      int S = 0;
      if (ends[w] > 0.0) {
        int ex;
        frexp(ends[w], &ex);
        S = (ex - 1) - 8 + 127;
        if (S < 0) S = 0;
        if (S > 254) S = 254;
      }
      int dup = 0;
      for (int q = 0; q < ns; ++q) dup |= Ss[q] == S;
      if (!dup) Ss[ns++] = S;
    }
    for (int i = 0; i < 32; ++i) {
      const int64_t k = b * 32 + i;
      double dm = 0.0;
      for (int si = 0; si < ns; ++si)
        for (int sgn = -1; sgn <= 1; ++sgn) {
          const double v = h[k] + sgn * tol[k];
          const int code = orc_e4m3_encode(ldexp(v, 127 - Ss[si]));
          const double dv = ldexp(orc_e4m3_value(code), Ss[si] - 127);
          if (fabs(dv - hq[k]) > dm) dm = fabs(dv - hq[k]);
        }
      delta[k] = dm;
    }
  }
}

/* Host sanitizer run of the fp64 oracle (test infrastructure): calls every
 * oracle entry point on small seeded inputs, including the edge cases the
 * GPU tests use (no tokens, no FFN experts, K = E, non-finite scores), so
 * that AddressSanitizer and UndefinedBehaviorSanitizer see each loop and
 * index computation once.  Exit status 0 when every call returns its
 * documented status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_exp(double z);
int orc_logits(int64_t T, int64_t d, int64_t E, int dt, const void* x, const void* wr,
               double* logits);
int orc_route(int64_t T, int64_t E, int64_t N, int64_t K, int gate_norm, const double* logits,
              const float* bias, double* keys_out, int32_t* topk_idx, double* gates,
              int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv);
int orc_forward(int64_t T, int64_t d, int64_t N, int64_t I, int64_t K, int dt, double out_scale,
                const void* x, const void* const* wg, const void* const* wu, const void* const* wd,
                const int32_t* topk_idx, const double* gates, int64_t n_tok, const int64_t* toks,
                double* out, double* y_slot);
int orc_backward(int64_t T, int64_t d, int64_t N, int64_t Z, int64_t I, int64_t K, int dt,
                 int gate_norm, double out_scale, const void* x, const void* wr,
                 const void* const* wg, const void* const* wu, const void* const* wd,
                 const double* logits, const int32_t* topk_idx, const double* gates,
                 const void* dY, int64_t n_tok, const int64_t* toks, const double* dl_extra,
                 double* dx, double* dwr, double* const* dwg, double* const* dwu,
                 double* const* dwd);
int orc_pid_update(int64_t N, int64_t Z, int64_t K, const int32_t* counts, int64_t T_all,
                   double mu, double K_e, float* bias);
int orc_lb_loss(int64_t T, int64_t E, int64_t N, int64_t K, int64_t D, double K_e, double alpha,
                const double* logits, const int32_t* topk_idx, double* out, double* dlogits);
int orc_route_stats(int64_t T, int64_t N, int64_t K, const int32_t* topk_idx, int32_t* hist,
                    double* mean, double* std);
int orc_mx_quantize(int64_t rows, int64_t cols, int dt, const void* src, uint8_t* codes,
                    uint8_t* scales);
int orc_mx_dequantize(int64_t rows, int64_t cols, const uint8_t* codes, const uint8_t* scales,
                      double* out);
int orc_forward_mx(int64_t T, int64_t d, int64_t N, int64_t I, int64_t K, int dt,
                   double out_scale, const void* x, const uint8_t* const* wgc,
                   const uint8_t* const* wgs, const uint8_t* const* wuc,
                   const uint8_t* const* wus, const uint8_t* const* wdc,
                   const uint8_t* const* wds, const int32_t* topk_idx, const double* gates,
                   int64_t n_tok, const int64_t* toks, double* out, double* y_out);
int orc_mx_flip_bound(int64_t T, int64_t d, int64_t N, int64_t I, int64_t K, int dt,
                      double out_scale, const void* x, const uint8_t* const* wgc,
                      const uint8_t* const* wgs, const uint8_t* const* wuc,
                      const uint8_t* const* wus, const uint8_t* const* wdc,
                      const uint8_t* const* wds, const int32_t* topk_idx, const double* gates,
                      int64_t n_tok, const int64_t* toks, double eps, double* flip);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static float* farr(int64_t n, double s) {
  float* a = malloc(sizeof(float) * (size_t)(n ? n : 1));
  for (int64_t i = 0; i < n; ++i) a[i] = (float)(s * urand());
  return a;
}
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } \
  } while (0)

static int layer(int64_t T, int64_t d, int64_t N, int64_t Z, int64_t I, int64_t K, int gate_norm,
                 int nonfinite) {
  const int64_t E = N + Z;
  float* x = farr(T * d, 1.0);
  float* wr = farr(E * d, 0.1);
  float* bias = farr(E, 0.05);
  float* dY = farr(T * d, 1.0);
  float* wg = farr(N * I * d, 0.1);
  float* wu = farr(N * I * d, 0.1);
  float* wd = farr(N * d * I, 0.1);
  const void** tg = malloc(sizeof(void*) * (size_t)(N ? N : 1));
  const void** tu = malloc(sizeof(void*) * (size_t)(N ? N : 1));
  const void** td = malloc(sizeof(void*) * (size_t)(N ? N : 1));
  double** gg = malloc(sizeof(double*) * (size_t)(N ? N : 1));
  double** gu = malloc(sizeof(double*) * (size_t)(N ? N : 1));
  double** gd = malloc(sizeof(double*) * (size_t)(N ? N : 1));
  for (int64_t e = 0; e < N; ++e) {
    tg[e] = wg + e * I * d; tu[e] = wu + e * I * d; td[e] = wd + e * d * I;
    gg[e] = calloc((size_t)(I * d), sizeof(double));
    gu[e] = calloc((size_t)(I * d), sizeof(double));
    gd[e] = calloc((size_t)(d * I), sizeof(double));
  }
  double* lg = malloc(sizeof(double) * (size_t)(T * E + 1));
  CHECK(orc_logits(T, d, E, 0, x, wr, lg) == 0);
  if (nonfinite && T > 2) { lg[0] = NAN; lg[E + 1] = INFINITY; for (int64_t j = 0; j < E; ++j) lg[2 * E + j] = -INFINITY; }
  double* keys = malloc(sizeof(double) * (size_t)(T * E + 1));
  int32_t* idx = malloc(sizeof(int32_t) * (size_t)(T * K + 1));
  double* gates = malloc(sizeof(double) * (size_t)(T * K + 1));
  int32_t* counts = malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = malloc(sizeof(int32_t) * (size_t)(N + 1));
  int32_t* perm = malloc(sizeof(int32_t) * (size_t)(T * K + 1));
  int32_t* inv = malloc(sizeof(int32_t) * (size_t)(T * K + 1));
  CHECK(orc_route(T, E, N, K, gate_norm, lg, bias, keys, idx, gates, counts, offsets, perm, inv) == 0);
  for (int64_t i = 0; i < T * K; ++i) CHECK(idx[i] >= 0 && idx[i] < E);
  double* out = malloc(sizeof(double) * (size_t)(T * d + 1));
  double* ys = malloc(sizeof(double) * (size_t)(T * K * d + 1));
  double* dx = malloc(sizeof(double) * (size_t)(T * d + 1));
  double* dwr = calloc((size_t)(E * d), sizeof(double));
  int32_t* hist = calloc((size_t)(K + 1), sizeof(int32_t));
  if (nonfinite) goto done;  /* NaN rows only check the routing */
  CHECK(orc_forward(T, d, N, I, K, 0, 1.0, x, tg, tu, td, idx, gates, 0, NULL, out, ys) == 0);
  CHECK(orc_backward(T, d, N, Z, I, K, 0, gate_norm, 0.5, x, wr, tg, tu, td, lg, idx, gates, dY,
                     0, NULL, NULL, dx, dwr, gg, gu, gd) == 0);
  CHECK(orc_backward(T, d, N, Z, I, K, 0, gate_norm, 0.5, x, wr, tg, tu, td, lg, idx, gates, dY,
                     0, NULL, NULL, NULL, NULL, gg, gu, gd) == 0);
  CHECK(orc_pid_update(N, Z, K, counts, T > 0 ? T : 1, 1.0, (double)K / 2.0, bias) == 0);
  if (N >= 2 && N % 2 == 0 && Z > 0 && K > 1) {
    double lb[1 + 2 * 3];
    double* dl = malloc(sizeof(double) * (size_t)(T * E + 1));
    CHECK(orc_lb_loss(T, E, N, K, 2, (double)K / 2.0, 1e-2, lg, idx, lb, dl) == 0);
    free(dl);
  }
  double mean, sd;
  CHECK(orc_route_stats(T, N, K, idx, hist, &mean, &sd) == 0);
  if (d % 32 == 0 && I % 32 == 0 && N > 0) {
    uint8_t **gc = malloc(sizeof(void*) * N), **gs = malloc(sizeof(void*) * N),
            **uc = malloc(sizeof(void*) * N), **us = malloc(sizeof(void*) * N),
            **dc = malloc(sizeof(void*) * N), **ds = malloc(sizeof(void*) * N);
    for (int64_t e = 0; e < N; ++e) {
      gc[e] = malloc((size_t)(I * d)); gs[e] = malloc((size_t)(I * d / 32));
      uc[e] = malloc((size_t)(I * d)); us[e] = malloc((size_t)(I * d / 32));
      dc[e] = malloc((size_t)(d * I)); ds[e] = malloc((size_t)(d * I / 32));
      CHECK(orc_mx_quantize(I, d, 0, tg[e], gc[e], gs[e]) == 0);
      CHECK(orc_mx_quantize(I, d, 0, tu[e], uc[e], us[e]) == 0);
      CHECK(orc_mx_quantize(d, I, 0, td[e], dc[e], ds[e]) == 0);
    }
    double* deq = malloc(sizeof(double) * (size_t)(I * d));
    CHECK(orc_mx_dequantize(I, d, gc[0], gs[0], deq) == 0);
    double* fl = malloc(sizeof(double) * (size_t)(T * d + 1));
    CHECK(orc_forward_mx(T, d, N, I, K, 0, 1.0, x, (const uint8_t* const*)gc,
                         (const uint8_t* const*)gs, (const uint8_t* const*)uc,
                         (const uint8_t* const*)us, (const uint8_t* const*)dc,
                         (const uint8_t* const*)ds, idx, gates, 0, NULL, out, ys) == 0);
    CHECK(orc_mx_flip_bound(T, d, N, I, K, 0, 1.0, x, (const uint8_t* const*)gc,
                            (const uint8_t* const*)gs, (const uint8_t* const*)uc,
                            (const uint8_t* const*)us, (const uint8_t* const*)dc,
                            (const uint8_t* const*)ds, idx, gates, 0, NULL, 1e-6, fl) == 0);
    for (int64_t e = 0; e < N; ++e) {
      free(gc[e]); free(gs[e]); free(uc[e]); free(us[e]); free(dc[e]); free(ds[e]);
    }
    free(gc); free(gs); free(uc); free(us); free(dc); free(ds); free(deq); free(fl);
  }
done:
  for (int64_t e = 0; e < N; ++e) { free(gg[e]); free(gu[e]); free(gd[e]); }
  free(x); free(wr); free(bias); free(dY); free(wg); free(wu); free(wd);
  free(tg); free(tu); free(td); free(gg); free(gu); free(gd); free(lg); free(keys); free(idx);
  free(gates); free(counts); free(offsets); free(perm); free(inv); free(out); free(ys);
  free(dx); free(dwr); free(hist);
  return 0;
}

int main(void) {
  CHECK(orc_exp(-1.0) > 0.36 && orc_exp(-800.0) == 0.0 && isnan(orc_exp(NAN)));
  /* T, d, N, Z, I, K, gate_norm, non-finite scores */
  CHECK(layer(12, 64, 4, 2, 32, 3, 1, 0) == 0);
  CHECK(layer(9, 64, 3, 3, 64, 6, 0, 0) == 0);      /* K = E */
  CHECK(layer(0, 32, 2, 2, 32, 2, 1, 0) == 0);      /* no tokens */
  CHECK(layer(7, 32, 0, 5, 32, 2, 1, 0) == 0);      /* no FFN experts */
  CHECK(layer(6, 32, 4, 0, 32, 1, 0, 0) == 0);      /* no zero-computation experts */
  CHECK(layer(5, 32, 4, 2, 32, 3, 1, 1) == 0);      /* NaN / inf scores */
  puts("oracle sanitizer run ok");
  return 0;
}

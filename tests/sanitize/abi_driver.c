/* Host sanitizer run of the C ABI's host code (test infrastructure): every
 * entry point is called with arguments its host-side checks reject -- NULL
 * and misaligned pointers, bad sizes and enums, short workspaces, oversized
 * allocation-free layers -- so argument validation, workspace sizing and
 * the error paths run under AddressSanitizer and UndefinedBehaviorSanitizer
 * without queuing any GPU work.  Exit status 0 when every call returns the
 * documented status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/zc_moe.h"

#define CHECK(c)                                                                \
  do {                                                                          \
    if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } \
  } while (0)

static zc_moe_desc desc(int64_t T, int64_t d, int64_t N, int64_t Z, int64_t I, int64_t K,
                        int dtype) {
  zc_moe_desc x;
  memset(&x, 0, sizeof x);
  x.T = T; x.d = d; x.N = N; x.Z = Z; x.I = I; x.K = K; x.dtype = dtype;
  x.gate_norm = 1; x.out_scale = 1.0f; x.weight_layout = ZC_WEIGHTS_ROWMAJOR; x.cu_limit = 0;
  return x;
}

int main(void) {
  void* F = (void*)(uintptr_t)(1u << 20);   /* never dereferenced */
  void* M = (void*)(uintptr_t)((1u << 20) + 4);
  zc_route_buf r = {(float*)F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                    (int32_t*)F};
  zc_moe_desc ok = desc(64, 128, 8, 4, 64, 2, ZC_F32);
  /* sizes: valid layers of every kind, and invalid ones (0) */
  const int64_t shapes[][7] = {{64, 128, 8, 4, 64, 2, ZC_F32}, {4096, 1024, 64, 32, 512, 6, ZC_BF16},
                               {256, 6144, 512, 256, 2048, 12, ZC_BF16}, {0, 64, 1, 1, 64, 1, ZC_BF16},
                               {5, 64, 0, 9, 64, 4, ZC_BF16}, {300, 64, 1024, 0, 64, 32, ZC_BF16}};
  for (unsigned i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    zc_moe_desc x = desc(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4],
                         shapes[i][5], (int)shapes[i][6]);
    for (int op = 0; op <= 4; ++op) (void)zc_moe_workspace_size(&x, op);
    CHECK(zc_moe_workspace_size(&x, ZC_OP_FORWARD) > 0 || x.T == 0);
    (void)zc_moe_saved_size(&x);
    for (int lay = 0; lay <= 2; ++lay) {
      x.weight_layout = lay;
      (void)zc_moe_workspace_size(&x, ZC_OP_FORWARD);
      (void)zc_moe_quantized_weight_bytes(&x);
    }
  }
  zc_moe_desc bad[10];
  for (int i = 0; i < 10; ++i) bad[i] = ok;
  bad[0].K = 0; bad[1].K = 13; bad[2].N = 0; bad[2].Z = 0; bad[3].N = 1000; bad[3].Z = 100;
  bad[4].T = -1; bad[5].d = 100; bad[6].gate_norm = 2; bad[7].out_scale = NAN;
  bad[8].cu_limit = 12; bad[9].weight_layout = 7;
  for (int i = 0; i < 10; ++i) {
    CHECK(zc_moe_workspace_size(&bad[i], ZC_OP_FORWARD) == 0);
    CHECK(zc_moe_route(&bad[i], F, F, (float*)F, &r, F, 1 << 30, NULL) != ZC_OK);
    CHECK(strlen(zc_last_error()) > 0);
  }
  /* pointers, alignment, workspace */
  CHECK(zc_moe_route(NULL, F, F, (float*)F, &r, F, 1 << 30, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_route(&ok, F, F, NULL, &r, F, 1 << 30, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_route(&ok, M, F, (float*)F, &r, F, 1 << 30, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_route(&ok, F, F, (float*)F, &r, F, 16, NULL) == ZC_ERR_WORKSPACE);
  CHECK(zc_moe_route(&ok, F, F, (float*)F, NULL, F, 1 << 30, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_forward(&ok, F, F, (float*)F, F, F, F, F, &r, NULL, F, 16, NULL) ==
        ZC_ERR_WORKSPACE);
  CHECK(zc_moe_forward(&ok, F, F, (float*)F, NULL, F, F, F, &r, NULL, F, 1 << 30, NULL) ==
        ZC_ERR_INVALID);
  zc_moe_desc packed = desc(64, 256, 8, 4, 256, 2, ZC_BF16);
  packed.weight_layout = ZC_WEIGHTS_PACKED;
  CHECK(zc_moe_forward(&packed, F, F, (float*)F, F, F, F, F, &r, F, F, 1 << 30, NULL) ==
        ZC_ERR_UNSUPPORTED);
  CHECK(zc_moe_backward(&packed, F, F, F, F, F, &r, F, F, F, F, F, F, F, NULL, F, 1 << 30,
                        NULL) == ZC_ERR_UNSUPPORTED);
  CHECK(zc_moe_backward(&ok, F, F, F, F, F, &r, F, F, F, F, F, F, F, NULL, F, 16, NULL) ==
        ZC_ERR_WORKSPACE);
  zc_lb_cfg lb = {3, 1.0, 0.1};  /* 3 does not divide N = 8 */
  CHECK(zc_moe_backward(&ok, F, F, F, F, F, &r, F, F, F, F, F, F, F, &lb, F, 1 << 30, NULL) ==
        ZC_ERR_INVALID);
  CHECK(zc_moe_lb_loss(&ok, &lb, &r, (double*)F, F, 1 << 30, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_route_stats(&ok, &r, NULL, (double*)F, F, 1 << 30, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_accumulate_counts(0, (int32_t*)F, (int32_t*)F, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_accumulate_counts(8, (int32_t*)F, (int32_t*)F, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_pid_update(8, 4, 2, (int32_t*)F, 0, 1.0, 1.0, (float*)F, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_pid_update(8, 4, 2, (int32_t*)F, 64, NAN, 1.0, (float*)F, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_pack_weights(&ok, ZC_PACK_GATE_UP, F, F, NULL) == ZC_ERR_UNSUPPORTED);
  CHECK(zc_moe_pack_weights(&packed, 5, F, F, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_pack_weights(&packed, ZC_PACK_DOWN, F, F, NULL) == ZC_ERR_INVALID);  /* overlap */
  CHECK(zc_moe_quantize_weights(&ok, ZC_PACK_GATE_UP, F, F, NULL) == ZC_ERR_UNSUPPORTED);
  zc_moe_desc big = desc(4096, 1024, 64, 32, 512, 6, ZC_BF16);
  CHECK(zc_moe_forward_noalloc(&big, F, F, (float*)F, F, F, F, F, &r, NULL) == ZC_ERR_WORKSPACE);
  CHECK(zc_moe_forward_noalloc(&bad[0], F, F, (float*)F, F, F, F, F, &r, NULL) == ZC_ERR_INVALID);
  /* helpers */
  for (int s = -1; s <= 5; ++s) CHECK(zc_status_string((zc_status)s) != NULL);
  for (int p = -1; p <= ZC_NUM_PHASES; ++p) CHECK(zc_moe_phase_name(p) != NULL);
  CHECK(zc_moe_profile_read(NULL, NULL) == ZC_ERR_INVALID);
  CHECK(zc_moe_profile(0) == ZC_OK);
  puts("host API sanitizer run ok");
  return 0;
}

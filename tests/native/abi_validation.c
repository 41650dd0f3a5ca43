/* Host-side argument validation of the C ABI (include/qlora.h), built with the address and
 * undefined-behaviour sanitizers on the host side only.  Every call below is refused, or answered
 * by a size helper, before anything reaches the GPU: no device memory is touched, so the buffers
 * are fake, 16-byte aligned addresses that are never dereferenced.  Exit status 0 when every call
 * returns the documented result; a sanitizer report aborts the program. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qlora.h"

static int failures = 0;

#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    long long got_ = (long long)(call);                                                     \
    if (got_ != (long long)(want)) {                                                        \
      fprintf(stderr, "line %d: %s returned %lld, expected %lld\n", __LINE__, #call, got_,  \
              (long long)(want));                                                           \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

int main(void) {
  void *const P = (void *)(uintptr_t)0x10000; /* aligned, never dereferenced */
  void *const MIS = (void *)(uintptr_t)0x10002;
  const uint16_t *const X = (const uint16_t *)P;
  uint16_t *const Y = (uint16_t *)P;
  float *const F = (float *)P;
  const int64_t BIG = (int64_t)1 << 37, HUGE = (int64_t)1 << 62;
  qlora_nf4_weight q = {4096, 4096, (uint8_t *)P, (uint8_t *)P, (float *)P, (float *)P, 0};
  qlora_nf4_weight bad_q = q;

  /* size helpers: huge, negative and overflowing shapes give 0, never wrap */
  EXPECT(qlora_nf4_bytes(4096, 4096), 4096 * 4096 / 2 + 4096 * 4096 / 64 + 4 * 1024 + 4);
  EXPECT(qlora_nf4_bytes(BIG, BIG), 0);
  EXPECT(qlora_nf4_bytes(HUGE, 2), 0);
  EXPECT(qlora_nf4_bytes(-1, 64), 0);
  EXPECT(qlora_nf4_bytes_flags(64, 64, 7u), 0);
  EXPECT(qlora_quantize_workspace_bytes(BIG, BIG), 0);
  EXPECT(qlora_linear_workspace_bytes(BIG, 4096, 4096, 64), 0);
  EXPECT(qlora_linear_workspace_bytes(HUGE, 64, 64, 8), 0);
  EXPECT(qlora_linear_workspace_bytes(16, 4096, 100, 8), 0);
  EXPECT(qlora_linear_workspace_bytes(16, 4096, 4096, 0), 0);
  EXPECT(qlora_linear_workspace_bytes(16, 4096, 4096, 257), 0);
  EXPECT(qlora_linear_workspace_bytes(0, 4096, 4096, 8) , 0);
  EXPECT(qlora_linear_dropout_workspace_bytes(HUGE, 64, 64, 8), 0);
  EXPECT(qlora_linear_workspace_bytes(2048, 4096, 4096, 64) > 0, 1);
  {
    const int64_t n3[3] = {4096, 4096, BIG};
    EXPECT(qlora_linear_set_workspace_bytes(16, 3, n3, 4096, 8), 0);
    EXPECT(qlora_linear_set_workspace_bytes(16, 5, n3, 4096, 8), 0);
    EXPECT(qlora_linear_set_workspace_bytes(16, 2, NULL, 4096, 8), 0);
    EXPECT(qlora_linear_set_workspace_bytes(HUGE, 2, n3, 4096, 8), 0);
  }
  {
    int64_t cb = 0, nb = 0, ng = 0;
    EXPECT(qlora_nf4_sizes(BIG, BIG, &cb, &nb, &ng), QLORA_ERR_SHAPE);
    EXPECT(qlora_nf4_sizes(3, 100, &cb, &nb, &ng), QLORA_OK);
    EXPECT(cb, 150);
    EXPECT(nb, 5);
    EXPECT(ng, 1);
  }
  /* status strings: every code, and out-of-range codes */
  for (int s = -3; s <= 12; ++s) EXPECT(qlora_status_string((qlora_status)s) != NULL, 1);
  {
    float cbk[16];
    qlora_nf4_codebook(cbk);
    EXPECT(cbk[7] == 0.0f && cbk[0] == -1.0f && cbk[15] == 1.0f, 1);
    qlora_nf4_codebook(NULL);
  }

  /* quantize */
  EXPECT(qlora_quantize(P, QLORA_F32, NULL, P, 1 << 20, NULL), QLORA_ERR_NULL);
  EXPECT(qlora_quantize(NULL, QLORA_F32, &q, P, 1 << 20, NULL), QLORA_ERR_NULL);
  EXPECT(qlora_quantize(MIS, QLORA_F32, &q, P, 1 << 20, NULL), QLORA_ERR_ALIGN);
  EXPECT(qlora_quantize(P, (qlora_dtype)7, &q, P, 1 << 20, NULL), QLORA_ERR_DTYPE);
  EXPECT(qlora_quantize(P, QLORA_F32, &q, P, 16, NULL), QLORA_ERR_WORKSPACE);
  bad_q.n_out = BIG;
  bad_q.n_in = BIG;
  EXPECT(qlora_quantize(P, QLORA_F32, &bad_q, P, 1 << 20, NULL), QLORA_ERR_SHAPE);
  bad_q = q;
  bad_q.flags = 2u;
  EXPECT(qlora_quantize(P, QLORA_F32, &bad_q, P, 1 << 20, NULL), QLORA_ERR_VALUE);
  bad_q = q;
  bad_q.codes = (uint8_t *)MIS;
  EXPECT(qlora_dequantize(&bad_q, Y, NULL), QLORA_ERR_ALIGN);
  bad_q = q;
  bad_q.absmax_mean = NULL;
  EXPECT(qlora_dequantize(&bad_q, Y, NULL), QLORA_ERR_NULL);
  EXPECT(qlora_dequantize(&q, NULL, NULL), QLORA_ERR_NULL);
  EXPECT(qlora_dequantize_many(&q, 9, &Y, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_dequantize_many(&q, 0, &Y, NULL), QLORA_ERR_SHAPE);

  /* linear calls */
  const size_t ws = qlora_linear_workspace_bytes(16, 4096, 4096, 8);
  EXPECT(qlora_linear_fwd(X, 0, &q, X, X, 8, 1.0f, Y, NULL, P, ws, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_linear_fwd(X, HUGE, &q, X, X, 8, 1.0f, Y, NULL, P, ws, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_linear_fwd(X, BIG / 2, &q, X, X, 8, 1.0f, Y, NULL, P, ws, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_linear_fwd(X, 16, &q, X, X, 0, 1.0f, Y, NULL, P, ws, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_linear_fwd(X, 16, &q, X, X, 8, NAN, Y, NULL, P, ws, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_linear_fwd(X, 16, &q, X, X, 8, INFINITY, Y, NULL, P, ws, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_linear_fwd(NULL, 16, &q, X, X, 8, 1.0f, Y, NULL, P, ws, NULL), QLORA_ERR_NULL);
  EXPECT(qlora_linear_fwd(X, 16, &q, X, X, 8, 1.0f, Y, (uint16_t *)MIS, P, ws, NULL), QLORA_ERR_ALIGN);
  EXPECT(qlora_linear_fwd(X, 16, &q, X, X, 8, 1.0f, Y, NULL, P, ws - 1, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_linear_bwd(X, X, 16, &q, X, X, 8, 1.0f, NULL, Y, F, NULL, P, ws, NULL), QLORA_ERR_NULL);
  EXPECT(qlora_linear_bwd(X, X, 16, &q, X, X, 8, 1.0f, NULL, (uint16_t *)MIS, F, F, P, ws, NULL),
         QLORA_ERR_ALIGN);
  EXPECT(qlora_linear_bwd(X, X, 16, &q, X, X, 8, 1.0f, NULL, Y, F, F, P, 0, NULL), QLORA_ERR_WORKSPACE);
  bad_q = q;
  bad_q.n_in = 100;
  EXPECT(qlora_linear_fwd(X, 16, &bad_q, X, X, 8, 1.0f, Y, NULL, P, ws, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_linear_fwd_dropout(X, 16, &q, X, X, 8, 1.0f, 1.0, 7, Y, NULL, P, 1 << 30, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_linear_fwd_dropout(X, 16, &q, X, X, 8, 1.0f, NAN, 7, Y, NULL, P, 1 << 30, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_linear_bwd_dropout(X, X, 16, &q, X, X, 8, 1.0f, -0.1, 7, NULL, Y, F, F, P, 1 << 30, NULL),
         QLORA_ERR_VALUE);
  EXPECT(qlora_dropout_mask(X, 16, 12, 0.1, 1, (uint32_t *)P, Y, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_dropout_mask(X, BIG, BIG, 0.1, 1, (uint32_t *)P, Y, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_dropout_mask(X, 16, 64, 1.5, 1, (uint32_t *)P, Y, NULL), QLORA_ERR_VALUE);
  /* the forward without a workspace refuses what its scratch cannot hold, before any GPU call */
  EXPECT(qlora_linear_fwd_noalloc_max_bytes() >= ((size_t)1 << 20), 1);
  EXPECT(qlora_linear_fwd_noalloc(X, 65536, &q, X, X, 256, 1.0f, Y, NULL, NULL), QLORA_ERR_SCRATCH);
  EXPECT(qlora_linear_fwd_noalloc(X, 16, &q, X, X, 300, 1.0f, Y, NULL, NULL), QLORA_ERR_SHAPE);

  /* projection sets */
  {
    qlora_nf4_weight qs[3] = {q, q, q};
    const uint16_t *Bs[3] = {X, X, X};
    uint16_t *Ys[3] = {Y, Y, Y};
    const size_t wss = qlora_linear_set_workspace_bytes(16, 3, (const int64_t[]){4096, 4096, 4096}, 4096, 8);
    EXPECT(qlora_linear_set_fwd(X, 16, 5, qs, X, Bs, 8, 1.0f, Ys, NULL, P, wss, NULL), QLORA_ERR_SHAPE);
    qs[1].n_in = 2048;
    EXPECT(qlora_linear_set_fwd(X, 16, 3, qs, X, Bs, 8, 1.0f, Ys, NULL, P, wss, NULL), QLORA_ERR_SHAPE);
    qs[1] = q;
    qs[2].flags = 1u;
    EXPECT(qlora_linear_set_fwd(X, 16, 3, qs, X, Bs, 8, 1.0f, Ys, NULL, P, wss, NULL), QLORA_ERR_VALUE);
    qs[2] = q;
    EXPECT(qlora_linear_set_fwd(X, 16, 3, qs, X, Bs, 8, 1.0f, Ys, NULL, P, wss - 1, NULL), QLORA_ERR_WORKSPACE);
    EXPECT(qlora_linear_set_fwd(X, 16, 3, NULL, X, Bs, 8, 1.0f, Ys, NULL, P, wss, NULL), QLORA_ERR_NULL);
  }

  /* optimizer: scalar checks come before any pointer is resolved */
  EXPECT(qlora_adamw_step(F, Y, F, F, F, -1, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, NULL), QLORA_ERR_SHAPE);
  EXPECT(qlora_adamw_step(F, Y, F, F, F, 16, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_adamw_step(F, Y, F, F, F, 16, 1, NAN, 0.9, 0.999, 1e-8, 0.0, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_adamw_step(F, Y, F, F, F, 16, 1, 1e-3, 1.0, 0.999, 1e-8, 0.0, NULL), QLORA_ERR_VALUE);
  EXPECT(qlora_adamw_step(F, Y, F, F, F, 0, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, NULL), QLORA_OK);
  EXPECT(qlora_adamw_step(NULL, Y, F, F, F, 16, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, NULL), QLORA_ERR_NULL);

  if (failures) {
    fprintf(stderr, "%d validation result(s) differ\n", failures);
    return 1;
  }
  printf("abi validation: all refusals as documented\n");
  return 0;
}

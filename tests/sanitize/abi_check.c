/* Calls the C ABI's host-side paths -- argument validation of every call (no
 * device work happens before validation), the selection counts, the
 * calibration search and the cost-model fit -- from a build whose host code
 * carries AddressSanitizer and UndefinedBehaviorSanitizer, so that the
 * validation and host logic are checked for out-of-bounds accesses and
 * undefined behaviour.  Needs no GPU.  Exit status 0 when every call returned
 * its documented status.  Test infrastructure only (tests/test_sanitize.py). */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "cachetune.h"

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed: %s (line %d): %s\n", #cond, __LINE__, cachetune_last_error()); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static double quad(double r, void* user) { (void)user; return (r - 0.23) * (r - 0.23); }

int main(void) {
  for (int s = -6; s <= 1; ++s) CHECK(cachetune_status_string(s) != NULL);
  CHECK(cachetune_version() >= 1);
  /* index-array check: argument validation (no device work before it) */
  int32_t dummy_bad = 0;
  CHECK(cachetune_check_indices(NULL, 4, 10, 1, &dummy_bad, NULL) == CT_E_INVALID);
  CHECK(cachetune_check_indices((const int32_t*)256, -1, 10, 1, &dummy_bad, NULL) == CT_E_INVALID);
  CHECK(cachetune_check_indices((const int32_t*)256, 4, -1, 1, &dummy_bad, NULL) == CT_E_INVALID);
  CHECK(cachetune_check_indices((const int32_t*)256, 4, 10, 1, NULL, NULL) == CT_E_INVALID);
  /* scoring: workspace queries and argument checks */
  int32_t ns[3] = {2048, 777, 2};
  size_t bytes = 0;
  CHECK(cachetune_score_chunk_ws(NULL, ns, 3, 32, 8, 128, 1, 16, CT_FFT_EXACT_N, &bytes) == CT_OK && bytes > 0);
  CHECK(cachetune_score_chunk_ws(NULL, ns, 3, 32, 8, 128, 1, 32, CT_FFT_ZEROPAD_POW2, &bytes) == CT_OK);
  CHECK(cachetune_score_variant_ws(NULL, ns, 3, 4, 8, 128, 1, 1, CT_FFT_EXACT_N, CT_SCORE_HIGHPASS, &bytes) == CT_OK);
  CHECK(cachetune_score_variant_ws(NULL, ns, 3, 4, 8, 128, 1, 16, CT_FFT_EXACT_N, (ct_score_variant)7, &bytes) == CT_E_INVALID);
  int32_t bad[2] = {2048, 9000};
  CHECK(cachetune_score_chunk_ws(NULL, bad, 2, 32, 8, 128, 1, 16, CT_FFT_EXACT_N, &bytes) == CT_E_INVALID);
  CHECK(cachetune_score_chunk_ws(NULL, ns, 3, 0, 8, 128, 1, 16, CT_FFT_EXACT_N, &bytes) == CT_E_INVALID);
  CHECK(cachetune_score_chunk_ws(NULL, ns, 3, 32, 3, 7, 1, 16, CT_FFT_EXACT_N, &bytes) == CT_E_UNSUPPORTED);
  CHECK(cachetune_score_chunk_ws(NULL, NULL, 3, 32, 8, 128, 1, 16, CT_FFT_EXACT_N, &bytes) == CT_E_INVALID);
  ct_chunk ch[2] = {{(const void*)256, (const void*)512, 2048}, {NULL, (const void*)512, 100}};
  float* fake = (float*)1024;
  CHECK(cachetune_score_chunk(NULL, ch, 2, 4, 8, 128, CT_BF16, 1, 16, CT_FFT_EXACT_N, CT_NORM_SUM, fake, NULL,
                              NULL, 0, NULL) == CT_E_INVALID);   /* NULL K */
  CHECK(cachetune_score_chunk(NULL, ch, 1, 4, 8, 128, CT_BF16, 1, 16, CT_FFT_EXACT_N, CT_NORM_SUM, fake, NULL,
                              NULL, 0, NULL) == CT_E_WORKSPACE);
  CHECK(cachetune_score_chunk(NULL, ch, 1, 4, 8, 128, CT_BF16, 1, 16, CT_FFT_EXACT_N, (ct_norm)9, fake, NULL,
                              NULL, 0, NULL) == CT_E_INVALID);
  CHECK(cachetune_band_energy_ws(ns, 3, 4, 8, 128, CT_FFT_EXACT_N, &bytes) == CT_OK);
  /* selection */
  int32_t k[3];
  CHECK(cachetune_select_topr_counts(ns, 3, 15, 100, k) == CT_OK && k[0] == 307 && k[1] == 116 && k[2] == 0);
  CHECK(cachetune_select_topr_counts(ns, 3, 3, 2, k) == CT_E_INVALID);
  CHECK(cachetune_select_topr(NULL, fake, ns, 3, 3, 2, NULL, (int32_t*)fake, NULL, k, NULL) == CT_E_INVALID);
  /* assembly */
  ct_place pl[1];
  memset(pl, 0, sizeof(pl));
  CHECK(cachetune_assemble_rope(NULL, pl, 1, NULL, NULL, 0, 0, 8, 96, CT_BF16, 10000.0, CT_ROPE_HALF, fake,
                                fake, 10, NULL) == CT_E_UNSUPPORTED);
  CHECK(cachetune_assemble_rope(NULL, pl, 1, NULL, NULL, 0, 0, 8, 128, CT_BF16, 10000.0, CT_ROPE_HALF,
                                (char*)fake + 2, fake, 10, NULL) == CT_E_INVALID);
  CHECK(cachetune_assemble_rope(NULL, pl, 1, NULL, NULL, 0, 0, 8, 128, CT_BF16, 0.5, CT_ROPE_HALF, fake, fake,
                                10, NULL) == CT_E_INVALID);
  /* attention */
  CHECK(cachetune_recompute_attn(NULL, NULL, NULL, 0, 6, NULL, NULL, 10, 4, 128, CT_BF16, 0.1f, 10000.0,
                                 CT_ROPE_HALF, NULL, NULL, NULL, 0, NULL) == CT_E_INVALID);
  CHECK(cachetune_recompute_attn(NULL, fake, (int32_t*)fake, 4, 8, fake, fake, 10, 8, 128, CT_BF16, -1.0f,
                                 10000.0, CT_ROPE_HALF, fake, NULL, NULL, 0, NULL) == CT_E_INVALID);
  CHECK(cachetune_recompute_attn_ws(NULL, 2584, 32, 16512, 8, 128, CT_BF16, &bytes) == CT_OK && bytes > 0);
  CHECK(cachetune_recompute_attn_ws(NULL, 2584, 32, 16512, 8, 100, CT_BF16, &bytes) == CT_E_UNSUPPORTED);
  CHECK(cachetune_recompute_attn_noalloc(NULL, NULL, NULL, 0, 6, NULL, NULL, 10, 4, 128, CT_BF16, 0.1f,
                                         10000.0, CT_ROPE_HALF, NULL, NULL, NULL) == CT_E_INVALID);
  /* recompute layer */
  CHECK(cachetune_rmsnorm(fake, fake, 4, 100, 1e-5f, CT_BF16, fake, NULL) == CT_E_INVALID);
  CHECK(cachetune_linear(fake, fake, NULL, 4, 12, 64, CT_BF16, fake, NULL) == CT_E_INVALID);
  CHECK(cachetune_qkv_proj(fake, fake, 4, 64, 12, 8, CT_BF16, fake, fake, fake, NULL) == CT_E_INVALID);
  CHECK(cachetune_silu_mul(fake, 3, 12, CT_BF16, fake, NULL) == CT_E_INVALID);
  /* host tier */
  CHECK(cachetune_rank_order(fake, fake, (int32_t*)fake, 0, 2, 8, 128, CT_BF16, fake, fake, NULL) == CT_E_INVALID);
  /* context handle without a usable device */
  ct_handle h = NULL;
  CHECK(cachetune_create(-1, &h) != CT_OK && h == NULL);
  cachetune_destroy(NULL);
  CHECK(cachetune_prepare_scoring(NULL, ns, 3, 1, 16, CT_FFT_EXACT_N, NULL) == CT_E_INVALID);
  /* calibration and the cost model */
  double r = 0.0;
  int32_t probes = 0;
  CHECK(cachetune_calibrate_ratio(1.0, 0.25, 0.0, 1.0, 0.1, 0.001, quad, NULL, &r, &probes) == CT_OK);
  CHECK(fabs(r - 0.23) < 0.01 && probes > 2);
  CHECK(cachetune_calibrate_ratio(-1.0, 0.25, 0.0, 1.0, 0.1, 0.001, quad, NULL, &r, &probes) == CT_E_INVALID);
  const double rs[6] = {0.02, 0.05, 0.10, 0.15, 0.20, 0.30};
  double ts[6];
  for (int i = 0; i < 6; ++i) {
    const double a = rs[i] * 65536 * 0.6e-3, b = (1 - rs[i]) * 65536 * 0.085e-3;
    ts[i] = 32 * (1.0 + (a > b ? a : b));
  }
  double tc = 0, ti = 0, to = 0;
  CHECK(cachetune_fit_cost_model(rs, ts, 6, 32, 65536, &tc, &ti, &to) == CT_OK);
  CHECK(fabs(tc - 0.6e-3) < 1e-9 && fabs(ti - 0.085e-3) < 1e-9 && fabs(to - 1.0) < 1e-6);
  CHECK(cachetune_fit_cost_model(rs, ts, 3, 32, 65536, &tc, &ti, &to) == CT_E_INVALID);
  printf("ABI sanitizer drive: %d failed checks\n", failures);
  return failures ? 1 : 0;
}

/* Drives every function of oracle/oracle.c over small and edge-case shapes
 * (lengths 1, 2, odd, prime and powers of two, both transform lengths, every
 * normalisation, k = 0 and k = n, both RoPE styles, fp32 and bf16 storage) so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer can report
 * any out-of-bounds access, leak, overflow or other undefined behaviour.
 * Exit status 0 when every call returned its documented status.  Test
 * infrastructure only (run by tests/test_sanitize.py). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t orc_round_bf16(double v);
int orc_nbins(int n);
int orc_kkeep(int nbins, int a_num, int a_den);
int orc_ksel(int n, int r_num, int r_den);
int orc_fft_len(int n, int mode);
void orc_rfft(const double* x, int n, double* re, double* im);
void orc_lowpass(const double* x, int n, int a_num, int a_den, int fftlen_mode, double* out);
int orc_score_chunk(const void* K, const void* V, int dtype, int L, int N, int H, int D, int a_num,
                    int a_den, int fftlen_mode, int norm, double* layer_score, double* score);
void orc_topr(const double* score, int N, int k, int* ranking, int* sel, int* comp);
void orc_offsets(const int* n_per_chunk, const int* order, int n_chunks, int prefix, int* offsets);
void orc_rope(const double* x, int D, double pos, double theta, int style, double* y);
void orc_assemble_chunk(const void* k_src, const void* v_src, const void* k_rec, const void* v_rec,
                        const int* sel, int n, int k, int offset, int H, int D, int dtype, double theta,
                        int style, void* k_out, void* v_out);
void orc_assemble_rows(const void* k_rows, const void* v_rows, int n, int start, int H, int D, int dtype,
                       double theta, int style, void* k_out, void* v_out);
int orc_attention(const void* q_pre, const int* qpos, int Hq, const void* k, const void* v, int T, int H,
                  int D, int dtype, double scale, double theta, int style, const int* rows, int n_rows,
                  double* out, double* lse);
int orc_score_l2(const void* K, const void* V, int dtype, int L, int N, int H, int D, int norm,
                 double* layer_score, double* score);
void orc_highpass(const double* x, int n, int a_num, int a_den, int fftlen_mode, double* out);
int orc_score_highpass(const void* K, const void* V, int dtype, int L, int N, int H, int D, int a_num,
                       int a_den, int fftlen_mode, int norm, double* layer_score, double* score);
int orc_band_energy(const void* X, int dtype, int L, int N, int H, int D, int fftlen_mode, int n_bands,
                    double* fraction, double* total);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uni(void) {  /* xorshift64*, uniform in [-2, 2) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0 * 4.0 - 2.0;
}

/* a buffer of `count` elements of the storage type, filled with values */
static void* fill(int dtype, size_t count) {
  if (dtype == 0) {
    float* f = malloc(sizeof(float) * (count ? count : 1));
    for (size_t i = 0; i < count; ++i) f[i] = (float)uni();
    return f;
  }
  uint16_t* h = malloc(sizeof(uint16_t) * (count ? count : 1));
  for (size_t i = 0; i < count; ++i) h[i] = orc_round_bf16(uni());
  return h;
}

static int failures = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                \
    }                                                            \
  } while (0)

int main(void) {
  const int lens[] = {1, 2, 3, 7, 16, 31, 64, 97};
  const int nl = (int)(sizeof(lens) / sizeof(lens[0]));
  for (int li = 0; li < nl; ++li) {
    const int n = lens[li];
    double* x = malloc(sizeof(double) * n);
    for (int i = 0; i < n; ++i) x[i] = uni();
    for (int mode = 0; mode < 2; ++mode) {
      const int nf = orc_fft_len(n, mode);
      CHECK(nf >= n);
      double* re = malloc(sizeof(double) * orc_nbins(nf));
      double* im = malloc(sizeof(double) * orc_nbins(nf));
      double* pad = calloc(nf, sizeof(double));
      memcpy(pad, x, sizeof(double) * n);
      orc_rfft(pad, nf, re, im);
      double* lo = malloc(sizeof(double) * n);
      double* hi = malloc(sizeof(double) * n);
      const int alphas[][2] = {{1, 16}, {1, 2}, {1, 1}};
      for (int a = 0; a < 3; ++a) {
        orc_lowpass(x, n, alphas[a][0], alphas[a][1], mode, lo);
        orc_highpass(x, n, alphas[a][0], alphas[a][1], mode, hi);
        for (int i = 0; i < n; ++i) CHECK(isfinite(lo[i]) && isfinite(hi[i]));
      }
      free(re);
      free(im);
      free(pad);
      free(lo);
      free(hi);
    }
    for (int k = 0; k <= n; k += (n > 4 ? n / 4 : 1)) {
      int* rk = malloc(sizeof(int) * n);
      int* sel = malloc(sizeof(int) * (k ? k : 1));
      int* comp = malloc(sizeof(int) * (n - k ? n - k : 1));
      orc_topr(x, n, k, rk, sel, comp);
      free(rk);
      free(sel);
      free(comp);
    }
    free(x);
  }
  /* scores, all norms and both storage types */
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int li = 1; li < nl; ++li) {
      const int L = 2, N = lens[li], H = 2, D = 4;
      void* K = fill(dtype, (size_t)L * N * H * D);
      void* V = fill(dtype, (size_t)L * N * H * D);
      double* ls = malloc(sizeof(double) * L * N);
      double* s = malloc(sizeof(double) * N);
      for (int norm = 0; norm < 4; ++norm)
        for (int mode = 0; mode < 2; ++mode) {
          CHECK(orc_score_chunk(K, V, dtype, L, N, H, D, 1, 16, mode, norm, ls, s) == 0);
          CHECK(orc_score_highpass(K, V, dtype, L, N, H, D, 1, 4, mode, norm, ls, s) == 0);
        }
      CHECK(orc_score_l2(K, V, dtype, L, N, H, D, 0, ls, s) == 0);
      CHECK(orc_score_chunk(K, V, dtype, 0, N, H, D, 1, 16, 0, 0, ls, s) == -1);
      const int nb = orc_nbins(N);
      double* fr = malloc(sizeof(double) * L * nb);
      double* tot = malloc(sizeof(double) * L);
      CHECK(orc_band_energy(K, dtype, L, N, H, D, 0, nb, fr, tot) == 0);
      free(fr);
      free(tot);
      free(ls);
      free(s);
      free(K);
      free(V);
    }
  /* offsets, RoPE, assembly and attention */
  {
    const int ns[] = {5, 3, 9}, order[] = {2, 0, 1};
    int offs[3];
    orc_offsets(ns, order, 3, 7, offs);
    CHECK(offs[2] == 7 && offs[0] == 16 && offs[1] == 21);
  }
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int style = 0; style < 2; ++style) {
      const int H = 2, D = 8, n = 11, k = 4, T = n + 3 + 2, Hq = 4;
      double xr[8], yr[8];
      for (int i = 0; i < D; ++i) xr[i] = uni();
      orc_rope(xr, D, 123456.0, 500000.0, style, yr);
      void* ks = fill(dtype, (size_t)n * H * D);
      void* vs = fill(dtype, (size_t)n * H * D);
      void* kr = fill(dtype, (size_t)k * H * D);
      void* vr = fill(dtype, (size_t)k * H * D);
      void* kx = fill(dtype, (size_t)2 * H * D);
      void* vx = fill(dtype, (size_t)2 * H * D);
      const int sel[] = {0, 3, 7, 10};
      const size_t es = dtype == 0 ? 4 : 2;
      void* ko = calloc((size_t)T * H * D, es);
      void* vo = calloc((size_t)T * H * D, es);
      orc_assemble_chunk(ks, vs, kr, vr, sel, n, k, 3, H, D, dtype, 10000.0, style, ko, vo);
      orc_assemble_chunk(ks, vs, NULL, NULL, sel, n, 0, 3, H, D, dtype, 10000.0, style, ko, vo);
      orc_assemble_rows(kx, vx, 2, n + 3, H, D, dtype, 10000.0, style, ko, vo);
      const int qpos[] = {0, 5, 13, 15};
      const int rows[] = {3, 0};
      void* q = fill(dtype, (size_t)4 * Hq * D);
      double* out = malloc(sizeof(double) * 4 * Hq * D);
      double* lse = malloc(sizeof(double) * 4 * Hq);
      const int all[] = {0, 1, 2, 3};
      CHECK(orc_attention(q, qpos, Hq, ko, vo, T, H, D, dtype, 0.35, 10000.0, style, all, 4, out, lse) == 0);
      CHECK(orc_attention(q, qpos, Hq, ko, vo, T, H, D, dtype, 0.35, 10000.0, style, rows, 2, out, NULL) == 0);
      CHECK(orc_attention(q, qpos, 3, ko, vo, T, H, D, dtype, 0.35, 10000.0, style, rows, 2, out, lse) == -1);
      free(ks); free(vs); free(kr); free(vr); free(kx); free(vx); free(ko); free(vo); free(q); free(out); free(lse);
    }
  CHECK(orc_ksel(512, 15, 100) == 76);
  CHECK(orc_kkeep(orc_nbins(2048), 1, 16) == 64);
  CHECK(orc_round_bf16(NAN) == 0x7fc0);
  CHECK(orc_round_bf16(1e39) == 0x7f80);
  CHECK(orc_round_bf16(-0.0) == 0x8000);
  printf("oracle sanitizer drive: %d failed checks\n", failures);
  return failures ? 1 : 0;
}

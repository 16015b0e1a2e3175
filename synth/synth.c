/*
 * Seeded synthetic inputs for the CacheTune hot path.
 *
 * This module holds the input value model only -- none of the method's
 * arithmetic.  Both the oracle and the GPU library consume the buffers it
 * writes, so the two sides see bit-identical inputs.
 *
 * Every value is a pure function of (seed, tensor, chunk, layer, token, head,
 * dim): a SplitMix64-based counter hash (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) keyed by those indices, turned
 * into uniforms and into normals by the Box-Muller transform.  Results do not
 * depend on the number of threads.
 *
 * Value model of one channel (chunk b, layer l, tensor t, head h, dim d), token n
 * of a chunk of N tokens:
 *   v[n] = ( z[n] + sum_{s<3} A_s cos(2 pi f_s n / N + phi_s) ) * (5 if n is a
 *          spike token of chunk b else 1)
 *   z[n] ~ N(0,1); f_s uniform on {1..8}; A_s ~ U(0.5, 2); phi_s ~ U[0, 2 pi);
 *   4 distinct spike tokens per chunk, shared by all layers, heads, channels
 *   and tensors.  Computed in fp64, stored with one round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SY_F32 0
#define SY_BF16 1

enum { TAG_SIN = 11, TAG_NOISE = 12, TAG_SPIKE = 13, TAG_EXTRA = 14, TAG_INTS = 15,
       TAG_PERM = 16, TAG_NORMAL = 17 };

static inline uint64_t sm64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t hkey(uint64_t seed, uint64_t a, uint64_t b, uint64_t c,
                            uint64_t d, uint64_t e, uint64_t f) {
  uint64_t h = sm64(seed);
  h = sm64(h ^ a);
  h = sm64(h ^ b);
  h = sm64(h ^ c);
  h = sm64(h ^ d);
  h = sm64(h ^ e);
  h = sm64(h ^ f);
  return h;
}

/* Uniform on (0, 1) from the top 53 bits. */
static inline double u01(uint64_t h) { return ((double)(h >> 11) + 0.5) * 0x1.0p-53; }

static inline double normal_from(uint64_t h) {
  double u1 = u01(sm64(h ^ 0x1111));
  double u2 = u01(sm64(h ^ 0x2222));
  return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

static uint16_t to_bf16(double v) {
  if (isnan(v)) return 0x7fc0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  double r = nearbyint(ldexp(a, -q));
  double back = ldexp(r, q);
  if (back > 0x1.fep127) return sign | 0x7f80;
  float f = (float)back;
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return sign | (uint16_t)((bits >> 16) & 0x7fff);
}

static void put(void* out, int dtype, size_t i, double v) {
  if (dtype == SY_F32) ((float*)out)[i] = (float)v;
  else ((uint16_t*)out)[i] = to_bf16(v);
}

static double stored(int dtype, double v) {
  if (dtype == SY_F32) return (double)(float)v;
  uint32_t bits = ((uint32_t)to_bf16(v)) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* The 4 distinct spike tokens of chunk `chunk` (N >= 4), ascending. */
void synth_spikes(uint64_t seed, int chunk, int N, int* out) {
  int cnt = 0;
  for (int attempt = 0; cnt < 4 && cnt < N; ++attempt) {
    int p = (int)(u01(hkey(seed, TAG_SPIKE, (uint64_t)chunk, (uint64_t)attempt, 0, 0, 0)) * N);
    if (p >= N) p = N - 1;
    int dup = 0;
    for (int i = 0; i < cnt; ++i) dup |= (out[i] == p);
    if (!dup) out[cnt++] = p;
  }
  for (int i = 0; i < cnt; ++i)
    for (int j = i + 1; j < cnt; ++j)
      if (out[j] < out[i]) { int t = out[i]; out[i] = out[j]; out[j] = t; }
}

typedef struct { int f[3]; double amp[3], cph[3], sph[3]; } chan_params;

static void channel_params(uint64_t seed, int tensor, int chunk, int layer, int ch,
                           chan_params* p) {
  for (int s = 0; s < 3; ++s) {
    uint64_t base = hkey(seed, TAG_SIN, (uint64_t)tensor, (uint64_t)chunk, (uint64_t)layer,
                         (uint64_t)ch, (uint64_t)s);
    int f = 1 + (int)(u01(sm64(base ^ 1)) * 8.0);
    if (f > 8) f = 8;
    p->f[s] = f;
    p->amp[s] = 0.5 + 1.5 * u01(sm64(base ^ 2));
    double ph = 2.0 * M_PI * u01(sm64(base ^ 3));
    p->cph[s] = cos(ph);
    p->sph[s] = sin(ph);
  }
}

/* Value of the model at (token n) for one channel, fp64. cosN/sinN: tables of
 * cos/sin(2 pi m / N). */
static double model_value(uint64_t seed, int tensor, int chunk, int layer, int ch, int n,
                          int N, const chan_params* p, const double* cosN,
                          const double* sinN, const int* spikes, int nspk) {
  double v = normal_from(hkey(seed, TAG_NOISE, (uint64_t)tensor, (uint64_t)chunk,
                              (uint64_t)layer, (uint64_t)ch, (uint64_t)n));
  for (int s = 0; s < 3; ++s) {
    int m = (int)(((long long)p->f[s] * n) % N);
    /* cos(a + phi) = cos a cos phi - sin a sin phi */
    v += p->amp[s] * (cosN[m] * p->cph[s] - sinN[m] * p->sph[s]);
  }
  for (int i = 0; i < nspk; ++i)
    if (spikes[i] == n) v *= 5.0;
  return v;
}

/* Evaluate the value model at the listed token rows of one (tensor, chunk,
 * layer): out[r][H*D] for r < nrows (rows == NULL means all N rows).
 * If extra_sigma > 0 the stored value is perturbed by extra_sigma * N(0,1)
 * (drawn from an independent stream) and stored again: this models rows that
 * were recomputed in the new context. */
void synth_rows(uint64_t seed, int tensor, int chunk, int layer, int N, int H, int D,
                const int* rows, int nrows, double extra_sigma, int dtype, void* out) {
  int Cn = H * D;
  double* cosN = malloc(sizeof(double) * N);
  double* sinN = malloc(sizeof(double) * N);
  for (int m = 0; m < N; ++m) {
    cosN[m] = cos(2.0 * M_PI * (double)m / (double)N);
    sinN[m] = sin(2.0 * M_PI * (double)m / (double)N);
  }
  int spikes[4];
  synth_spikes(seed, chunk, N, spikes);
  int nspk = N < 4 ? N : 4;
  chan_params* prm = malloc(sizeof(chan_params) * Cn);
#pragma omp parallel for schedule(static)
  for (int ch = 0; ch < Cn; ++ch) channel_params(seed, tensor, chunk, layer, ch, &prm[ch]);
  if (rows == NULL) nrows = N;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < nrows; ++r) {
    int n = rows ? rows[r] : r;
    for (int ch = 0; ch < Cn; ++ch) {
      double v = model_value(seed, tensor, chunk, layer, ch, n, N, &prm[ch], cosN, sinN,
                             spikes, nspk);
      if (extra_sigma > 0.0) {
        v = stored(dtype, v);
        v += extra_sigma * normal_from(hkey(seed, TAG_EXTRA, (uint64_t)tensor,
                                            (uint64_t)chunk, (uint64_t)layer, (uint64_t)ch,
                                            (uint64_t)n));
      }
      put(out, dtype, (size_t)r * Cn + ch, v);
    }
  }
  free(prm);
  free(cosN);
  free(sinN);
}

/* Whole chunk tensor [L][N][H][D] for layers [l0, l0+L). */
void synth_chunk(uint64_t seed, int tensor, int chunk, int l0, int L, int N, int H, int D,
                 int dtype, void* out) {
  size_t es = dtype == SY_F32 ? 4 : 2;
  for (int l = 0; l < L; ++l)
    synth_rows(seed, tensor, chunk, l0 + l, N, H, D, NULL, N, 0.0, dtype,
               (char*)out + es * (size_t)l * N * H * D);
}

/* n integers uniform on [lo, hi]. */
void synth_uniform_ints(uint64_t seed, int stream, int n, int lo, int hi, int* out) {
  for (int i = 0; i < n; ++i) {
    double u = u01(hkey(seed, TAG_INTS, (uint64_t)stream, (uint64_t)i, 0, 0, 0));
    int v = lo + (int)(u * (double)(hi - lo + 1));
    if (v > hi) v = hi;
    out[i] = v;
  }
}

/* A uniformly random permutation of [0, n) (Fisher-Yates). */
void synth_permutation(uint64_t seed, int stream, int n, int* out) {
  for (int i = 0; i < n; ++i) out[i] = i;
  for (int i = n - 1; i > 0; --i) {
    double u = u01(hkey(seed, TAG_PERM, (uint64_t)stream, (uint64_t)i, 0, 0, 0));
    int j = (int)(u * (double)(i + 1));
    if (j > i) j = i;
    int t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/* n i.i.d. N(mean, sigma^2) values of stream `stream` (element i from the
 * counter-based hash of (seed, stream, i)), stored in dtype.  Synthetic
 * weights, gains and hidden rows of the recompute layer. */
void synth_normal(uint64_t seed, int stream, long long n, double mean, double sigma, int dtype,
                  void* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < n; ++i)
    put(out, dtype, (size_t)i, mean + sigma * normal_from(hkey(seed, TAG_NORMAL, (uint64_t)stream,
                                                                (uint64_t)i, 0, 0, 0)));
}

/*
 * Reference oracle for the CacheTune hot path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU implementation of what the method computes, written
 * from "Adaptive KV Cache Reuse for Fast Long-Context LLM Serving" (CacheTune):
 *   - offline scoring, App. B.1 "Offline Preparation" (and Sec. 4.1);
 *   - index mapping, App. B.1 (last paragraph);
 *   - assembly with deferred RoPE, App. B.2 "Sparse KV Reuse Pipeline" and
 *     App. B.3 "Deferred RoPE for Positional Alignment";
 *   - selected-query causal attention, Sec. 4.1 "Recomputing in the new context".
 *
 * Only tests, the smoke entry and the bench's CPU-baseline leg may load this
 * library.  It shares no code with the GPU library: every helper here
 * (widening, rounding, trig tables) is written independently.
 *
 * Parity status of each function is stated in its comment; every function is
 * pinned by closed forms, invariants or brute force in the CPU test-suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_FFT_EXACT_N 0
#define ORC_FFT_ZEROPAD_POW2 1

#define ORC_NORM_SUM 0
#define ORC_NORM_MAX 1
#define ORC_NORM_MINMAX 2
#define ORC_NORM_NONE 3

#define ORC_ROPE_HALF 0
#define ORC_ROPE_INTERLEAVED 1

/* ---- storage helpers (exact widening; single RNE rounding on store) ---- */

static double load_elem(const void* base, int dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* Round a double to the nearest bfloat16 (ties to even) in one step. */
uint16_t orc_round_bf16(double v) {
  if (isnan(v)) return 0x7fc0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  /* bf16: 8 significant bits, exponent range of binary32. */
  int e;
  frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
  int q = e - 8;                /* quantum exponent for normals */
  if (q < -133) q = -133;       /* subnormal quantum 2^-133 */
  double scaled = ldexp(a, -q); /* exact */
  double r = nearbyint(scaled); /* ties to even under default rounding */
  double back = ldexp(r, q);
  if (back > 0x1.fep127) return sign | 0x7f80; /* beyond the largest finite */
  float f = (float)back; /* exact: back has <= 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return sign | (uint16_t)((bits >> 16) & 0x7fff);
}

/* v rounded once to the storage type and widened back (exact). */
static double round_to_storage(double v, int dtype) {
  if (dtype == ORC_F32) return (double)(float)v;
  uint32_t bits = (uint32_t)orc_round_bf16(v) << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static void store_elem(void* base, int dtype, size_t i, double v) {
  if (dtype == ORC_F32)
    ((float*)base)[i] = (float)v; /* C conversion rounds to nearest even */
  else
    ((uint16_t*)base)[i] = orc_round_bf16(v);
}

/* ---- sizes (App. B.1) ---- */

/* Number of non-redundant rFFT bins of a real sequence of length n. */
int orc_nbins(int n) { return n / 2 + 1; }

/* Retained low-frequency bins: the lowest alpha fraction of the bins, at least
 * one (the DC bin), at most all of them. alpha = a_num / a_den. */
int orc_kkeep(int nbins, int a_num, int a_den) {
  long long k = ((long long)a_num * nbins) / a_den;
  if (k < 1) k = 1;
  if (k > nbins) k = nbins;
  return (int)k;
}

/* Size of the recomputation set: the top-ranked r*N positions, r = r_num/r_den. */
int orc_ksel(int n, int r_num, int r_den) {
  long long k = ((long long)r_num * n) / r_den;
  if (k < 0) k = 0;
  if (k > n) k = n;
  return (int)k;
}

/* Transform length used for a chunk of n tokens. */
int orc_fft_len(int n, int mode) {
  if (mode == ORC_FFT_EXACT_N) return n;
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

/* ---- discrete Fourier transform, direct O(N * bins) ---- */

/* c[m] = cos(2*pi*m/n), s[m] = sin(2*pi*m/n), m in [0, n).  The angle is split
 * into a quarter-turn count and a remainder so that the values at multiples of
 * a quarter turn are exactly 0 and +-1. */
static void trig_table(int n, double* c, double* s) {
  for (int m = 0; m < n; ++m) {
    long long t = 4LL * m;
    int quad = (int)(t / n);
    long long rem = t - (long long)quad * n; /* angle = (quad + rem/n) * pi/2 */
    double a = (M_PI / 2.0) * ((double)rem / (double)n);
    double ca = cos(a), sa = sin(a);
    if (rem == 0) { ca = 1.0; sa = 0.0; }
    switch (quad & 3) {
      case 0: c[m] = ca;  s[m] = sa;  break;
      case 1: c[m] = -sa; s[m] = ca;  break;
      case 2: c[m] = -ca; s[m] = -sa; break;
      default: c[m] = sa; s[m] = -ca; break;
    }
  }
}

/* X[j] = sum_n x[n] * exp(-2*pi*i*j*n/n_len) for j < nb, returned as re/im. */
static void dft_bins(const double* x, int n_len, int nb, const double* c,
                     const double* s, double* re, double* im) {
  for (int j = 0; j < nb; ++j) {
    double acc_r = 0.0, acc_i = 0.0;
    int m = 0; /* (j * n) mod n_len, advanced exactly */
    for (int n = 0; n < n_len; ++n) {
      acc_r += x[n] * c[m];
      acc_i -= x[n] * s[m];
      m += j;
      if (m >= n_len) m -= n_len;
    }
    re[j] = acc_r;
    im[j] = acc_i;
  }
}

/* Inverse real transform with output length n_len (the irfft(n=N) convention:
 * 1/N scaling, bins strictly between DC and Nyquist counted twice, the real
 * part only of DC and Nyquist) of a spectrum whose bins >= kkeep are zero.
 * Bins at and above the cutoff contribute zero, so only j < kkeep are summed. */
static void inverse_lowpass(const double* re, const double* im, int n_len,
                            int kkeep, const double* c, const double* s,
                            double* out) {
  for (int n = 0; n < n_len; ++n) {
    double acc = 0.0;
    int m = 0; /* (j * n) mod n_len */
    for (int j = 0; j < kkeep; ++j) {
      double w = 2.0;
      if (j == 0) w = 1.0;
      if ((n_len % 2 == 0) && j == n_len / 2) w = 1.0;
      double term = re[j] * c[m];
      if (!(j == 0 || ((n_len % 2 == 0) && j == n_len / 2))) term -= im[j] * s[m];
      acc += w * term;
      m += n;
      if (m >= n_len) m -= n_len;
    }
    out[n] = acc / (double)n_len;
  }
}

/* Full spectrum of a real sequence, bins [0, nbins): exported for tests. */
void orc_rfft(const double* x, int n, double* re, double* im) {
  double* c = malloc(sizeof(double) * n);
  double* s = malloc(sizeof(double) * n);
  trig_table(n, c, s);
  dft_bins(x, n, orc_nbins(n), c, s, re, im);
  free(c);
  free(s);
}

/* Low-frequency reconstruction of one real sequence of n tokens (App. B.1):
 * rFFT over the transform length, keep the lowest alpha fraction of the
 * bins, inverse transform, positions [0, n). */
void orc_lowpass(const double* x, int n, int a_num, int a_den, int fftlen_mode,
                 double* out) {
  int nf = orc_fft_len(n, fftlen_mode);
  int kk = orc_kkeep(orc_nbins(nf), a_num, a_den);
  double* c = malloc(sizeof(double) * nf);
  double* s = malloc(sizeof(double) * nf);
  double* xp = calloc(nf, sizeof(double));
  double* re = malloc(sizeof(double) * kk);
  double* im = malloc(sizeof(double) * kk);
  double* rec = malloc(sizeof(double) * nf);
  memcpy(xp, x, sizeof(double) * n);
  trig_table(nf, c, s);
  dft_bins(xp, nf, kk, c, s, re, im);
  inverse_lowpass(re, im, nf, kk, c, s, rec);
  memcpy(out, rec, sizeof(double) * n);
  free(c); free(s); free(xp); free(re); free(im); free(rec);
}

/* ---- chunk scoring (App. B.1, second paragraph) ---- */

/* Per-token magnitude of the low-passed tensor of one layer: the L2 norm over
 * all H*D channels of the token.  x is [N][C] (C = H*D) in storage dtype. */
static void layer_magnitude(const void* x, int dtype, size_t layer_off, int N,
                            int C, int nf, int kk, const double* c,
                            const double* s, double* mag) {
  double* rec = malloc(sizeof(double) * (size_t)C * N);
#pragma omp parallel
  {
    double* seq = calloc(nf, sizeof(double));
    double* re = malloc(sizeof(double) * kk);
    double* im = malloc(sizeof(double) * kk);
    double* out = malloc(sizeof(double) * nf);
#pragma omp for schedule(static)
    for (int ch = 0; ch < C; ++ch) {
      for (int n = 0; n < N; ++n)
        seq[n] = load_elem(x, dtype, layer_off + (size_t)n * C + ch);
      dft_bins(seq, nf, kk, c, s, re, im);
      inverse_lowpass(re, im, nf, kk, c, s, out);
      memcpy(rec + (size_t)ch * N, out, sizeof(double) * N);
    }
    free(seq); free(re); free(im); free(out);
  }
  for (int n = 0; n < N; ++n) {
    double e = 0.0;
    for (int ch = 0; ch < C; ++ch) {
      double v = rec[(size_t)ch * N + n];
      e += v * v;
    }
    mag[n] = sqrt(e);
  }
  free(rec);
}

/* Per-layer normalisation of a non-negative score vector. */
static void normalise(double* v, int N, int norm) {
  if (norm == ORC_NORM_NONE) return;
  if (norm == ORC_NORM_SUM) {
    double t = 0.0;
    for (int n = 0; n < N; ++n) t += v[n];
    for (int n = 0; n < N; ++n) v[n] = (t > 0.0) ? v[n] / t : 1.0 / (double)N;
    return;
  }
  double mx = v[0], mn = v[0];
  for (int n = 1; n < N; ++n) {
    if (v[n] > mx) mx = v[n];
    if (v[n] < mn) mn = v[n];
  }
  if (norm == ORC_NORM_MAX) {
    for (int n = 0; n < N; ++n) v[n] = (mx > 0.0) ? v[n] / mx : 0.0;
  } else {
    double d = mx - mn;
    for (int n = 0; n < N; ++n) v[n] = (d > 0.0) ? (v[n] - mn) / d : 0.0;
  }
}

/* Importance score of one chunk.  K, V: [L][N][H][D] pre-RoPE, storage dtype.
 * For each layer: magnitudes of the low-frequency K and of the low-frequency
 * V at each position, combined with equal weights (1/2 each), normalised
 * within the layer; the layer scores are then averaged.
 * layer_score (optional, [L][N]) receives the normalised per-layer scores.
 * Returns 0, or -1 on bad arguments. */
int orc_score_chunk(const void* K, const void* V, int dtype, int L, int N,
                    int H, int D, int a_num, int a_den, int fftlen_mode,
                    int norm, double* layer_score, double* score) {
  if (L < 1 || N < 1 || H < 1 || D < 1 || a_den <= 0 || a_num <= 0) return -1;
  int C = H * D;
  int nf = orc_fft_len(N, fftlen_mode);
  int kk = orc_kkeep(orc_nbins(nf), a_num, a_den);
  double* c = malloc(sizeof(double) * nf);
  double* s = malloc(sizeof(double) * nf);
  trig_table(nf, c, s);
  double* a = malloc(sizeof(double) * N);
  double* b = malloc(sizeof(double) * N);
  double* sl = malloc(sizeof(double) * N);
  for (int n = 0; n < N; ++n) score[n] = 0.0;
  for (int l = 0; l < L; ++l) {
    size_t off = (size_t)l * N * C;
    layer_magnitude(K, dtype, off, N, C, nf, kk, c, s, a);
    layer_magnitude(V, dtype, off, N, C, nf, kk, c, s, b);
    for (int n = 0; n < N; ++n) sl[n] = 0.5 * a[n] + 0.5 * b[n];
    normalise(sl, N, norm);
    if (layer_score) memcpy(layer_score + (size_t)l * N, sl, sizeof(double) * N);
    for (int n = 0; n < N; ++n) score[n] += sl[n];
  }
  for (int n = 0; n < N; ++n) score[n] /= (double)L;
  free(c); free(s); free(a); free(b); free(sl);
  return 0;
}

/* ---- top-r selection (App. B.1: the highest-scoring floor(rN) positions) ---- */

static const double* g_sort_key;
static int cmp_rank(const void* pa, const void* pb) {
  int ia = *(const int*)pa, ib = *(const int*)pb;
  double a = g_sort_key[ia], b = g_sort_key[ib];
  if (a > b) return -1; /* higher score first */
  if (a < b) return 1;
  return (ia < ib) ? -1 : (ia > ib); /* equal scores: lower index first */
}
static int cmp_int(const void* pa, const void* pb) {
  int a = *(const int*)pa, b = *(const int*)pb;
  return (a > b) - (a < b);
}

/* ranking: all N local indices by (score desc, index asc); sel: the first k of
 * the ranking in ascending order; comp: the other N-k in ascending order.
 * Any output pointer may be NULL. */
void orc_topr(const double* score, int N, int k, int* ranking, int* sel,
              int* comp) {
  int* idx = malloc(sizeof(int) * (N > 0 ? N : 1));
  for (int i = 0; i < N; ++i) idx[i] = i;
  g_sort_key = score;
  qsort(idx, N, sizeof(int), cmp_rank);
  if (ranking) memcpy(ranking, idx, sizeof(int) * N);
  if (sel) {
    memcpy(sel, idx, sizeof(int) * k);
    qsort(sel, k, sizeof(int), cmp_int);
  }
  if (comp) {
    memcpy(comp, idx + k, sizeof(int) * (N - k));
    qsort(comp, N - k, sizeof(int), cmp_int);
  }
  free(idx);
}

/* ---- index mapping (App. B.1, last paragraph) ---- */

/* order[p] = id of the chunk placed p-th in the prompt; the chunk placed first
 * starts at global position `prefix`.  offsets[id] = global start of chunk id.
 * Local index i (0-based) of chunk b maps to offsets[b] + i. */
void orc_offsets(const int* n_per_chunk, const int* order, int n_chunks,
                 int prefix, int* offsets) {
  int pos = prefix;
  for (int p = 0; p < n_chunks; ++p) {
    offsets[order[p]] = pos;
    pos += n_per_chunk[order[p]];
  }
}

/* ---- RoPE (App. B.3) ---- */

/* Inverse frequencies f_j = theta^(-2j/D), j < D/2. */
void orc_rope_freqs(int D, double theta, double* f) {
  for (int j = 0; j < D / 2; ++j) f[j] = pow(theta, -2.0 * (double)j / (double)D);
}

/* Rotate one head vector x[D] to position pos.  Pairs are (j, j+D/2) for the
 * rotate-half style and (2j, 2j+1) for the interleaved style; pair j turns by
 * the angle pos * f_j. */
void orc_rope(const double* x, int D, double pos, double theta, int style,
              double* y) {
  for (int j = 0; j < D / 2; ++j) {
    double ang = pos * pow(theta, -2.0 * (double)j / (double)D);
    double cs = cos(ang), sn = sin(ang);
    int i0 = (style == ORC_ROPE_HALF) ? j : 2 * j;
    int i1 = (style == ORC_ROPE_HALF) ? j + D / 2 : 2 * j + 1;
    double a = x[i0], b = x[i1];
    y[i0] = a * cs - b * sn;
    y[i1] = a * sn + b * cs;
  }
}

/* ---- assembly of one layer's working buffer (App. B.2 / B.3) ---- */

/* Write one row: K rotated to global position g, V copied. */
static void put_row(const void* ksrc, const void* vsrc, size_t src_row, int H,
                    int D, int dtype, double theta, int style, int g,
                    void* k_out, void* v_out) {
  double* x = malloc(sizeof(double) * D);
  double* y = malloc(sizeof(double) * D);
  size_t so = src_row * (size_t)H * D, dst = (size_t)g * H * D;
  for (int h = 0; h < H; ++h) {
    for (int d = 0; d < D; ++d) x[d] = load_elem(ksrc, dtype, so + (size_t)h * D + d);
    orc_rope(x, D, (double)g, theta, style, y);
    for (int d = 0; d < D; ++d) {
      store_elem(k_out, dtype, dst + (size_t)h * D + d, y[d]);
      /* V is a plain copy of the stored value. */
      store_elem(v_out, dtype, dst + (size_t)h * D + d,
                 load_elem(vsrc, dtype, so + (size_t)h * D + d));
    }
  }
  free(x);
  free(y);
}

/* Place one chunk of n rows at global offset `offset`.
 * k_src/v_src: the chunk's cached pre-RoPE rows of this layer, [n][H][D].
 * k_rec/v_rec: recomputed pre-RoPE rows, [k][H][D], in the order of sel.
 * sel: ascending local indices of the recomputation set (k of them).
 * Rows not in sel come from the cache (the reuse complement); rows in sel come
 * from the recomputation buffer.  Every key is rotated at its global position. */
void orc_assemble_chunk(const void* k_src, const void* v_src, const void* k_rec,
                        const void* v_rec, const int* sel, int n, int k,
                        int offset, int H, int D, int dtype, double theta,
                        int style, void* k_out, void* v_out) {
  char* in_sel = calloc(n > 0 ? n : 1, 1);
  int* sel_pos = malloc(sizeof(int) * (n > 0 ? n : 1));
  for (int t = 0; t < k; ++t) {
    in_sel[sel[t]] = 1;
    sel_pos[sel[t]] = t;
  }
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i) {
    if (in_sel[i])
      put_row(k_rec, v_rec, (size_t)sel_pos[i], H, D, dtype, theta, style,
              offset + i, k_out, v_out);
    else
      put_row(k_src, v_src, (size_t)i, H, D, dtype, theta, style, offset + i,
              k_out, v_out);
  }
  free(in_sel);
  free(sel_pos);
}

/* Uncached rows (e.g. the new query suffix) at positions start .. start+n-1. */
void orc_assemble_rows(const void* k_rows, const void* v_rows, int n, int start,
                       int H, int D, int dtype, double theta, int style,
                       void* k_out, void* v_out) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; ++i)
    put_row(k_rows, v_rows, (size_t)i, H, D, dtype, theta, style, start + i,
            k_out, v_out);
}

/* ---- selected-query causal attention (Sec. 4.1, App. B.2) ---- */

/* For each requested query row r (rows[t], t < n_rows) at global position
 * qpos[r] and each query head h: q = RoPE(q_pre[r][h], qpos[r]) rounded once
 * to the storage type (the stored rotated query); kv head
 * floor(h * H / Hq); logits z_t = scale * <q, k_t> over keys t <= qpos[r];
 * out = sum softmax(z)_t v_t.  k/v are the assembled (already rotated) [T][H][D]
 * buffers in storage dtype.  out: [n_rows][Hq][D] fp64; lse: [n_rows][Hq] fp64
 * (natural-log sum of exp of the logits), may be NULL. */
int orc_attention(const void* q_pre, const int* qpos, int Hq, const void* k,
                  const void* v, int T, int H, int D, int dtype, double scale,
                  double theta, int style, const int* rows, int n_rows,
                  double* out, double* lse) {
  if (H < 1 || Hq % H != 0) return -1;
  int group = Hq / H;
#pragma omp parallel
  {
    double* x = malloc(sizeof(double) * D);
    double* q = malloc(sizeof(double) * D);
    double* z = malloc(sizeof(double) * (T > 0 ? T : 1));
    double* acc = malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (long long w = 0; w < (long long)n_rows * Hq; ++w) {
      int t = (int)(w / Hq), h = (int)(w % Hq);
      int r = rows[t];
      int p = qpos[r];
      int kvh = h / group;
      for (int d = 0; d < D; ++d)
        x[d] = load_elem(q_pre, dtype, ((size_t)r * Hq + h) * D + d);
      orc_rope(x, D, (double)p, theta, style, q);
      /* The recomputed query is stored rotated, like a rotated key (App. B.3):
       * one rounding to the storage type before the products. */
      for (int d = 0; d < D; ++d) q[d] = round_to_storage(q[d], dtype);
      int nk = p + 1;
      if (nk > T) nk = T;
      double mx = -INFINITY;
      for (int j = 0; j < nk; ++j) {
        double dot = 0.0;
        size_t ko = ((size_t)j * H + kvh) * D;
        for (int d = 0; d < D; ++d) dot += q[d] * load_elem(k, dtype, ko + d);
        z[j] = scale * dot;
        if (z[j] > mx) mx = z[j];
      }
      double den = 0.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int j = 0; j < nk; ++j) {
        double e = exp(z[j] - mx);
        den += e;
        size_t vo = ((size_t)j * H + kvh) * D;
        for (int d = 0; d < D; ++d) acc[d] += e * load_elem(v, dtype, vo + d);
      }
      for (int d = 0; d < D; ++d)
        out[((size_t)t * Hq + h) * D + d] = (nk > 0) ? acc[d] / den : 0.0;
      if (lse) lse[(size_t)t * Hq + h] = (nk > 0) ? mx + log(den) : -INFINITY;
    }
    free(x); free(q); free(z); free(acc);
  }
  return 0;
}

/* ---- scoring without the frequency analysis (§5.4 "L2-norm selection") ----
 * The same joint K/V magnitudes, per-layer normalisation and layer mean as
 * orc_score_chunk, on the stored K and V themselves: a = ||K_l[n]||_2 over the
 * H*D channels, b = ||V_l[n]||_2, s = a/2 + b/2. */
int orc_score_l2(const void* K, const void* V, int dtype, int L, int N, int H, int D, int norm,
                 double* layer_score, double* score) {
  if (L < 1 || N < 1 || H < 1 || D < 1) return -1;
  int C = H * D;
  double* sl = malloc(sizeof(double) * N);
  for (int n = 0; n < N; ++n) score[n] = 0.0;
  for (int l = 0; l < L; ++l) {
    for (int n = 0; n < N; ++n) {
      size_t base = ((size_t)l * N + n) * C;
      double ek = 0.0, ev = 0.0;
      for (int ch = 0; ch < C; ++ch) {
        double k = load_elem(K, dtype, base + ch), v = load_elem(V, dtype, base + ch);
        ek += k * k;
        ev += v * v;
      }
      sl[n] = 0.5 * sqrt(ek) + 0.5 * sqrt(ev);
    }
    normalise(sl, N, norm);
    if (layer_score) memcpy(layer_score + (size_t)l * N, sl, sizeof(double) * N);
    for (int n = 0; n < N; ++n) score[n] += sl[n];
  }
  for (int n = 0; n < N; ++n) score[n] /= (double)L;
  free(sl);
  return 0;
}

/* ---- high-frequency-guided selection (Sec. 5.4, Table 3, Figure 1) ---- */

/* Inverse real transform with output length n_len (irfft(n=n_len) convention,
 * as inverse_lowpass) of the bins j in [j0, nb) alone: every bin below the
 * cutoff j0 is treated as zero. */
static void inverse_highband(const double* re, const double* im, int n_len, int j0, int nb,
                             const double* c, const double* s, double* out) {
  for (int n = 0; n < n_len; ++n) {
    double acc = 0.0;
    int m = (int)(((long long)j0 * n) % n_len); /* (j * n) mod n_len, advanced exactly */
    for (int j = j0; j < nb; ++j) {
      int edge = (j == 0) || ((n_len % 2 == 0) && j == n_len / 2);
      double term = re[j] * c[m];
      if (!edge) term = 2.0 * (term - im[j] * s[m]);
      acc += term;
      m += n;
      if (m >= n_len) m -= n_len;
    }
    out[n] = acc / (double)n_len;
  }
}

/* High-frequency reconstruction of one real sequence of n tokens: rFFT over
 * the transform length, keep the bins at and above the low-pass cutoff (the
 * bins the low-pass view discards), inverse transform, positions [0, n). */
void orc_highpass(const double* x, int n, int a_num, int a_den, int fftlen_mode, double* out) {
  int nf = orc_fft_len(n, fftlen_mode);
  int nb = orc_nbins(nf);
  int kk = orc_kkeep(nb, a_num, a_den);
  double* c = malloc(sizeof(double) * nf);
  double* s = malloc(sizeof(double) * nf);
  double* xp = calloc(nf, sizeof(double));
  double* re = malloc(sizeof(double) * nb);
  double* im = malloc(sizeof(double) * nb);
  double* rec = malloc(sizeof(double) * nf);
  memcpy(xp, x, sizeof(double) * n);
  trig_table(nf, c, s);
  dft_bins(xp, nf, nb, c, s, re, im);
  inverse_highband(re, im, nf, kk, nb, c, s, rec);
  memcpy(out, rec, sizeof(double) * n);
  free(c); free(s); free(xp); free(re); free(im); free(rec);
}

/* Importance score of the high-frequency-guided strategy the pages compare
 * against: the same joint K/V magnitudes, per-layer normalisation and layer
 * mean as orc_score_chunk, taken of the high-frequency reconstruction (bins
 * at and above the cutoff kk) instead of the low-frequency one.  Reading: the
 * cutoff is the low-pass one for the same alpha, so the two views split the
 * spectrum between them. */
int orc_score_highpass(const void* K, const void* V, int dtype, int L, int N, int H, int D,
                       int a_num, int a_den, int fftlen_mode, int norm, double* layer_score,
                       double* score) {
  if (L < 1 || N < 1 || H < 1 || D < 1 || a_den <= 0 || a_num <= 0) return -1;
  int C = H * D;
  int nf = orc_fft_len(N, fftlen_mode);
  int nb = orc_nbins(nf);
  int kk = orc_kkeep(nb, a_num, a_den);
  double* c = malloc(sizeof(double) * nf);
  double* s = malloc(sizeof(double) * nf);
  trig_table(nf, c, s);
  double* mag[2];
  mag[0] = malloc(sizeof(double) * N);
  mag[1] = malloc(sizeof(double) * N);
  double* sl = malloc(sizeof(double) * N);
  double* rec = malloc(sizeof(double) * (size_t)C * N);
  for (int n = 0; n < N; ++n) score[n] = 0.0;
  for (int l = 0; l < L; ++l) {
    size_t off = (size_t)l * N * C;
    for (int t = 0; t < 2; ++t) {
      const void* x = t ? V : K;
#pragma omp parallel
      {
        double* seq = calloc(nf, sizeof(double));
        double* re = malloc(sizeof(double) * nb);
        double* im = malloc(sizeof(double) * nb);
        double* out = malloc(sizeof(double) * nf);
#pragma omp for schedule(static)
        for (int ch = 0; ch < C; ++ch) {
          for (int n = 0; n < N; ++n) seq[n] = load_elem(x, dtype, off + (size_t)n * C + ch);
          dft_bins(seq, nf, nb, c, s, re, im);
          inverse_highband(re, im, nf, kk, nb, c, s, out);
          memcpy(rec + (size_t)ch * N, out, sizeof(double) * N);
        }
        free(seq); free(re); free(im); free(out);
      }
      for (int n = 0; n < N; ++n) {
        double e = 0.0;
        for (int ch = 0; ch < C; ++ch) {
          double v = rec[(size_t)ch * N + n];
          e += v * v;
        }
        mag[t][n] = sqrt(e);
      }
    }
    for (int n = 0; n < N; ++n) sl[n] = 0.5 * mag[0][n] + 0.5 * mag[1][n];
    normalise(sl, N, norm);
    if (layer_score) memcpy(layer_score + (size_t)l * N, sl, sizeof(double) * N);
    for (int n = 0; n < N; ++n) score[n] += sl[n];
  }
  for (int n = 0; n < N; ++n) score[n] /= (double)L;
  free(c); free(s); free(mag[0]); free(mag[1]); free(sl); free(rec);
  return 0;
}

/* ---- frequency-band energy fractions (App. E.1, Figure 9) ---- */

/* Energy of one real tensor X ([L][N][H][D], storage dtype) per band of rFFT
 * bins, taken along the tokens of each channel and summed over the H*D
 * channels.  Bin j of a length-nf transform carries w_j |X_j|^2 / nf with w_j
 * = 1 at DC and Nyquist, else 2 (the two-sided spectrum folded; by Parseval
 * the bins sum to the energy of the sequence).  Reading: "bands" are n_bands
 * equal parts of the bin range [0, nb), bin j in band floor(j * n_bands / nb).
 * fraction [L][n_bands] = band energy / total; total [L] (may be NULL).
 * Returns 0, or -1 on bad arguments (n_bands outside [1, nb]). */
int orc_band_energy(const void* X, int dtype, int L, int N, int H, int D, int fftlen_mode,
                    int n_bands, double* fraction, double* total) {
  if (L < 1 || N < 1 || H < 1 || D < 1) return -1;
  int C = H * D;
  int nf = orc_fft_len(N, fftlen_mode);
  int nb = orc_nbins(nf);
  if (n_bands < 1 || n_bands > nb) return -1;
  double* c = malloc(sizeof(double) * nf);
  double* s = malloc(sizeof(double) * nf);
  trig_table(nf, c, s);
  double* ebin = malloc(sizeof(double) * (size_t)C * nb); /* [channel][bin] */
  for (int l = 0; l < L; ++l) {
    size_t off = (size_t)l * N * C;
#pragma omp parallel
    {
      double* seq = calloc(nf, sizeof(double));
      double* re = malloc(sizeof(double) * nb);
      double* im = malloc(sizeof(double) * nb);
#pragma omp for schedule(static)
      for (int ch = 0; ch < C; ++ch) {
        for (int n = 0; n < N; ++n) seq[n] = load_elem(X, dtype, off + (size_t)n * C + ch);
        dft_bins(seq, nf, nb, c, s, re, im);
        for (int j = 0; j < nb; ++j) {
          int edge = (j == 0) || ((nf % 2 == 0) && j == nf / 2);
          ebin[(size_t)ch * nb + j] = (edge ? 1.0 : 2.0) * (re[j] * re[j] + im[j] * im[j]) / nf;
        }
      }
      free(seq); free(re); free(im);
    }
    double* fr = fraction + (size_t)l * n_bands;
    for (int b = 0; b < n_bands; ++b) fr[b] = 0.0;
    double tot = 0.0;
    for (int j = 0; j < nb; ++j) {
      double e = 0.0;
      for (int ch = 0; ch < C; ++ch) e += ebin[(size_t)ch * nb + j];
      fr[(int)(((long long)j * n_bands) / nb)] += e;
      tot += e;
    }
    for (int b = 0; b < n_bands; ++b) fr[b] = tot > 0.0 ? fr[b] / tot : 0.0;
    if (total) total[l] = tot;
  }
  free(c); free(s); free(ebin);
  return 0;
}

/* ---- storage rounding of whole arrays (used by the layer oracle) ---- */

/* out[i] = bf16 bit pattern of v[i], rounded to nearest even (orc_round_bf16). */
void orc_round_bf16_array(const double* v, long long n, uint16_t* out) {
  for (long long i = 0; i < n; ++i) out[i] = orc_round_bf16(v[i]);
}

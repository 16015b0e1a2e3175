// Chunk scoring on gfx950 -- "Adaptive KV Cache Reuse for Fast Long-Context
// LLM Serving" (CacheTune), App. B.1 "Offline Preparation".
//
// For every (chunk, layer, K|V) problem with channels c = (head, dim) and
// tokens n < N, the low-frequency energy per token
//     E[n] = sum_c xlow_c[n]^2,
//     xlow_c = inverse real DFT (length nf) of the lowest kk bins of x_c,
// is computed exactly (up to rounding) without forming xlow:
//  1. band projection on the matrix cores: Y = [cos | sin](j*n) . X, i.e. the
//     real and imaginary parts R_j, S_j (j < kk) of the retained bins for all
//     channels at once.  For bf16 data the transform is folded on its
//     real-input symmetry (tokens n and nf - n share their twiddles, up to the
//     sine's sign), so the cosine rows take x[n] + x[nf-n] and the sine rows
//     x[n] - x[nf-n] over half the tokens.  Those sums enter the fp16 matrix
//     cores as an exact fp16 hi + lo pair, against the twiddles as an fp16
//     hi + lo pair (t = t1 + t2 to 2^-24): three MFMAs give fp32-accurate
//     coefficients.  A tile whose sums leave fp16's range, or that meets a
//     non-finite value, is redone at once unfolded, with the twiddles as three
//     bf16 planes (t1 + t2 + t3 to ~2^-25) against the bf16 data (three
//     MFMAs); fp32 data are split the same way (six MFMAs).
//  2. the channel Gram G = Y Y^T (fp64);
//  3. E[n] as a trigonometric polynomial of degree 2(kk-1) in phi = 2*pi*n/nf,
//     whose coefficients are diagonal and anti-diagonal sums of G; evaluated
//     in fp64 by Clenshaw's recurrence, once per token pair (n, nf - n).
//  4. per token a = sqrt(E_K), b = sqrt(E_V), s = a/2 + b/2, per-layer
//     normalisation, mean over layers (fp64, fixed-order reductions).
#include "ct_device.h"
#include "ct_internal.h"

namespace ct {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---- rounding helpers ----------------------------------------------------

__device__ inline uint32_t bf16_rne_from_f32_bits(uint32_t u) { return bf16_bits_rne(__uint_as_float(u)); }

__device__ inline double f64_from_bf16(uint16_t h) {
  return (double)__uint_as_float(((uint32_t)h) << 16);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round a double to fp16 with a single rounding (round-to-odd to binary32,
// then round to nearest even).
__device__ inline _Float16 f16_from_f64(double d) {
  float f = __double2float_rz(d);
  uint32_t u = __float_as_uint(f);
  if ((double)f != d) u |= 1u;
  return (_Float16)__uint_as_float(u);
}

__device__ inline uint32_t pack_f16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// cos and sin of 2*pi*m/nf (0 <= m < nf): quarter turns are taken out exactly
// so that multiples of pi/2 give exact 0 and +-1.
__device__ inline void turn_sincos(long long m, int nf, double* s, double* c) {
  long long t = 4 * m;
  long long q = t / nf;
  long long rem = t - q * nf;
  double a = 1.5707963267948966 * ((double)rem / (double)nf);
  double sa, ca;
  sincos(a, &sa, &ca);
  if (rem == 0) { sa = 0.0; ca = 1.0; }
  switch ((int)(q & 3)) {
    case 0: *c = ca;  *s = sa;  break;
    case 1: *c = -sa; *s = ca;  break;
    case 2: *c = -ca; *s = -sa; break;
    default: *c = sa; *s = -ca; break;
  }
}

// ---- 1a. twiddle planes ----------------------------------------------------
// Row p < kk holds cos(2*pi*p*n/nf); row kk + j holds sin(2*pi*j*n/nf);
// rows >= 2kk are zero.  Each value is stored as three bf16 planes and as an
// fp16 pair (both are always written, so a table serves bf16 and fp32 data).
__global__ __launch_bounds__(256) void k_twiddle(ScoreLaunch sl) {
  const ScoreChunkDesc& d = sl.c[blockIdx.y];
  if (!d.tw_owner) return;
  const int ppad = d.ppad, ntp = d.ntok_pad, kk = d.kk, nf = d.nf;
  uint16_t* tw = d.tw;
  _Float16* tw16 = reinterpret_cast<_Float16*>(d.tw16);
  const long long plane = (long long)ppad * ntp;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < plane;
       e += (long long)gridDim.x * blockDim.x) {
    int p = (int)(e / ntp), n = (int)(e % ntp);
    double v = 0.0;
    if (p < 2 * kk) {
      int j = p < kk ? p : p - kk;
      double s, c;
      turn_sincos(((long long)j * n) % nf, nf, &s, &c);
      v = p < kk ? c : s;
    }
    uint16_t t1 = bf16_from_f64(v);
    double r1 = v - f64_from_bf16(t1);
    uint16_t t2 = bf16_from_f64(r1);
    double r2 = r1 - f64_from_bf16(t2);
    uint16_t t3 = bf16_from_f64(r2);
    tw[e] = t1;
    tw[plane + e] = t2;
    tw[2 * plane + e] = t3;
    const _Float16 h1 = f16_from_f64(v);
    tw16[e] = h1;
    tw16[plane + e] = f16_from_f64(v - (double)h1);
  }
  double2* trig = d.trig;
  for (long long m = (long long)blockIdx.x * blockDim.x + threadIdx.x; m < nf;
       m += (long long)gridDim.x * blockDim.x) {
    double s, c;
    turn_sincos(m, nf, &s, &c);
    trig[m] = make_double2(c, s);
  }
}

// ---- 1b. band projection on the matrix cores --------------------------------
// Block: 256 threads = 4 waves; one (chunk, layer, K|V) problem, 128 band rows,
// 256 channels (64 per wave).  Per 32-token step the three twiddle planes of
// the 128 rows are staged in LDS (row stride 40 bf16 = 80 B, conflict-free for
// 16-byte fragment reads); each lane loads its 2 channels for 8 tokens directly
// from HBM and transposes them in registers into MFMA B fragments.
//   v_mfma_f32_32x32x16_bf16:  D[i][j] += sum_k A[i][k] B[k][j]
//   A (band rows x tokens): lane -> row lane%32, tokens 8*(lane/32) + 0..7
//   B (tokens x channels):  lane -> col lane%32, same tokens
//   D: lane -> col lane%32, rows 8*(v/4) + 4*(lane/32) + v%4, v < 16
// Channel of column j in B tile m (m = 0, 1): base + 2j + m.
constexpr int kTwStride = 40;

template <int DT>
__global__ __launch_bounds__(256) void k_band_fwd(ScoreLaunch sl, char* ws) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * 128 * kTwStride];

  const int L = sl.L, C = sl.C;
  const int prob = blockIdx.z;
  const int b = prob / (2 * L);
  const int layer = (prob / 2) % L;
  const int kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int pbase = blockIdx.y * 128;
  if (pbase >= d.ppad) return;
  const int ntiles = min(4, (d.ppad - pbase) / 32);
  const int N = d.n, ntp = d.ntok_pad, ppad = d.ppad;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const int cbase = blockIdx.x * 256 + wave * 64;
  const bool active = cbase < C;
  const int c0 = cbase + 2 * col;

  const uint16_t* tw = d.tw;
  const long long plane = (long long)ppad * ntp;
  const char* src = reinterpret_cast<const char*>(kv ? d.v : d.k);
  const size_t esz = DT == CT_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)C * esz;
  const char* xbase = src + ((size_t)layer * N) * row_bytes + (size_t)c0 * esz;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][m][v] = 0.f;

  for (int n0 = 0; n0 < N; n0 += 32) {
    // stage the twiddle slab: 3 planes x 128 rows x 32 tokens
    for (int item = tid; item < 3 * 128 * 4; item += 256) {
      int q = item / 512, r = (item / 4) % 128, i = item % 4;
      if (r < ntiles * 32) {
        const u32x4_t* gsrc = reinterpret_cast<const u32x4_t*>(
            tw + q * plane + (long long)(pbase + r) * ntp + n0 + 8 * i);
        *reinterpret_cast<u32x4_t*>(&lds[(q * 128 + r) * kTwStride + 8 * i]) = *gsrc;
      }
    }
    // this lane's data: 2 k-steps x 8 tokens x 2 channels
    uint32_t wb[2][8];
    float2 wf[2][8];
    if (active) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          int n = n0 + 16 * s + 8 * g + t;
          if constexpr (DT == CT_BF16) {
            wb[s][t] = n < N ? *reinterpret_cast<const uint32_t*>(xbase + (size_t)n * row_bytes) : 0u;
          } else {
            wf[s][t] = n < N ? *reinterpret_cast<const float2*>(xbase + (size_t)n * row_bytes)
                             : make_float2(0.f, 0.f);
          }
        }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t a[4][3];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          if (pt < ntiles)
#pragma unroll
            for (int q = 0; q < 3; ++q)
              a[pt][q] = *reinterpret_cast<const bf16x8_t*>(
                  &lds[(q * 128 + pt * 32 + col) * kTwStride + 16 * s + 8 * g]);
        if constexpr (DT == CT_BF16) {
          u32x4_t bu[2];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            uint32_t w0 = wb[s][2 * h], w1 = wb[s][2 * h + 1];
            bu[0][h] = (w0 & 0xffffu) | (w1 << 16);
            bu[1][h] = (w0 >> 16) | (w1 & 0xffff0000u);
          }
          bf16x8_t bfr[2] = {__builtin_bit_cast(bf16x8_t, bu[0]), __builtin_bit_cast(bf16x8_t, bu[1])};
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
            if (pt < ntiles)
#pragma unroll
              for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int q = 0; q < 3; ++q)
                  acc[pt][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pt][q], bfr[m], acc[pt][m], 0, 0, 0);
        } else {
          // exact three-way bf16 split of each fp32 value
          u32x4_t bu[3][2];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            uint32_t lo[3][2], hi[3][2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              float2 v2 = wf[s][2 * h + e];
#pragma unroll
              for (int m = 0; m < 2; ++m) {
                float x = m ? v2.y : v2.x;
                uint32_t p1 = bf16_rne_from_f32_bits(__float_as_uint(x));
                float r1 = x - __uint_as_float(p1 << 16);
                uint32_t p2 = bf16_rne_from_f32_bits(__float_as_uint(r1));
                float r2 = r1 - __uint_as_float(p2 << 16);
                uint32_t p3 = bf16_rne_from_f32_bits(__float_as_uint(r2));
                uint32_t parts[3] = {p1, p2, p3};
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) {
                  if (e == 0) lo[pl][m] = parts[pl];
                  else hi[pl][m] = parts[pl];
                }
              }
            }
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
#pragma unroll
              for (int m = 0; m < 2; ++m) bu[pl][m][h] = lo[pl][m] | (hi[pl][m] << 16);
          }
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
            if (pt < ntiles)
#pragma unroll
              for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
#pragma unroll
                  for (int q = 0; q < 3; ++q)
                    if (pl + q <= 2)
                      acc[pt][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                          a[pt][q], __builtin_bit_cast(bf16x8_t, bu[pl][m]), acc[pt][m], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (!active) return;
  float* Y = reinterpret_cast<float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    if (pt >= ntiles) break;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int row = pbase + pt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      *reinterpret_cast<float2*>(Y + (size_t)row * C + c0) = make_float2(acc[pt][0][v], acc[pt][1][v]);
    }
  }
}

// Energy per token from the Gram of one problem (NTH threads):
// coefficients of E * nf^2 = sum_k A_k cos(k phi) + B_k sin(k phi), k < 2kk-1.
// With weights w_j (1 for DC and the Nyquist bin, 2 otherwise) and
// RR = G[j][j'], SS = G[kk+j][kk+j'], RS = G[j][kk+j']:
//   alpha_d = sum_{j-j'=d} w w (RR+SS),  beta_s = sum_{j+j'=s} w w (RR-SS),
//   gamma_s = 2 sum_{j+j'=s} w w RS,     delta_d = 2 sum_{j-j'=d} w w RS,
//   A_0 = (alpha_0 + beta_0)/2,  A_k = (2 alpha_k + beta_k)/2,
//   B_k = (gamma_k - delta_k + delta_{-k})/2.
// E is then evaluated in fp64 by Clenshaw's recurrence, once per token pair.
template <int NTH>
__device__ void poly_energy(const ScoreChunkDesc& d, int layer, int kv, const double* G, int ldg,
                            double* coef, char* ws) {
  const int tid = threadIdx.x;
  const int kk = d.kk, P2 = 2 * kk, nf = d.nf, N = d.n;
  const int K2 = 2 * kk - 1;
  const bool even = (nf % 2) == 0;
  // the five sums of coefficient k over j = j0, j0 + jstep, ... < kk
  struct Sums { double alpha, beta, gamma, dpos, dneg; };
  auto wt = [&](int j) { return (j == 0 || (even && 2 * j == nf)) ? 1.0 : 2.0; };
  auto sums = [&](int k, int j0, int jstep) {
    Sums t = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int j = j0; j < kk; j += jstep) {
      const double wj = wt(j);
      const int jp = j - k;  // j - j' = k
      if (jp >= 0) {
        const double w = wj * wt(jp);
        t.alpha += w * (G[(size_t)j * ldg + jp] + G[(size_t)(kk + j) * ldg + kk + jp]);
        t.dpos += w * G[(size_t)j * ldg + kk + jp];
      }
      const int jn = j + k;  // j - j' = -k
      if (k > 0 && jn < kk) t.dneg += wj * wt(jn) * G[(size_t)j * ldg + kk + jn];
      const int js = k - j;  // j + j' = k
      if (js >= 0 && js < kk) {
        const double w = wj * wt(js);
        t.beta += w * (G[(size_t)j * ldg + js] - G[(size_t)(kk + j) * ldg + kk + js]);
        t.gamma += w * G[(size_t)j * ldg + kk + js];
      }
    }
    return t;
  };
  auto store = [&](int k, const Sums& t) {
    coef[2 * k] = (k == 0) ? 0.5 * (t.alpha + t.beta) : 0.5 * ((k < kk ? 2.0 * t.alpha : 0.0) + t.beta);
    coef[2 * k + 1] =  // (interleaved: one 16-byte load per recurrence step)
        (k == 0) ? 0.0 : 0.5 * (2.0 * t.gamma - (k < kk ? 2.0 * (t.dpos - t.dneg) : 0.0));
  };
  if (8 * K2 <= NTH) {
    // 8 lanes per coefficient, each taking every 8th j; a fixed butterfly
    // combines their sums (deterministic)
    const int k = tid >> 3;
    Sums t = k < K2 ? sums(k, tid & 7, 8) : Sums{0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      t.alpha += __shfl_xor(t.alpha, o);
      t.beta += __shfl_xor(t.beta, o);
      t.gamma += __shfl_xor(t.gamma, o);
      t.dpos += __shfl_xor(t.dpos, o);
      t.dneg += __shfl_xor(t.dneg, o);
    }
    if ((tid & 7) == 0 && k < K2) store(k, t);
  } else {
    for (int k = tid; k < K2; k += NTH) store(k, sums(k, 0, 1));
  }
  __syncthreads();

  // E = U + V with U = sum_k A_k cos(k phi), V = sum_k B_k sin(k phi).  Tokens
  // m and nf - m share U and have opposite V, so each thread evaluates both
  // series once for a pair, by Clenshaw's recurrence for the cos/sin basis
  // (b_k = c_k + 2 cos(phi) b_{k+1} - b_{k+2}; U = A_0 + b_1 cos(phi) - b_2,
  // V = d_1 sin(phi)).  Token 0 (phi = 0) is the sum of the A_k, taken by
  // wave 0 in a fixed order.
  const double2* trig = d.trig;
  const double2* cf = reinterpret_cast<const double2*>(coef);  // {A_k, B_k}
  double* E = reinterpret_cast<double*>(ws + d.e_off) + (size_t)(layer * 2 + kv) * N;
  const double inv = 1.0 / ((double)nf * (double)nf);
  for (int m = tid + 1; m <= nf / 2; m += NTH) {
    const double2 z = trig[m];
    const double c2 = 2.0 * z.x;
    double u1 = 0.0, u2 = 0.0, v1 = 0.0, v2 = 0.0;  // b_{k+1}, b_{k+2} of U and of V
#pragma unroll 4
    for (int k = K2 - 1; k >= 1; --k) {
      const double2 ab = cf[k];
      const double u0 = fma(c2, u1, ab.x - u2);
      const double v0 = fma(c2, v1, ab.y - v2);
      u2 = u1;
      u1 = u0;
      v2 = v1;
      v1 = v0;
    }
    const double U = cf[0].x + u1 * z.x - u2, V = v1 * z.y;
    if (m < N) E[m] = (U + V) * inv;
    const int mp = nf - m;
    if (mp != m && mp < N) E[mp] = (U - V) * inv;
  }
  if (tid < 64) {
    double a0 = 0.0;
    for (int k = tid; k < K2; k += 64) a0 += cf[k].x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a0 += __shfl_xor(a0, o);
    if (tid == 0) E[0] = a0 * inv;
  }
}

// bf16 data: the same projection, software-pipelined.  X (the HBM stream) is
// loaded two 32-token steps ahead into registers; the twiddle slab of the
// next step is loaded one step ahead and written to the other of two LDS
// buffers after the current step's MFMAs, so each step has one barrier.  The
// step loop is unrolled by two so that both register and LDS buffers are
// compile-time, and its body has no conditional code: vector-memory loads
// complete in issue order, and a branch around a load or a compute block
// makes the compiler's wait counts at the loop head assume the worst path,
// which would hold each step until the next step's loads had landed.

// Rows of a band block.  A block of NTL = 2 * NC tiles of 32 rows serves the
// bins b0 .. b0 + 32 NC - 1 (b0 = rblk * 32 NC): tile pt < NC holds their
// cosine rows and tile NC + pt their sine rows, so that no tile mixes the two
// kinds.  The table (and Y) row of bin b is b for the cosine and kk + b for
// the sine; bins at or past kk have none.
template <int NC>
__device__ inline int band_table_row(int r, int b0, int kk) {
  const int pt = r >> 5, bin = b0 + 32 * (pt % NC) + (r & 31);
  if (bin >= kk) return -1;
  return pt < NC ? bin : kk + bin;
}
// Y row a tile row is stored to: as above, and a sine tile's rows past the
// last bin fill the padding rows 2kk .. ppad - 1 (with zeros: their twiddle
// rows read zeros); -1 for rows stored nowhere.
template <int NC>
__device__ inline int band_y_row(int pt, int rt, int b0, int kk, int ppad) {
  const int bin = b0 + 32 * (pt % NC) + rt;
  if (pt < NC) return bin < kk ? bin : -1;
  return kk + bin < ppad ? kk + bin : -1;
}

// LDS of a band block: two buffers of the twiddle slab of one step (F16: the
// fp16 pair, else the three bf16 planes), rows 80 bytes apart.
template <int NTL, bool F16>
struct BandLds {
  static constexpr int kPlanes = F16 ? 2 : 3;  // twiddle planes
  uint16_t buf[2][kPlanes * 32 * NTL * kTwStride];
};

// x = hi + lo with hi the round-to-nearest-even fp16 of x and lo the fp16 of
// the remainder.  For x the fp32 sum or difference of two bf16 values the
// split is exact (unless the remainder falls below fp16's normal range, 2^-14,
// where it is rounded by at most 2^-25): when the two do not nearly cancel,
// the larger one's 8 significant bits lie within hi's 11, so the remainder is
// made of the smaller one's bits; hi is rounded up only when the smaller one
// reaches half of hi's last place, and then the remainder spans at most 9
// bits.  (Nearly cancelling operands leave at most 10 bits, all in hi.)
// |lo| <= 2^-11 |x|.  |x| >= 65520, or a non-finite x, gives a non-finite hi.
// The remainders are formed by the mixed-precision FMA, x - 1.0 * hi with hi
// read as fp16 from its half of the packed register (one instruction each,
// exact: the difference is representable in fp32).
__device__ inline uint2 split_f16(float a, float b) {
  const uint32_t h = pack_f16(a, b);
  float ra, rb;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(h), "v"(a));
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(h), "v"(b));
  return make_uint2(h, pack_f16(ra, rb));
}

// One 512-channel x (32 * 2NC)-row tile (channel block cblk, bin block rblk)
// of problem prob, by the 512 threads of the calling block, fp16 pass.
// The real-input symmetry of the transform halves its length: for 0 < n <
// nf/2 the twiddles of tokens n and nf - n are equal (cosine) and opposite
// (sine), so
//   R_j = x[0] + sum_{0<n<nf/2} cos(2 pi j n/nf) (x[n] + x[nf-n]) [+ (-1)^j x[nf/2]],
//   S_j =        sum_{0<n<nf/2} sin(2 pi j n/nf) (x[n] - x[nf-n]),
// the bracket for even nf (tokens past N are zeros).  u = x[n] + x[nf-n] and
// v = x[n] - x[nf-n] are formed in fp32 from the bf16 data and split exactly
// into fp16 hi + lo; against the twiddle pair t = t1 + t2 the products
// t1*hi + t2*hi + t1*lo (three MFMAs per tile and k-step, on half the
// tokens) leave out t2*lo, below 2^-23 |u|.  The nf/2 term is added in fp32
// after the loop.  Returns together on every thread (every condition below
// is uniform over the block): true when a tile met a value outside fp16's
// range (|u| or |v| >= 65520, or non-finite data), without writing Y.
template <int NC>
__device__ __forceinline__ bool band_fold(const ScoreLaunch& sl, char* ws, int cblk, int rblk, int prob,
                                          BandLds<2 * NC, true>& sh) {
  constexpr int NTL = 2 * NC, NPL = 2;
  auto& lds = sh.buf;

  const int L = sl.L, C = sl.C;
  const int b = prob / (2 * L);
  const int layer = (prob / 2) % L;
  const int kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int kk = d.kk, b0 = rblk * 32 * NC;
  if (b0 >= kk) return false;
  const int N = d.n, nf = d.nf, ntp = d.ntok_pad, ppad = d.ppad;
  const int nh = (nf + 1) / 2;      // folded columns n = 0 .. nh - 1
  const int nsteps = (nh + 31) / 32;
  const int m0 = nf - nh + 1;       // first mirrored token
  const int nfwd = min(nh, N), nmir = max(0, N - m0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const int cbase = cblk * 512 + wave * 64;
  const bool active = cbase < C;
  const int c0 = cbase + 2 * col;

  // Buffer resources (gfx9 word 3): a load whose VGPR offset is at or past
  // num_records returns 0.  fres covers the tokens n < nh (and < N) and mres
  // the mirrored tokens m0 .. N - 1, so every folded column at or past nh,
  // and the mirror of column 0 (token nf), reads zeros on both sides.  The
  // whole offset is kept in the VGPR operand (the scalar offset is 0), so the
  // range check covers every load; a mirrored offset that would be negative
  // is clamped to the end of the range.
  const uint16_t* tw = d.tw16;
  const long long plane = (long long)ppad * ntp;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(kv ? d.v : d.k) + (size_t)layer * N * C;
  const __amdgpu_buffer_rsrc_t fres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src), 0, nfwd * C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t mres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src + (size_t)min(m0, N) * C), 0, nmir * C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(tw), 0, (int)(NPL * plane * 2), 0x00020000);
  const int fvoff = active ? (c0 + 8 * g * C) * 2 : nfwd * C * 2;
  // mirror of column n: token nf - n, at (nh - 1 - n) tokens into mres.  An
  // inactive wave's offsets stay past the range for every column the loop
  // loads (n < 32 * nsteps + 96 <= nh + 127).
  const int mvoff = active ? ((nh - 1 - 8 * g) * C + c0) * 2 : (nmir + nh + 128) * C * 2;
  const uint32_t mend = (uint32_t)(nmir * C * 2);

  f32x16_t acc[NTL][2];
#pragma unroll
  for (int i = 0; i < NTL; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][m][v] = 0.f;

  // X of a step: 2 k-steps x 8 columns x (2 channels in one dword), the
  // columns' own tokens (xf) and their mirrors (xm)
  uint32_t xfa[16], xma[16], xfb[16], xmb[16];
  // columns t0 .. t1 - 1 of k-step s2 of a step
  auto load_x_part = [&](int step, uint32_t* xf, uint32_t* xm, int s2, int t0, int t1) {
#pragma unroll
    for (int t = t0; t < t1; ++t) {
      const int k = (step * 32 + 16 * s2 + t) * C * 2;
      xf[8 * s2 + t] = __builtin_amdgcn_raw_buffer_load_b32(fres, fvoff + k, 0, 0);
      xm[8 * s2 + t] = __builtin_amdgcn_raw_buffer_load_b32(mres, (int)min((uint32_t)(mvoff - k), mend), 0, 0);
    }
  };
  auto load_x = [&](int step, uint32_t* xf, uint32_t* xm) {
    load_x_part(step, xf, xm, 0, 0, 8);
    load_x_part(step, xf, xm, 1, 0, 8);
  };
  // twiddle slab of a step: NPL planes x 32*NTL rows x 32 columns (16-byte chunks)
  constexpr int TWN = NPL * 32 * NTL * 4;  // chunks per slab
  constexpr int TWI = (TWN + 511) / 512;   // chunks per thread (the last may be partial)
  u32x4_t twr[TWI];
  int twoff[TWI];
#pragma unroll
  for (int it = 0; it < TWI; ++it) {
    const int item = tid + 512 * it;
    const int q = item / (128 * NTL), r = (item / 4) % (32 * NTL), i = item % 4;
    const int trow = band_table_row<NC>(r, b0, kk);
    // rows without a bin read past the table (zeros)
    twoff[it] = (item < TWN && trow >= 0) ? (int)((q * plane + (long long)trow * ntp + 8 * i) * 2)
                                          : (int)(NPL * plane * 2);
  }
  auto load_tw = [&](int step) {
#pragma unroll
    for (int it = 0; it < TWI; ++it)
      twr[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(tres, twoff[it] + step * 64, 0, 0));
  };
  auto store_tw = [&](uint16_t* buf) {
#pragma unroll
    for (int it = 0; it < TWI; ++it) {
      const int item = tid + 512 * it;
      if (TWN % 512 != 0 && item >= TWN) break;
      const int q = item / (128 * NTL), r = (item / 4) % (32 * NTL), i = item % 4;
      *reinterpret_cast<u32x4_t*>(&buf[(q * 32 * NTL + r) * kTwStride + 8 * i]) = twr[it];
    }
  };
  // the three products of one tile and k-step against the B pair (hi, lo) of
  // both channel halves
  auto tile3 = [&](const uint16_t* buf, int pt, int s2, const u32x4_t* hi, const u32x4_t* lo) {
    const uint16_t* ap = &buf[(pt * 32 + col) * kTwStride + 16 * s2 + 8 * g];
    const f16x8_t a1 = *reinterpret_cast<const f16x8_t*>(ap);
    const f16x8_t a2 = *reinterpret_cast<const f16x8_t*>(ap + 32 * NTL * kTwStride);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      acc[pt][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, __builtin_bit_cast(f16x8_t, hi[m]), acc[pt][m], 0, 0, 0);
      acc[pt][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a2, __builtin_bit_cast(f16x8_t, hi[m]), acc[pt][m], 0, 0, 0);
      acc[pt][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, __builtin_bit_cast(f16x8_t, lo[m]), acc[pt][m], 0, 0, 0);
    }
  };
  // one step; the loads of X for step sn go into xf and xm as their values
  // are used up (k-step s2's columns, during its products), so the loads of a
  // block's waves do not all reach the memory pipeline at once
  auto compute = [&](const uint16_t* buf, uint32_t* xf, uint32_t* xm, int sn) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      // B fragments: column pairs (2h, 2h+1) of channel half m, as the fp16
      // hi and lo of u = x[n] + x[nf-n] and v = x[n] - x[nf-n]
      u32x4_t uh[2], ul[2], vh[2], vl[2];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t f0 = xf[8 * s2 + 2 * h], f1 = xf[8 * s2 + 2 * h + 1];
        const uint32_t r0 = xm[8 * s2 + 2 * h], r1 = xm[8 * s2 + 2 * h + 1];
        // bf16 -> fp32 is exact
        const float fa0 = __uint_as_float(f0 << 16), fa1 = __uint_as_float(f1 << 16);
        const float ra0 = __uint_as_float(r0 << 16), ra1 = __uint_as_float(r1 << 16);
        const float fb0 = __uint_as_float(f0 & 0xffff0000u), fb1 = __uint_as_float(f1 & 0xffff0000u);
        const float rb0 = __uint_as_float(r0 & 0xffff0000u), rb1 = __uint_as_float(r1 & 0xffff0000u);
        const uint2 u0 = split_f16(fa0 + ra0, fa1 + ra1), u1 = split_f16(fb0 + rb0, fb1 + rb1);
        const uint2 v0 = split_f16(fa0 - ra0, fa1 - ra1), v1 = split_f16(fb0 - rb0, fb1 - rb1);
        uh[0][h] = u0.x; ul[0][h] = u0.y; uh[1][h] = u1.x; ul[1][h] = u1.y;
        vh[0][h] = v0.x; vl[0][h] = v0.y; vh[1][h] = v1.x; vl[1][h] = v1.y;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pt = 0; pt < 2 * NC; ++pt) {
        if (pt < NC)
          tile3(buf, pt, s2, uh, ul);
        else
          tile3(buf, pt, s2, vh, vl);
        load_x_part(sn, xf, xm, s2, (8 * pt) / (2 * NC), (8 * (pt + 1)) / (2 * NC));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Loads of steps at or past nsteps read past the buffers' ranges and return
  // zeros, so the loop issues them without a test: a straight-line body with
  // one back edge lets every wait count only the loads of the step it needs.
  // A wave with no channels computes on zeros (its loads are all out of range).
  // The prologue leaves the loads in the order the loop body issues them
  // (X of this step, then the twiddles and X of the next), so the loop entry
  // needs no stricter waits than the back edge.
  load_tw(0);
  load_x(0, xfa, xma);
  store_tw(lds[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_tw(1);
  __builtin_amdgcn_sched_barrier(0);
  load_x(1, xfb, xmb);
  for (int step = 0; step < nsteps; step += 2) {
    // even step: LDS buffer 0, registers xfa/xma.  The next step's slab goes
    // to the other buffer first (its last reads came before the barrier),
    // then the twiddle load of the step after, ahead of X
    __syncthreads();
    store_tw(lds[1]);
    load_tw(step + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(lds[0], xfa, xma, step + 2);
    // odd step: LDS buffer 1, registers xfb/xmb (past the end when nsteps is
    // odd: zero operands leave the sums unchanged)
    __syncthreads();
    store_tw(lds[0]);
    load_tw(step + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(lds[1], xfb, xmb, step + 3);
  }

  // The range test costs nothing inside the loop: |u| >= 65520 becomes +-inf
  // in fp16 and a NaN stays NaN, and every product with it is non-finite (a
  // zero twiddle gives NaN), so every tile of the channel block of that kind
  // sees a non-finite sum; finite fp16 data cannot overflow the fp32 sums at
  // these lengths.  So a non-finite sum marks exactly the blocks that need the
  // bf16 pass.  (Inactive lanes hold zeros.)
  bool bad = false;
#pragma unroll
  for (int pt = 0; pt < NTL; ++pt)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) bad |= !(__builtin_fabsf(acc[pt][m][v]) < __builtin_inff());
  if (__syncthreads_or((int)bad)) return true;  // the caller redoes the tile in bf16
  if (!active) return false;

  // even nf: the column nf/2 pairs with itself, with cosine (-1)^j and sine 0.
  // A row's bin parity is its accumulator index's (b0 and the tile and group
  // offsets are even).
  if ((nf & 1) == 0 && nf / 2 < N) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src + (size_t)(nf / 2) * C + c0);
    const float xn[2] = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
#pragma unroll
    for (int pt = 0; pt < NC; ++pt)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[pt][m][v] += (v & 1) ? -xn[m] : xn[m];
  }
  float* Y = reinterpret_cast<float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
#pragma unroll
  for (int pt = 0; pt < NTL; ++pt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = band_y_row<NC>(pt, 8 * (v >> 2) + 4 * g + (v & 3), b0, kk, ppad);
      if (row >= 0) *reinterpret_cast<float2*>(Y + (size_t)row * C + c0) = make_float2(acc[pt][0][v], acc[pt][1][v]);
    }
  return false;
}

// Radix-4 form of the fp16 pass, for transform lengths nf divisible by 128
// (M = nf/4 a whole number of pairs of 16-column k-steps).  With n = q M + m (q < 4,
// m < M), W^{jn} = W^{jm} (-i)^{jq}, so bin j needs only the sums
//   y0 = (x0 + x2) + (x1 + x3),  y2 = (x0 + x2) - (x1 + x3),
//   a = x0 - x2,  b = x1 - x3      (xq = x[q M + m]),
// over M columns, against cos and sin of 2 pi j m / nf (the first M columns of
// the same table):
//   j = 0, 2 mod 4:  R = sum c y,          S = sum s y      (y = y0, y2)
//   j = 1 mod 4:     R = sum (c a - s b),  S = sum (s a + c b)
//   j = 3 mod 4:     R = sum (c a + s b),  S = sum (s a - c b).
// The block's 64 bins b0 .. b0 + 63 form four tiles by class k = j mod 4:
// rows i < 16 the cosine rows (R) of bins b0 + 4i + k, rows 16 + i their sine
// rows (S).  The b products of classes 1 and 3 take the tile's rows swapped
// (row i reads row i ^ 16), the sine half negated for class 1 and the cosine
// half for class 3 (a signed copy of those rows is kept in LDS).  Each sum enters as an fp16 hi + lo pair (hi the nearest
// fp16, lo the fp16 of the remainder: exact for a and b, the difference of two
// bf16 values; the four-term y0 and y2 are rounded in fp32 and their remainder
// can need more than fp16's 11 bits, which bounds the pair's error by 2^-22 of
// the sum plus 2^-23 of the four values' magnitudes), against the twiddle
// pair.  Six product groups of three MFMAs per channel half and k-step (class
// 0 with y0, 2 with y2, 1 and 3 with a and with b): 36 MFMAs per 64 tokens
// (48 folded, 64 unfolded).  Returns together on every thread: true when a
// tile met a value outside fp16's range (a sum reaching 65520 included).
__device__ __forceinline__ int band_r4_table_row(int r, int b0, int kk) {
  const int k = r >> 5, i = r & 31, bin = b0 + 4 * (i & 15) + k;
  if (bin >= kk) return -1;
  return i < 16 ? bin : kk + bin;
}
__device__ __forceinline__ bool band_r4(const ScoreLaunch& sl, char* ws, int cblk, int rblk, int prob,
                                        BandLds<4, true>& sh) {
  constexpr int NPL = 2, TS = 24;  // twiddle planes; LDS row stride of a 16-column slab
  static_assert((2 * 128 + 2 * 64) * TS <= 2 * 32 * 4 * kTwStride, "radix-4 slab exceeds an LDS buffer");
  uint16_t* lds0 = &sh.buf[0][0];
  uint16_t* lds1 = &sh.buf[1][0];

  const int L = sl.L, C = sl.C;
  const int b = prob / (2 * L);
  const int layer = (prob / 2) % L;
  const int kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int kk = d.kk, b0 = rblk * 64;
  if (b0 >= kk) return false;
  const int N = d.n, nf = d.nf, ntp = d.ntok_pad, ppad = d.ppad;
  const int M = nf / 4;
  const int nks = M / 16;  // k-steps of 16 columns (even)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const int cbase = cblk * 512 + wave * 64;
  const bool active = cbase < C;
  const int c0 = cbase + 2 * col;

  // X through a buffer resource over the chunk's N tokens: tokens q M + m at
  // or past N (zero padding) read zeros.  Offsets grow with q and m.
  const long long plane = (long long)ppad * ntp;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(kv ? d.v : d.k) + (size_t)layer * N * C;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src), 0, N * C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(d.tw16), 0, (int)(NPL * plane * 2), 0x00020000);
  const int xvoff = active ? (c0 + 8 * g * C) * 2 : N * C * 2;
  const int qstep = M * C * 2;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][m][v] = 0.f;

  // X of a k-step: 4 quarters x 8 columns x (2 channels in one dword)
  uint32_t xa[32], xb[32];
  // (the k-step's base offset passes through an empty asm, so that each
  // load's offset is formed when it is issued instead of being kept in a
  // register of its own across the loop)
  auto x_base = [&](int j) {
    int base = j < nks ? xvoff + j * 16 * C * 2 : N * C * 2;  // past the last k-step: no reads
    asm volatile("" : "+v"(base));
    return base;
  };
  // loads u0 .. u1 - 1 of a k-step's 32 (quarter u / 8, column u % 8)
  auto load_x_part = [&](int base, uint32_t* dst, int u0, int u1) {
#pragma unroll
    for (int u = u0; u < u1; ++u)
      dst[u] = __builtin_amdgcn_raw_buffer_load_b32(xres, base + (u >> 3) * qstep + (u & 7) * C * 2, 0, 0);
  };
  auto load_x = [&](int j, uint32_t* dst) { load_x_part(x_base(j), dst, 0, 32); };
  // twiddle slab of a k-step: 2 planes x 128 rows x 16 columns, one 16-byte
  // chunk per thread
  u32x4_t twr;
  int twoff;
  {
    const int q = tid >> 8, r = (tid >> 1) & 127, i = tid & 1;
    const int trow = band_r4_table_row(r, b0, kk);
    twoff = trow >= 0 ? (int)((q * plane + (long long)trow * ntp + 8 * i) * 2) : (int)(NPL * plane * 2);
  }
  auto load_tw = [&](int j) {
    const int off = j < nks ? twoff + j * 32 : (int)(NPL * plane * 2);  // past the last k-step: no reads
    twr = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(tres, off, 0, 0));
  };
  // The slab in LDS: rows 0 .. 127 of each plane as read from the table, then
  // 64 rows per plane for the b products of classes 1 and 3 (row 32 (k >> 1)
  // + i holds tile row i ^ 16 of class k, negated where the b product
  // subtracts it), written by the threads of those rows (whole waves).
  auto store_tw = [&](uint16_t* buf) {
    const int q = tid >> 8, r = (tid >> 1) & 127, i = tid & 1;
    *reinterpret_cast<u32x4_t*>(&buf[(q * 128 + r) * TS + 8 * i]) = twr;
    if (r & 32) {
      const int k = r >> 5, ii = r & 31;
      const uint32_t sgn = (k == 1 ? ii >= 16 : ii < 16) ? 0x80008000u : 0u;
      u32x4_t w = twr;
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] ^= sgn;
      *reinterpret_cast<u32x4_t*>(&buf[(256 + q * 64 + 32 * (k >> 1) + (ii ^ 16)) * TS + 8 * i]) = w;
    }
  };
  auto prod3 = [&](f32x16_t& ac, const f16x8_t& a1, const f16x8_t& a2, const u32x4_t& hi, const u32x4_t& lo) {
    ac = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, __builtin_bit_cast(f16x8_t, hi), ac, 0, 0, 0);
    ac = __builtin_amdgcn_mfma_f32_32x32x16_f16(a2, __builtin_bit_cast(f16x8_t, hi), ac, 0, 0, 0);
    ac = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, __builtin_bit_cast(f16x8_t, lo), ac, 0, 0, 0);
  };
  // twiddle fragments (hi and lo planes) of slab row `row`, planes `pstride`
  // rows apart
  auto frag_a = [&](const uint16_t* buf, int row, int pstride, f16x8_t& a1, f16x8_t& a2) {
    const uint16_t* ap = &buf[row * TS + 8 * g];
    a1 = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(ap));
    a2 = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(ap + pstride * TS));
  };
  // the quarters' values of column pair (2h, 2h+1) in channel half m (bf16 ->
  // fp32 is exact): v[q][e] = x[q M + column 2h + e]
  auto quarters = [&](const uint32_t* xs, int m, int h, float (*v)[2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w = xs[8 * q + 2 * h + e];
        v[q][e] = __uint_as_float(m == 0 ? w << 16 : w & 0xffff0000u);
      }
  };
  // the four data terms of channel half m (y0, y2, a, b), split in one pass
  // over the quarters' values
  auto split = [&](const uint32_t* xs, int m, u32x4_t* hi, u32x4_t* lo) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v[4][2];
      quarters(xs, m, h, v);
      float p[4][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float s02 = v[0][e] + v[2][e], s13 = v[1][e] + v[3][e];
        p[0][e] = s02 + s13;
        p[1][e] = s02 - s13;
        p[2][e] = v[0][e] - v[2][e];
        p[3][e] = v[1][e] - v[3][e];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint2 w = split_f16(p[t][0], p[t][1]);
        hi[t][h] = w.x;
        lo[t][h] = w.y;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // channel half m's 18 products in six groups (class 0 with y0, 2 with y2,
  // 1 and 3 with a and with b); after each group, a sixth of the loads of
  // X for k-step jn (nothing when dst is null)
  auto products = [&](const uint16_t* buf, int m, const u32x4_t* hi, const u32x4_t* lo, int jn, uint32_t* dst) {
    constexpr int row[6] = {0, 64, 32, 96, 256, 288}, ps[6] = {128, 128, 128, 128, 64, 64};
    constexpr int cls[6] = {0, 2, 1, 3, 1, 3}, term[6] = {0, 1, 2, 2, 3, 3};
    const int base = dst ? x_base(jn) : 0;
#pragma unroll
    for (int gi = 0; gi < 6; ++gi) {
      f16x8_t a1, a2;
      frag_a(buf, row[gi] + col, ps[gi], a1, a2);
      prod3(acc[cls[gi]][m], a1, a2, hi[term[gi]], lo[term[gi]]);
      if (dst) load_x_part(base, dst, (32 * gi) / 6, (32 * (gi + 1)) / 6);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // one k-step on the slab in buf and the X in xs; the loads of X for k-step
  // jn go into xs as its values are used up (during half 1's products), so
  // the loads of a block's waves do not all reach the memory pipeline at once
  auto compute = [&](const uint16_t* buf, uint32_t* xs, int jn) {
    u32x4_t hi[4], lo[4];
    split(xs, 0, hi, lo);
    products(buf, 0, hi, lo, 0, nullptr);
    split(xs, 1, hi, lo);
    products(buf, 1, hi, lo, jn, xs);
  };

  // software pipeline: X two k-steps ahead, the twiddle slab one ahead (each
  // k-step writes the next one's slab to the other LDS buffer, last read
  // before this k-step's barrier), one barrier per k-step, a straight-line
  // body (loads past the end read nothing)
  load_tw(0);
  load_x(0, xa);
  store_tw(lds0);
  __builtin_amdgcn_sched_barrier(0);
  load_tw(1);
  __builtin_amdgcn_sched_barrier(0);
  load_x(1, xb);
  for (int j = 0; j < nks; j += 2) {
    __syncthreads();
    store_tw(lds1);
    load_tw(j + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(lds0, xa, j + 2);
    __syncthreads();
    store_tw(lds0);
    load_tw(j + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(lds1, xb, j + 3);
  }

  bool bad = false;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) bad |= !(__builtin_fabsf(acc[pt][m][v]) < __builtin_inff());
  if (__syncthreads_or((int)bad)) return true;  // the caller redoes the tile in bf16
  if (!active) return false;
  float* Y = reinterpret_cast<float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * g + (v & 3), bin = b0 + 4 * (i & 15) + k;
      const int row = i < 16 ? (bin < kk ? bin : -1) : (kk + bin < ppad ? kk + bin : -1);
      if (row >= 0) *reinterpret_cast<float2*>(Y + (size_t)row * C + c0) = make_float2(acc[k][0][v], acc[k][1][v]);
    }
  return false;
}

// The same tile unfolded, over all tokens.  F16: X converted to fp16 in
// registers (exact below 65536) against the fp16 twiddle pair, two MFMAs per
// tile and k-step; returns true, without writing Y, when a tile met a value
// outside fp16's range (the same finiteness test as the folded pass).
// Otherwise X stays bf16 against the three bf16 planes (three MFMAs): every
// bf16 value enters exactly, whatever its range; returns false.
template <int NC, bool F16>
__device__ __forceinline__ bool band_unfolded(const ScoreLaunch& sl, char* ws, int cblk, int rblk, int prob,
                                              BandLds<2 * NC, F16>& sh) {
  constexpr int NTL = 2 * NC, NPL = F16 ? 2 : 3;
  auto& lds = sh.buf;

  const int L = sl.L, C = sl.C;
  const int b = prob / (2 * L);
  const int layer = (prob / 2) % L;
  const int kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int kk = d.kk, b0 = rblk * 32 * NC;
  if (b0 >= kk) return false;
  const int N = d.n, ntp = d.ntok_pad, ppad = d.ppad;
  const int nsteps = (N + 31) / 32;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const int cbase = cblk * 512 + wave * 64;
  const bool active = cbase < C;
  const int c0 = cbase + 2 * col;

  // range-checked buffer loads as in the folded pass: tokens at and past N and
  // rows without a bin read zeros
  const long long plane = (long long)ppad * ntp;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(kv ? d.v : d.k);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src + (size_t)layer * N * C), 0, N * C * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(F16 ? d.tw16 : d.tw), 0, (int)(NPL * plane * 2), 0x00020000);
  const int xvoff = active ? (c0 + 8 * g * C) * 2 : N * C * 2;

  f32x16_t acc[NTL][2];
#pragma unroll
  for (int i = 0; i < NTL; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][m][v] = 0.f;

  uint32_t xa[16], xb[16];
  auto load_x = [&](int step, uint32_t* dst) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        dst[8 * s2 + t] = __builtin_amdgcn_raw_buffer_load_b32(xres, xvoff + (step * 32 + 16 * s2 + t) * C * 2, 0, 0);
  };
  constexpr int TWN = NPL * 32 * NTL * 4;
  constexpr int TWI = (TWN + 511) / 512;
  u32x4_t twr[TWI];
  int twoff[TWI];
#pragma unroll
  for (int it = 0; it < TWI; ++it) {
    const int item = tid + 512 * it;
    const int q = item / (128 * NTL), r = (item / 4) % (32 * NTL), i = item % 4;
    const int trow = band_table_row<NC>(r, b0, kk);
    twoff[it] = (item < TWN && trow >= 0) ? (int)((q * plane + (long long)trow * ntp + 8 * i) * 2)
                                          : (int)(NPL * plane * 2);
  }
  auto load_tw = [&](int step) {
#pragma unroll
    for (int it = 0; it < TWI; ++it)
      twr[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(tres, twoff[it] + step * 64, 0, 0));
  };
  auto store_tw = [&](uint16_t* buf) {
#pragma unroll
    for (int it = 0; it < TWI; ++it) {
      const int item = tid + 512 * it;
      if (TWN % 512 != 0 && item >= TWN) break;
      const int q = item / (128 * NTL), r = (item / 4) % (32 * NTL), i = item % 4;
      *reinterpret_cast<u32x4_t*>(&buf[(q * 32 * NTL + r) * kTwStride + 8 * i]) = twr[it];
    }
  };
  auto compute = [&](const uint16_t* buf, const uint32_t* xs) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4_t bu[2];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t w0 = xs[8 * s2 + 2 * h], w1 = xs[8 * s2 + 2 * h + 1];
        if constexpr (F16) {
          // bf16 -> fp32 is exact; fp32 -> fp16 is exact below 65536
          bu[0][h] = pack_f16(__uint_as_float(w0 << 16), __uint_as_float(w1 << 16));
          bu[1][h] = pack_f16(__uint_as_float(w0 & 0xffff0000u), __uint_as_float(w1 & 0xffff0000u));
        } else {
          bu[0][h] = (w0 & 0xffffu) | (w1 << 16);
          bu[1][h] = (w0 >> 16) | (w1 & 0xffff0000u);
        }
      }
#pragma unroll
      for (int pt = 0; pt < NTL; ++pt) {
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
          const uint16_t* ap = &buf[(q * 32 * NTL + pt * 32 + col) * kTwStride + 16 * s2 + 8 * g];
          if constexpr (F16) {
            const f16x8_t a = *reinterpret_cast<const f16x8_t*>(ap);
            acc[pt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8_t, bu[0]), acc[pt][0], 0, 0, 0);
            acc[pt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8_t, bu[1]), acc[pt][1], 0, 0, 0);
          } else {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ap);
            acc[pt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bu[0]), acc[pt][0], 0, 0, 0);
            acc[pt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bu[1]), acc[pt][1], 0, 0, 0);
          }
        }
      }
    }
  };

  load_tw(0);
  load_x(0, xa);
  store_tw(lds[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_tw(1);
  __builtin_amdgcn_sched_barrier(0);
  load_x(1, xb);
  for (int step = 0; step < nsteps; step += 2) {
    __syncthreads();
    compute(lds[0], xa);
    store_tw(lds[1]);
    load_tw(step + 2);
    __builtin_amdgcn_sched_barrier(0);
    load_x(step + 2, xa);
    __syncthreads();
    compute(lds[1], xb);
    store_tw(lds[0]);
    load_tw(step + 3);
    __builtin_amdgcn_sched_barrier(0);
    load_x(step + 3, xb);
  }

  if constexpr (F16) {
    bool bad = false;
#pragma unroll
    for (int pt = 0; pt < NTL; ++pt)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) bad |= !(__builtin_fabsf(acc[pt][m][v]) < __builtin_inff());
    if (__syncthreads_or((int)bad)) return true;  // the caller redoes the tile in bf16
  }
  if (!active) return false;
  float* Y = reinterpret_cast<float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
#pragma unroll
  for (int pt = 0; pt < NTL; ++pt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = band_y_row<NC>(pt, 8 * (v >> 2) + 4 * g + (v & 3), b0, kk, ppad);
      if (row >= 0) *reinterpret_cast<float2*>(Y + (size_t)row * C + c0) = make_float2(acc[pt][0][v], acc[pt][1][v]);
    }
  return false;
}

// One tile per block: an fp16 pass, and for a tile that meets a value outside
// fp16's range, the bf16 pass of the same tile right after it (the
// three-plane layout is the larger, so it holds both passes' LDS).  With
// NC = 2 a block whose bins fill two tiles of each kind takes the radix-4
// fp16 pass when the transform length is a multiple of 128, else the folded
// one: there the MFMAs these forms save (a quarter folded, nearly half in
// radix-4) outweigh their vector work (the split of every data value).  A block with one tile's worth of
// bins (a shorter chunk of the launch) runs as the NC = 1 block of its first
// 32 bins, unfolded, and so does every block of an NC = 1 launch.  No loop
// then carries a per-tile test; tiles with some bins past kk multiply zero
// twiddle rows.
template <int NC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_band_bf16(ScoreLaunch sl, char* ws) {
  __shared__ __attribute__((aligned(16))) BandLds<2 * NC, false> sh;
  static_assert(sizeof(BandLds<2 * NC, true>) <= sizeof(BandLds<2 * NC, false>), "LDS of the fp16 pass");
  const int cblk = blockIdx.x, prob = blockIdx.z;
  if constexpr (NC == 2) {
    const ScoreChunkDesc& d = sl.c[prob / (2 * sl.L)];
    const int kk = d.kk, rblk = blockIdx.y;
    if (kk - rblk * 64 > 32) {
      auto& sh16 = *reinterpret_cast<BandLds<4, true>*>(&sh);
      if (d.nf % 128 == 0 ? band_r4(sl, ws, cblk, rblk, prob, sh16) : band_fold<2>(sl, ws, cblk, rblk, prob, sh16)) {
        __syncthreads();  // the fp16 pass's LDS reads are done
        band_unfolded<2, false>(sl, ws, cblk, rblk, prob, sh);
      }
      return;
    }
    // bins rblk * 64 .. kk - 1 (at most 32; none when the chunk ends before)
    if (band_unfolded<1, true>(sl, ws, cblk, 2 * rblk, prob, *reinterpret_cast<BandLds<2, true>*>(&sh))) {
      __syncthreads();
      band_unfolded<1, false>(sl, ws, cblk, 2 * rblk, prob, *reinterpret_cast<BandLds<2, false>*>(&sh));
    }
  } else {
    if (band_unfolded<1, true>(sl, ws, cblk, blockIdx.y, prob, *reinterpret_cast<BandLds<2, true>*>(&sh))) {
      __syncthreads();
      band_unfolded<1, false>(sl, ws, cblk, blockIdx.y, prob, sh);
    }
  }
}

// ---- 2/3. Gram of the band coefficients and energy evaluation ----------------
// One block per (chunk, layer, K|V) problem (blocks loop over problems); the
// block's Gram and polynomial coefficients live in its workspace slot.
__global__ __launch_bounds__(256) void k_gram_eval(ScoreLaunch sl, char* ws, int n_probs) {
  __shared__ float sa[32][132];
  __shared__ float sb[32][132];
  const int L = sl.L, C = sl.C;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  double* slot = reinterpret_cast<double*>(ws + sl.slot_off + (size_t)blockIdx.x * sl.slot_bytes);

  for (int prob = blockIdx.x; prob < n_probs; prob += gridDim.x) {
    const int b = prob / (2 * L), layer = (prob / 2) % L, kv = prob % 2;
    const ScoreChunkDesc& d = sl.c[b];
    const int kk = d.kk, P2 = 2 * kk, ppad = d.ppad, nf = d.nf, N = d.n;
    const float* Y = reinterpret_cast<const float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
    double* G = slot;                          // [P2][P2]
    double* coef = slot + (size_t)P2 * P2;     // [2kk-1][2]: cos and sin coefficient of each k
    const int nblk = (P2 + 127) / 128;

    for (int bi = 0; bi < nblk; ++bi)
      for (int bj = 0; bj < nblk; ++bj) {
        double acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
        for (int cc = 0; cc < C; cc += 32) {
          __syncthreads();
          for (int item = tid; item < 128 * 8; item += 256) {
            int r = item >> 3, q4 = (item & 7) * 4;
            int ra = bi * 128 + r, rb = bj * 128 + r;
            float4 va = ra < P2 ? *reinterpret_cast<const float4*>(Y + (size_t)ra * C + cc + q4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            float4 vb = rb < P2 ? *reinterpret_cast<const float4*>(Y + (size_t)rb * C + cc + q4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            sa[q4 + 0][r] = va.x; sa[q4 + 1][r] = va.y; sa[q4 + 2][r] = va.z; sa[q4 + 3][r] = va.w;
            sb[q4 + 0][r] = vb.x; sb[q4 + 1][r] = vb.y; sb[q4 + 2][r] = vb.z; sb[q4 + 3][r] = vb.w;
          }
          __syncthreads();
#pragma unroll 4
          for (int ch = 0; ch < 32; ++ch) {
            double a[8], bv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = (double)sa[ch][8 * ty + i];
#pragma unroll
            for (int j = 0; j < 8; ++j) bv[j] = (double)sb[ch][8 * tx + j];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], bv[j], acc[i][j]);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            int r = bi * 128 + 8 * ty + i, c = bj * 128 + 8 * tx + j;
            if (r < P2 && c < P2) G[(size_t)r * P2 + c] = acc[i][j];
          }
      }
    __syncthreads();

    poly_energy<256>(d, layer, kv, G, P2, coef, ws);
    __syncthreads();
  }
}

// ---- 4. magnitudes, per-layer normalisation, mean over layers ----------------
constexpr int kFinThreads = 1024;
constexpr int kFinPer = kMaxN / kFinThreads;  // tokens per thread

__device__ double block_reduce(double v, int op, double* red) {
  // op: 0 sum, 1 max, 2 min -- fixed pairing order, deterministic
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = kFinThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      double a = red[tid], b = red[tid + s];
      red[tid] = op == 0 ? a + b : (op == 1 ? fmax(a, b) : fmin(a, b));
    }
    __syncthreads();
  }
  double r = red[0];
  __syncthreads();
  return r;
}

// ---- 2'. Gram on the matrix cores (problems with 2*kk <= 128) ----------------
// G = Y Y^T over the C channels.  Y (fp32) is split per stage of 64 channels
// into three bf16 planes Y = Y1 + Y2 + Y3 (each the round-to-nearest-even
// bf16 of the previous remainder, exact to 2^-26), and
//   G = Y1Y1 + Y1Y2 + Y2Y1 + Y1Y3 + Y3Y1 + Y2Y2   (dropped terms < 2^-25 |G|)
// with bf16 products exact in fp32; accumulation in fp32 over 256 channels,
// then in fp64.  Only tiles on or above the diagonal are computed, one per
// wave (at most 10 of the 16 waves); each writes both halves.  Both MFMA
// operands are "8 channels of one band row", so A and B are read from the
// same plane rows (no transpose).  The planes are double-buffered: after the
// one barrier of a stage, the waves take that stage's products and then
// convert the next stage (loaded one stage ahead into registers) into the
// other buffer, so conversion and loads overlap the matrix cores.
constexpr int kGramCh = 64;            // channels per stage
constexpr int kGramPS = kGramCh + 8;   // plane row stride (bf16): 144 B
constexpr int kGramThreads = 1024;

// x = h1 + h2 + h3 (bf16 pairs, element 0 in the low half), each part the
// round-to-nearest-even bf16 of what the previous parts leave; the
// remainders are exact in fp32.
__device__ inline void split3_bf16(f32x2_t x, uint32_t& h1, uint32_t& h2, uint32_t& h3) {
  h1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  const f32x2_t r1 = {x[0] - __uint_as_float(h1 << 16), x[1] - __uint_as_float(h1 & 0xffff0000u)};
  h2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r1, bf16x2_t));
  const f32x2_t r2 = {r1[0] - __uint_as_float(h2 << 16), r1[1] - __uint_as_float(h2 & 0xffff0000u)};
  h3 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2_t));
}

__global__ __launch_bounds__(kGramThreads) void k_gram_mfma(ScoreLaunch sl, char* ws) {
  // two buffers of three bf16 planes during the accumulation, then the fp64
  // Gram and coefficients
  // G rows are P2 + 1 doubles apart: an odd stride puts the column-wise
  // (transposed) writes and the coefficient sums' reads on different banks
  __shared__ __attribute__((aligned(16))) double lds_g[128 * 129 + 256];
  typedef uint16_t plane_t[128 * kGramPS];
  plane_t* pl = reinterpret_cast<plane_t*>(lds_g);  // [buffer * 3 + plane]
  static_assert(sizeof(uint16_t) * 6 * 128 * kGramPS <= sizeof(double) * 128 * 129, "plane alias");
  const int L = sl.L, C = sl.C;
  const int prob = blockIdx.x;
  const int b = prob / (2 * L), layer = (prob / 2) % L, kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int ppad = d.ppad, P2 = 2 * d.kk, nt = ppad / 32;
  const float* Y = reinterpret_cast<const float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, col = lane & 31;

  // upper tile number `wave` of the nt x nt tile grid (nt <= 4: at most 10)
  int tI = 0, tJ = 0;
  bool own = false;
  {
    int u = 0;
    for (int ti = 0; ti < nt; ++ti)
      for (int tj = ti; tj < nt; ++tj, ++u)
        if (u == wave) { tI = ti; tJ = tj; own = true; }
  }
  f32x16_t acc;
  double accd[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) { acc[v] = 0.f; accd[v] = 0.0; }

  // one stage of Y: 128 rows x 16 float4, 2 per thread; two register sets,
  // so that each stage is loaded two stages ahead.  Loads go through a buffer
  // resource whose range check returns zeros for rows at or past ppad and,
  // through an offset past the range, for stages at or past nst: no load or
  // conversion is conditional, and the loop below has no conditional code
  // around them (vector-memory loads complete in issue order, and a branch
  // around a load makes the compiler's wait counts assume the worst path).
  constexpr int kPf = 128 * (kGramCh / 4) / kGramThreads;
  static_assert(kPf * kGramThreads == 128 * (kGramCh / 4), "Y stage split");
  const int nst = C / kGramCh;
  const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(Y), 0, ppad * C * 4, 0x00020000);
  u32x4_t pfa[kPf], pfb[kPf];
  auto load_stage = [&](int stage, u32x4_t* pf) {
    const int sbase = stage < nst ? stage * kGramCh * 4 : ppad * C * 4;
#pragma unroll
    for (int it = 0; it < kPf; ++it) {
      const int item = tid + kGramThreads * it, r = item / (kGramCh / 4), q4 = 4 * (item % (kGramCh / 4));
      pf[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(yres, sbase + (r * C + q4) * 4, 0, 0));
    }
  };
  // rows at or past ppad convert zeros into plane rows no tile reads
  auto convert = [&](int buf, const u32x4_t* pf) {
#pragma unroll
    for (int it = 0; it < kPf; ++it) {
      const int item = tid + kGramThreads * it;
      const int r = item / (kGramCh / 4), q4 = 4 * (item % (kGramCh / 4));
      uint32_t h[3][2];
      split3_bf16((f32x2_t){__uint_as_float(pf[it][0]), __uint_as_float(pf[it][1])}, h[0][0], h[1][0], h[2][0]);
      split3_bf16((f32x2_t){__uint_as_float(pf[it][2]), __uint_as_float(pf[it][3])}, h[0][1], h[1][1], h[2][1]);
#pragma unroll
      for (int q = 0; q < 3; ++q)
        *reinterpret_cast<uint2*>(&pl[3 * buf + q][r * kGramPS + q4]) = make_uint2(h[q][0], h[q][1]);
    }
  };

  // products of stage st on buffer st & 1; then stage st + 1 (loaded two
  // stages ago) converted into the other buffer, and stage st + 3 loaded
  // into the register set that conversion freed.  With nst odd the last
  // call runs on stage nst, all zeros, and adds nothing.
  auto stage_step = [&](int st, int buf, const u32x4_t* pf_next, u32x4_t* pf_free) {
    // Stage st's planes are complete, and stage st-1's reads of the other
    // buffer are done, once every wave has passed this barrier.
    __syncthreads();
    if (own) {
      const plane_t* pb = pl + 3 * buf;
#pragma unroll
      for (int ks = 0; ks < kGramCh / 16; ++ks) {
        const int ra = (tI * 32 + col) * kGramPS + 16 * ks + 8 * g;
        const int rb = (tJ * 32 + col) * kGramPS + 16 * ks + 8 * g;
        bf16x8_t a[3], bb[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          a[q] = *reinterpret_cast<const bf16x8_t*>(&pb[q][ra]);
          bb[q] = *reinterpret_cast<const bf16x8_t*>(&pb[q][rb]);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], bb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], bb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], bb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], bb[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], bb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], bb[1], acc, 0, 0, 0);
      }
    }
    convert(buf ^ 1, pf_next);
    load_stage(st + 3, pf_free);
    if ((((st + 1) * kGramCh) % 256) == 0 || st + 1 == nst) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        accd[v] += (double)acc[v];
        acc[v] = 0.f;
      }
    }
  };
  // the prologue leaves stage 1, then stage 2, in flight: the order the loop
  // body issues its loads in
  load_stage(0, pfa);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(1, pfb);
  convert(0, pfa);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(2, pfa);
  for (int st = 0; st < nst; st += 2) {
    stage_step(st, 0, pfb, pfb);      // pfb: stage st + 1, then st + 3
    stage_step(st + 1, 1, pfa, pfa);  // pfa: stage st + 2, then st + 4
  }
  __syncthreads();  // planes no longer read: the buffer now holds G [P2][P2 + 1]
  double* Gs = lds_g;
  const int ldg = P2 + 1;
  if (own) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = tI * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      const int c = tJ * 32 + col;
      if (r < P2 && c < P2) {
        Gs[r * ldg + c] = accd[v];
        Gs[c * ldg + r] = accd[v];
      }
    }
  }
  __syncthreads();
  poly_energy<kGramThreads>(d, layer, kv, Gs, ldg, lds_g + 128 * 129, ws);
}

// ---- L2 variant: energies without the frequency analysis ----------------------
// E[n] = sum_c x_c[n]^2 over the token's H*D channels (the alpha = 1 energies,
// App. E.4), written where the band path writes its low-pass energies, so the
// same layer normalisation and mean follow.  One wave per token row; each lane
// sums C/64 squares in fp64 (exact products), then a fixed-order wave
// reduction (deterministic).
template <int DT>
__global__ __launch_bounds__(256) void k_energy_l2(ScoreLaunch sl, char* ws) {
  const int L = sl.L, C = sl.C;
  const int prob = blockIdx.y;
  const int b = prob / (2 * L), layer = (prob / 2) % L, kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d.n) return;
  const size_t base = ((size_t)layer * d.n + row) * C;
  double e = 0.0;
  if (DT == CT_BF16) {
    const uint16_t* x = reinterpret_cast<const uint16_t*>(kv ? d.v : d.k) + base;
    for (int c = 8 * lane; c < C; c += 8 * 64) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(x + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xffff0000u);
        e = fma(lo, lo, e);
        e = fma(hi, hi, e);
      }
    }
  } else {
    const float* x = reinterpret_cast<const float*>(kv ? d.v : d.k) + base;
    for (int c = 4 * lane; c < C; c += 4 * 64) {
      const float4 w = *reinterpret_cast<const float4*>(x + c);
      e = fma((double)w.x, (double)w.x, e);
      e = fma((double)w.y, (double)w.y, e);
      e = fma((double)w.z, (double)w.z, e);
      e = fma((double)w.w, (double)w.w, e);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o);
  if (lane == 0) reinterpret_cast<double*>(ws + d.e_off)[(size_t)(layer * 2 + kv) * d.n + row] = e;
}


// ---- high-frequency view: energies of x - xlow ----------------------------------
// At the stored positions n < N the inverse transform of every bin returns the
// row itself, so the bins at and above the cutoff reconstruct x - xlow there,
// and (Sec. 5.4, App. E.2: the high-frequency-guided strategy)
//     E_high[n] = |x[n]|^2 - 2 <x[n], xlow[n]> + E_low[n].
// E_low comes from the band path above.  The cross term is
//     <x[n], xlow[n]> = (1/nf) sum_p w_p t_p(n) Z[p][n],   Z = Y X^T,
// with t_p the twiddle row p, w_p the bin weight (1 for DC and Nyquist, else
// 2), and Z the band coefficients contracted with the stored row over the
// channels, on the matrix cores: Y (fp32) in three bf16 planes as the Gram
// takes it, bf16 X exact (three products), fp32 X in three planes too (six).
// One wave per 32 tokens, 8 waves per block; a 64-channel stage of the Y
// planes is shared in LDS, the next stage's Y and X are loaded during the
// current stage's products; the band is taken 128 rows at a time.  Z is
// accumulated in fp32 over the channels, the sums over p and the energies in
// fp64.  The result overwrites E_low (read first by the same lane).
template <int DT>
__global__ __launch_bounds__(512) void k_highpass(ScoreLaunch sl, char* ws) {
  __shared__ __attribute__((aligned(16))) uint16_t pl[3][128 * kGramPS];
  const int L = sl.L, C = sl.C;
  const int prob = blockIdx.y;
  const int b = prob / (2 * L), layer = (prob / 2) % L, kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int N = d.n, kk = d.kk, P2 = 2 * kk, ppad = d.ppad, nf = d.nf;
  const int t0 = blockIdx.x * 256;
  if (t0 >= N) return;  // block-uniform
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const int n = t0 + wave * 32 + col;
  const int nrow = min(n, N - 1);  // lanes past N read a valid row; their results are dropped
  const float* Y = reinterpret_cast<const float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * ppad) * C;
  const size_t xoff = ((size_t)layer * N + nrow) * C + 8 * g;
  const double2* trig = d.trig;
  constexpr int XW = DT == CT_BF16 ? 4 : 8;  // dwords of X per lane per 16-channel step

  double etot = 0.0, cross = 0.0;
  uint32_t xr[4][XW];
  float4 yr[4];
  auto load_x = [&](int c0) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (DT == CT_BF16) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const uint16_t*>(kv ? d.v : d.k) + xoff + c0 + 16 * ks);
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[ks][i] = v[i];
      } else {
        const float* p = reinterpret_cast<const float*>(kv ? d.v : d.k) + xoff + c0 + 16 * ks;
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(p);
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { xr[ks][i] = v0[i]; xr[ks][XW / 2 + i] = v1[i]; }
      }
    }
  };
  // Y rows [pg, pg + 128) x channels [c0, c0 + 64): 16 floats per thread
  auto load_y = [&](int pg, int c0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = tid + 512 * it, r = item >> 4, q4 = 4 * (item & 15);
      yr[it] = pg + r < ppad ? *reinterpret_cast<const float4*>(Y + (size_t)(pg + r) * C + c0 + q4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_y = [&]() {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = tid + 512 * it, r = item >> 4, q4 = 4 * (item & 15);
      const float x[4] = {yr[it].x, yr[it].y, yr[it].z, yr[it].w};
      uint32_t h[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b1 = bf16_rne_from_f32_bits(__float_as_uint(x[e]));
        const float r1 = x[e] - __uint_as_float(b1 << 16);
        const uint32_t b2 = bf16_rne_from_f32_bits(__float_as_uint(r1));
        const float r2 = r1 - __uint_as_float(b2 << 16);
        h[0][e] = b1;
        h[1][e] = b2;
        h[2][e] = bf16_rne_from_f32_bits(__float_as_uint(r2));
      }
#pragma unroll
      for (int q = 0; q < 3; ++q)
        *reinterpret_cast<uint2*>(&pl[q][r * kGramPS + q4]) =
            make_uint2(h[q][0] | (h[q][1] << 16), h[q][2] | (h[q][3] << 16));
    }
  };

  for (int pg = 0; pg < ppad; pg += 128) {
    const int nt = min(4, (ppad - pg) / 32);  // block-uniform
    f32x16_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    load_x(0);
    load_y(pg, 0);
    for (int c0 = 0; c0 < C; c0 += 64) {
      __syncthreads();  // the previous stage's planes are no longer read
      store_y();
      __syncthreads();
      uint32_t xs[4][XW];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < XW; ++i) xs[ks][i] = xr[ks][i];
      if (c0 + 64 < C) {
        load_x(c0 + 64);
        load_y(pg, c0 + 64);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t bx[3];
        if (DT == CT_BF16) {
          u32x4_t u;
#pragma unroll
          for (int i = 0; i < 4; ++i) u[i] = xs[ks][i];
          bx[0] = __builtin_bit_cast(bf16x8_t, u);
          if (pg == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const double lo = (double)__uint_as_float(xs[ks][i] << 16);
              const double hi = (double)__uint_as_float(xs[ks][i] & 0xffff0000u);
              etot = fma(lo, lo, etot);
              etot = fma(hi, hi, etot);
            }
          }
        } else {
          u32x4_t u[3];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = __uint_as_float(xs[ks][e]);
            const uint32_t b1 = bf16_rne_from_f32_bits(xs[ks][e]);
            const float r1 = x - __uint_as_float(b1 << 16);
            const uint32_t b2 = bf16_rne_from_f32_bits(__float_as_uint(r1));
            const float r2 = r1 - __uint_as_float(b2 << 16);
            const uint32_t b3 = bf16_rne_from_f32_bits(__float_as_uint(r2));
            const int w = e >> 1, sh = 16 * (e & 1);
            if (sh == 0) { u[0][w] = b1; u[1][w] = b2; u[2][w] = b3; }
            else { u[0][w] |= b1 << 16; u[1][w] |= b2 << 16; u[2][w] |= b3 << 16; }
            if (pg == 0) etot = fma((double)x, (double)x, etot);
          }
#pragma unroll
          for (int q = 0; q < 3; ++q) bx[q] = __builtin_bit_cast(bf16x8_t, u[q]);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          if (pt >= nt) break;
          const int ra = (pt * 32 + col) * kGramPS + 16 * ks + 8 * g;
          bf16x8_t a[3];
#pragma unroll
          for (int q = 0; q < 3; ++q) a[q] = *reinterpret_cast<const bf16x8_t*>(&pl[q][ra]);
          acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], bx[0], acc[pt], 0, 0, 0);
          acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], bx[0], acc[pt], 0, 0, 0);
          acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], bx[0], acc[pt], 0, 0, 0);
          if (DT != CT_BF16) {
            acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], bx[1], acc[pt], 0, 0, 0);
            acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], bx[1], acc[pt], 0, 0, 0);
            acc[pt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], bx[2], acc[pt], 0, 0, 0);
          }
        }
      }
    }
    // cross term of this band slice: lane holds Z[p][n] for 16 rows p per tile
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if (pt >= nt) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int p = pg + pt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        if (p < P2) {
          const int j = p < kk ? p : p - kk;
          const uint32_t m = ((uint32_t)j * (uint32_t)nrow) % (uint32_t)nf;
          const double2 cs = trig[m];
          const double w = (j == 0 || 2 * j == nf) ? 1.0 : 2.0;
          cross = fma(w * (p < kk ? cs.x : cs.y), (double)acc[pt][v], cross);
        }
      }
    }
  }
  cross += __shfl_xor(cross, 32);
  etot += __shfl_xor(etot, 32);
  if (g == 0 && n < N) {
    double* E = reinterpret_cast<double*>(ws + d.e_off) + (size_t)(layer * 2 + kv) * N;
    E[n] = etot - 2.0 * cross / (double)nf + E[n];
  }
}

// ---- App. E.1: energy fractions of frequency bands ------------------------------
// With every bin kept (kk = nb), Y holds R_j and S_j of all bins for all
// channels.  Bin j carries e_j = w_j (|R_j|^2 + |S_j|^2) / nf summed over the
// channels (w_j = 1 at DC and Nyquist, else 2), and the bins sum to the
// energy of the stored sequence (Parseval).  Band b of n_bands holds the bins
// j with floor(j * n_bands / nb) = b.  One block per problem: each wave sums
// the squares of a cos row and its sin row in fp64 (fixed order), the bins
// go to LDS, then each band and the total are summed in bin order.
constexpr int kMaxBins = kMaxN / 2 + 1;
constexpr int kMaxBands = 1024;

__global__ __launch_bounds__(512) void k_bin_energy(ScoreLaunch sl, char* ws, int n_bands,
                                                    double* fraction, double* total) {
  __shared__ double ebin[kMaxBins];
  __shared__ double eband[kMaxBands];
  __shared__ double etot;
  const int L = sl.L, C = sl.C;
  const int prob = blockIdx.x;
  const int b = prob / (2 * L), layer = (prob / 2) % L, kv = prob % 2;
  const ScoreChunkDesc& d = sl.c[b];
  const int nb = d.kk, nf = d.nf;
  const float* Y = reinterpret_cast<const float*>(ws + d.y_off) + ((size_t)(layer * 2 + kv) * d.ppad) * C;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int j = wave; j < nb; j += 8) {
    const float* rc = Y + (size_t)j * C;
    const float* rs = Y + (size_t)(nb + j) * C;
    double e = 0.0;
    for (int c = 4 * lane; c < C; c += 256) {
      const float4 a = *reinterpret_cast<const float4*>(rc + c);
      const float4 q = *reinterpret_cast<const float4*>(rs + c);
      e = fma((double)a.x, (double)a.x, e);
      e = fma((double)a.y, (double)a.y, e);
      e = fma((double)a.z, (double)a.z, e);
      e = fma((double)a.w, (double)a.w, e);
      e = fma((double)q.x, (double)q.x, e);
      e = fma((double)q.y, (double)q.y, e);
      e = fma((double)q.z, (double)q.z, e);
      e = fma((double)q.w, (double)q.w, e);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o);
    if (lane == 0) ebin[j] = ((j == 0 || 2 * j == nf) ? 1.0 : 2.0) * e / (double)nf;
  }
  __syncthreads();
  for (int bd = tid; bd < n_bands; bd += 512) {
    // first bin of band bd: the least j with j * n_bands >= bd * nb
    const int j0 = (int)(((long long)bd * nb + n_bands - 1) / n_bands);
    const int j1 = (int)(((long long)(bd + 1) * nb + n_bands - 1) / n_bands);
    double e = 0.0;
    for (int j = j0; j < j1; ++j) e += ebin[j];
    eband[bd] = e;
  }
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int bd = 0; bd < n_bands; ++bd) t += eband[bd];
    etot = t;
  }
  __syncthreads();
  const size_t row = (size_t)(b * L + layer) * 2 + kv;
  for (int bd = tid; bd < n_bands; bd += 512)
    fraction[row * n_bands + bd] = etot > 0.0 ? eband[bd] / etot : 0.0;
  if (tid == 0 && total) total[row] = etot;
}

// ---- 4'. per (chunk, layer): magnitudes and normalisation --------------------
// s = sqrt(E_K)/2 + sqrt(E_V)/2 per token, normalised within the layer; the
// result overwrites the E_K row of the layer (read before written by the same
// thread).  Fixed-order block reductions keep it deterministic.
__global__ __launch_bounds__(kFinThreads) void k_layer_norm(ScoreLaunch sl, char* ws,
                                                            float* layer_score) {
  __shared__ double red[kFinThreads];
  const ScoreChunkDesc& d = sl.c[blockIdx.x];
  const int l = blockIdx.y, N = d.n, tid = threadIdx.x;
  double* ek = reinterpret_cast<double*>(ws + d.e_off) + (size_t)(l * 2) * N;
  const double* ev = ek + N;
  double s[kFinPer];
  double part_sum = 0.0, part_max = -INFINITY, part_min = INFINITY;
#pragma unroll
  for (int i = 0; i < kFinPer; ++i) {  // token i * kFinThreads + tid: coalesced, all threads busy
    const int n = i * kFinThreads + tid;
    s[i] = 0.0;
    if (n < N) {
      s[i] = 0.5 * sqrt(fmax(ek[n], 0.0)) + 0.5 * sqrt(fmax(ev[n], 0.0));
      part_sum += s[i];
      part_max = fmax(part_max, s[i]);
      part_min = fmin(part_min, s[i]);
    }
  }
  // normalisation: v = (s - shift) / denom, or the constant `fill`
  double denom = 1.0, shift = 0.0, fill = -1.0;
  if (sl.norm == CT_NORM_SUM) {
    const double t = block_reduce(part_sum, 0, red);
    if (t > 0.0) denom = t; else fill = 1.0 / (double)N;
  } else if (sl.norm == CT_NORM_MAX) {
    const double mx = block_reduce(part_max, 1, red);
    if (mx > 0.0) denom = mx; else fill = 0.0;
  } else if (sl.norm == CT_NORM_MINMAX) {
    const double mx = block_reduce(part_max, 1, red);
    const double mn = block_reduce(part_min, 2, red);
    if (mx - mn > 0.0) { denom = mx - mn; shift = mn; } else fill = 0.0;
  }
#pragma unroll
  for (int i = 0; i < kFinPer; ++i) {
    const int n = i * kFinThreads + tid;
    if (n < N) {
      double v = fill >= 0.0 ? fill : (s[i] - shift) / denom;
      if (sl.norm == CT_NORM_NONE) v = s[i];
      ek[n] = v;
      if (layer_score) layer_score[(size_t)l * sl.total_tokens + d.tok_off + n] = (float)v;
    }
  }
}

// ---- 4''. mean over layers, in layer order ------------------------------------
__global__ __launch_bounds__(256) void k_layer_mean(ScoreLaunch sl, char* ws, float* score) {
  const ScoreChunkDesc& d = sl.c[blockIdx.y];
  const int n = blockIdx.x * 256 + threadIdx.x, N = d.n, L = sl.L;
  if (n >= N) return;
  const double* e = reinterpret_cast<const double*>(ws + d.e_off);
  // sum in layer order; the loads of 8 layers are issued before they are added
  double acc = 0.0;
  int l = 0;
  for (; l + 8 <= L; l += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = e[(size_t)((l + u) * 2) * N + n];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; l < L; ++l) acc += e[(size_t)(l * 2) * N + n];
  score[d.tok_off + n] = (float)(acc / (double)L);
}

}  // namespace

// ---- host side ----------------------------------------------------------------

int fft_len(int n, ct_fftlen mode) {
  if (mode == CT_FFT_EXACT_N) return n;
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

int kkeep(int nf, int a_num, int a_den) {
  long long nb = nf / 2 + 1;
  long long k = ((long long)a_num * nb) / a_den;
  if (k < 1) k = 1;
  if (k > nb) k = nb;
  return (int)k;
}

size_t score_tables_bytes(int nf, int kk, int ntp, size_t* tw16_off, size_t* trig_off) {
  const int ppad = band_rows_padded(kk);
  size_t off = align256((size_t)3 * ppad * ntp * 2);
  if (tw16_off) *tw16_off = off;
  off = align256(off + (size_t)2 * ppad * ntp * 2);
  if (trig_off) *trig_off = off;
  return align256(off + (size_t)nf * 16);
}

ct_status score_plan(const int32_t* n_per_chunk, int32_t n_chunks, int32_t L, int32_t H,
                     int32_t D, int32_t a_num, int32_t a_den, ct_fftlen fftlen, size_t* bytes,
                     std::vector<ScoreLaunch>* launches, int32_t variant, const Context* ctx) {
  const int C = H * D;
  const bool band = variant != CT_SCORE_L2;  // the L2 variant needs only the energies
  size_t off = 0;
  struct Tab { int nf, kk, ntp; int64_t tw, tw16, trig; };
  std::vector<Tab> tabs;
  std::vector<ScoreChunkDesc> desc(n_chunks);
  int max_p2 = 0;
  int64_t tok = 0;
  for (int b = 0; b < n_chunks; ++b) {
    ScoreChunkDesc& d = desc[b];
    d = ScoreChunkDesc{};
    d.n = n_per_chunk[b];
    d.nf = fft_len(d.n, fftlen);
    d.kk = kkeep(d.nf, a_num, a_den);
    d.ppad = band_rows_padded(d.kk);
    d.ntok_pad = ((d.n + 31) / 32) * 32;
    d.tok_off = tok;
    tok += d.n;
    if (2 * d.kk > max_p2) max_p2 = 2 * d.kk;
    if (!band) continue;
    // tables held by the context are used as they are; the others get a
    // workspace region, written by the first chunk of the call that needs it
    ScoreTables held;
    if (ctx && context_find_tables(ctx, d.nf, d.kk, d.ntok_pad, &held)) {
      d.tw = held.tw;
      d.tw16 = held.tw16;
      d.trig = held.trig;
      d.tw_off = d.tw16_off = d.trig_off = -1;
      continue;
    }
    int found = -1;
    for (size_t t = 0; t < tabs.size(); ++t)
      if (tabs[t].nf == d.nf && tabs[t].kk == d.kk && tabs[t].ntp == d.ntok_pad) found = (int)t;
    if (found < 0) {
      Tab t{d.nf, d.kk, d.ntok_pad, (int64_t)off, 0, 0};
      size_t o16 = 0, otr = 0;
      off += score_tables_bytes(d.nf, d.kk, d.ntok_pad, &o16, &otr);
      t.tw16 = t.tw + (int64_t)o16;
      t.trig = t.tw + (int64_t)otr;
      tabs.push_back(t);
      d.tw_owner = 1;
      found = (int)tabs.size() - 1;
    }
    d.tw_off = tabs[found].tw;
    d.tw16_off = tabs[found].tw16;
    d.trig_off = tabs[found].trig;
  }
  for (int b = 0; b < n_chunks && band; ++b) {
    desc[b].y_off = (int64_t)off;
    off = align256(off + (size_t)L * 2 * desc[b].ppad * C * 4);
  }
  for (int b = 0; b < n_chunks; ++b) {
    desc[b].e_off = (int64_t)off;
    off = align256(off + (size_t)L * 2 * desc[b].n * 8);
  }
  const int64_t slot_bytes = (int64_t)align256(((size_t)max_p2 * max_p2 + 2 * (size_t)max_p2) * 8);
  int64_t probs_max = (int64_t)std::min(n_chunks, kMaxChunksPerLaunch) * L * 2;
  // Matrix-core Gram (2kk <= 128) keeps G in LDS and needs no slot; larger
  // bands take the fp64 path, whose blocks loop over problems and slots.
  const bool mfma_gram = max_p2 <= 128;
  const bool gram = band && variant != kVariantBandEnergy;
  int64_t n_slots = (mfma_gram || !gram) ? 0 : std::min<int64_t>(probs_max, 1024);
  const int64_t slot_budget = (int64_t)1 << 30;
  while (!mfma_gram && n_slots > 1 && n_slots * slot_bytes > slot_budget) n_slots /= 2;
  const int64_t slot_off = (int64_t)off;
  off += (size_t)(n_slots * slot_bytes);
  *bytes = align256(off);

  if (launches) {
    launches->clear();
    for (int b0 = 0; b0 < n_chunks; b0 += kMaxChunksPerLaunch) {
      ScoreLaunch sl{};
      sl.n_chunks = std::min(kMaxChunksPerLaunch, n_chunks - b0);
      sl.L = L; sl.H = H; sl.D = D; sl.C = C;
      sl.total_tokens = tok;
      sl.n_slots = (int32_t)n_slots;
      sl.slot_p2 = max_p2;
      sl.slot_off = slot_off;
      sl.slot_bytes = slot_bytes;
      sl.variant = variant;
      sl.max_ppad = 0;
      for (int i = 0; i < sl.n_chunks; ++i) {
        sl.c[i] = desc[b0 + i];
        sl.max_ppad = std::max(sl.max_ppad, sl.c[i].ppad);
      }
      launches->push_back(sl);
    }
  }
  return CT_OK;
}

void score_bind(std::vector<ScoreLaunch>* launches, char* ws) {
  for (ScoreLaunch& sl : *launches)
    for (int i = 0; i < sl.n_chunks; ++i) {
      ScoreChunkDesc& d = sl.c[i];
      if (d.tw_off < 0) continue;  // held by the context
      d.tw = reinterpret_cast<uint16_t*>(ws + d.tw_off);
      d.tw16 = reinterpret_cast<uint16_t*>(ws + d.tw16_off);
      d.trig = reinterpret_cast<double2*>(ws + d.trig_off);
    }
}

static ct_status launch_twiddle(const ScoreLaunch& sl, hipStream_t stream) {
  int max_elems = 0;
  bool any = false;
  for (int i = 0; i < sl.n_chunks; ++i) {
    if (!sl.c[i].tw_owner) continue;
    any = true;
    max_elems = std::max(max_elems, std::max(sl.c[i].ppad * sl.c[i].ntok_pad, sl.c[i].nf));
  }
  if (!any) return CT_OK;
  dim3 gt((max_elems + 255) / 256 < 2048 ? (max_elems + 255) / 256 : 2048, sl.n_chunks);
  {
    TimedLaunch tl_("twiddle", stream);
    hipLaunchKernelGGL(k_twiddle, gt, dim3(256), 0, stream, sl);
  }
  return check_launch("twiddle");
}

ct_status score_tables_build(int nf, int kk, int ntp, int dtype, const ScoreTables& t, hipStream_t stream) {
  ScoreLaunch sl{};
  sl.n_chunks = 1;
  sl.dtype = dtype;
  ScoreChunkDesc& d = sl.c[0];
  d.nf = nf;
  d.kk = kk;
  d.ppad = band_rows_padded(kk);
  d.ntok_pad = ntp;
  d.n = ntp;
  d.tw_owner = 1;
  d.tw = t.tw;
  d.tw16 = t.tw16;
  d.trig = t.trig;
  return launch_twiddle(sl, stream);
}

// Twiddle planes (tables not held by a context) and the band projection Y of
// every problem of a launch.
static ct_status band_project(const ScoreLaunch& sl, char* ws, hipStream_t stream) {
  if (ct_status s = launch_twiddle(sl, stream)) return s;

  dim3 gb((sl.C + 255) / 256, (sl.max_ppad + 127) / 128, sl.n_chunks * sl.L * 2);
  if (sl.dtype == CT_BF16) {
    // Bins per block: 32 (2 tiles) when no chunk keeps more, else 64 (4
    // tiles, 128 accumulator registers).  Each block streams X from HBM once,
    // so more blocks per band means more reads of X.
    int max_kk = 0;
    for (int i = 0; i < sl.n_chunks; ++i) max_kk = std::max(max_kk, sl.c[i].kk);
    const int nc = max_kk <= 32 ? 1 : 2;
    // 8 waves x 64 channels per block: every twiddle slab staged in LDS
    // serves 512 channels (the slabs, not X, are most of the L2 traffic)
    dim3 gq((sl.C + 511) / 512, (max_kk + 32 * nc - 1) / (32 * nc), sl.n_chunks * sl.L * 2);
    {
      TimedLaunch tl_("band", stream);
      if (nc == 1)
        hipLaunchKernelGGL((k_band_bf16<1>), gq, dim3(512), 0, stream, sl, ws);
      else
        hipLaunchKernelGGL((k_band_bf16<2>), gq, dim3(512), 0, stream, sl, ws);
    }
  } else {
    TimedLaunch tl_("band", stream);
    hipLaunchKernelGGL(k_band_fwd<CT_F32>, gb, dim3(256), 0, stream, sl, ws);
  }
  if (ct_status s = check_launch("band projection")) return s;
  return CT_OK;
}

// Energies -> per-layer scores -> layer mean.
static ct_status score_finish(const ScoreLaunch& sl, char* ws, float* score, float* layer_score,
                              hipStream_t stream) {
  int max_n = 0;
  for (int i = 0; i < sl.n_chunks; ++i) max_n = std::max(max_n, sl.c[i].n);
  {
    TimedLaunch tl_("layer_norm", stream);
    hipLaunchKernelGGL(k_layer_norm, dim3(sl.n_chunks, sl.L), dim3(kFinThreads), 0, stream, sl, ws,
                       layer_score);
  }
  if (ct_status s = check_launch("layer normalisation")) return s;
  {
    TimedLaunch tl_("layer_mean", stream);
    hipLaunchKernelGGL(k_layer_mean, dim3((max_n + 255) / 256, sl.n_chunks), dim3(256), 0, stream,
                       sl, ws, score);
  }
  return check_launch("layer mean");
}

ct_status score_run(const std::vector<ScoreLaunch>& launches, char* ws, float* score,
                    float* layer_score, hipStream_t stream) {
  for (const ScoreLaunch& sl : launches) {
    if (sl.variant == CT_SCORE_L2) {
      int max_n = 0;
      for (int i = 0; i < sl.n_chunks; ++i) max_n = std::max(max_n, sl.c[i].n);
      dim3 ge((max_n + 3) / 4, sl.n_chunks * sl.L * 2);
      {
        TimedLaunch tl_("energy_l2", stream);
        if (sl.dtype == CT_BF16)
          hipLaunchKernelGGL(k_energy_l2<CT_BF16>, ge, dim3(256), 0, stream, sl, ws);
        else
          hipLaunchKernelGGL(k_energy_l2<CT_F32>, ge, dim3(256), 0, stream, sl, ws);
      }
      if (ct_status s = check_launch("L2 energies")) return s;
      if (ct_status s = score_finish(sl, ws, score, layer_score, stream)) return s;
      continue;
    }
    if (ct_status s = band_project(sl, ws, stream)) return s;

    const int n_probs = sl.n_chunks * sl.L * 2;
    if (sl.slot_p2 <= 128) {
      TimedLaunch tl_("gram", stream);
      hipLaunchKernelGGL(k_gram_mfma, dim3(n_probs), dim3(kGramThreads), 0, stream, sl, ws);
      if (ct_status s = check_launch("gram/energy")) return s;
    } else {
      const int grid = std::min(n_probs, sl.n_slots);
      TimedLaunch tl_("gram", stream);
      hipLaunchKernelGGL(k_gram_eval, dim3(grid), dim3(256), 0, stream, sl, ws, n_probs);
      if (ct_status s = check_launch("gram/eval")) return s;
    }

    if (sl.variant == CT_SCORE_HIGHPASS) {
      int max_n = 0;
      for (int i = 0; i < sl.n_chunks; ++i) max_n = std::max(max_n, sl.c[i].n);
      TimedLaunch tl_("highpass", stream);
      dim3 gh((max_n + 255) / 256, n_probs);
      if (sl.dtype == CT_BF16)
        hipLaunchKernelGGL(k_highpass<CT_BF16>, gh, dim3(512), 0, stream, sl, ws);
      else
        hipLaunchKernelGGL(k_highpass<CT_F32>, gh, dim3(512), 0, stream, sl, ws);
      if (ct_status s = check_launch("high-frequency energies")) return s;
    }

    if (ct_status s = score_finish(sl, ws, score, layer_score, stream)) return s;
  }
  return CT_OK;
}

ct_status band_energy_run(const std::vector<ScoreLaunch>& launches, char* ws, int n_bands,
                          double* fraction, double* total, hipStream_t stream) {
  if (n_bands < 1 || n_bands > kMaxBands) return fail(CT_E_INVALID, "n_bands out of range");
  size_t done = 0;  // (chunk, layer, K|V) rows written by earlier launches
  for (const ScoreLaunch& sl : launches) {
    if (ct_status s = band_project(sl, ws, stream)) return s;
    const int n_probs = sl.n_chunks * sl.L * 2;
    {
      TimedLaunch tl_("bin_energy", stream);
      hipLaunchKernelGGL(k_bin_energy, dim3(n_probs), dim3(512), 0, stream, sl, ws, n_bands,
                         fraction + done * n_bands, total ? total + done : nullptr);
    }
    if (ct_status s = check_launch("band energies")) return s;
    done += (size_t)n_probs;
  }
  return CT_OK;
}

}  // namespace ct

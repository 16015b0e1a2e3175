// Selected-query causal GQA attention -- "Adaptive KV Cache Reuse for Fast
// Long-Context LLM Serving" (CacheTune), Sec. 4.1 "Recomputing in the new
// context" and App. B.2 (check layer: the selected positions' queries attend
// over the complete assembled layer under the causal mask).
//
// This file holds the path for fp32 storage (the bf16 path is attn.hip).
// Flash-style kernel on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16),
// computed transposed so that each query's softmax row lives in two lanes:
//   S^T (keys x queries) = K . Q^T      A = K rows from LDS, B = Q (registers)
//   O^T (dims x queries) += V^T . P^T   A = V^T from LDS,   B = P (registers)
// A wave owns 32 query rows of one query head; a block has 4 waves that share
// one KV head (grouped-query attention), so each 64-key K/V block staged in
// LDS serves all of them.  Queries are rotated to their positions (fp64 angle
// and sincos); softmax runs in fp32 with exp2.
// Precision: one bf16 rounding of the rotated query or of the probabilities
// moves the output by up to ~0.5 on inputs whose logits reach tens, so both
// enter the matrix cores as a bf16 hi + lo pair (16 significant bits; two
// MFMAs each).  fp32 K and V are split the same way (K_hi q_hi + K_hi q_lo +
// K_lo q_hi, and likewise for V and P).
// MFMA layouts (32x32x16): A lane -> row lane%32, k-group lane/32; B lane ->
// col lane%32, k-group lane/32; D lane -> col lane%32, rows
// 8*(v/4) + 4*(lane/32) + v%4.  The contraction index of a k-group only has
// to agree between A and B, which lets P stay in the accumulator layout.
#include "ct_device.h"
#include "ct_internal.h"

namespace ct {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BK = 64;   // keys per block
constexpr int VTS = 68;  // V^T row stride (bf16): 136 B keeps 8-byte reads conflict-free

template <int DT>
__device__ inline double ld_q(const void* p, size_t i) {
  if constexpr (DT == CT_F32) return (double)reinterpret_cast<const float*>(p)[i];
  else return (double)__uint_as_float(((uint32_t)reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

// 8 consecutive elements as packed bf16 (hi); fp32 inputs also give the bf16
// residual (lo), so that hi + lo carries 16 significant bits.
template <int DT>
__device__ inline void ld8_split(const void* base, size_t i, u32x4_t* hi, u32x4_t* lo) {
  if constexpr (DT == CT_BF16) {
    *hi = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + i);
  } else {
    const float4* f = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
    float4 a = f[0], b = f[1];
    float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t h0 = bf16_bits_rne(x[2 * h]), h1 = bf16_bits_rne(x[2 * h + 1]);
      float r0 = x[2 * h] - __uint_as_float(h0 << 16), r1 = x[2 * h + 1] - __uint_as_float(h1 << 16);
      (*hi)[h] = h0 | (h1 << 16);
      (*lo)[h] = bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16);
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int KS = D + 8;        // K row stride (bf16): 16-byte reads conflict-free
  constexpr int NS = D / 16;       // k-steps over the head dimension
  constexpr int NDT = D / 32;      // output tiles over the head dimension
  constexpr int NPL = DT == CT_F32 ? 2 : 1;  // bf16 planes of K and V in LDS
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NPL][BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[NPL][D * VTS];
  __shared__ int wmax[4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const int G = a.group, H = a.H, Hq = a.Hq, T = a.T;
  const int kvh = blockIdx.y;
  const int ntiles = (a.n_q + 31) / 32;
  const int n_units = ntiles * G;
  const int wg = gridDim.x - 1 - blockIdx.x;  // latest (longest) rows first
  const int unit = wg * 4 + wave;
  const bool active = unit < n_units;
  const int tile = active ? unit / G : 0;
  const int hq = kvh * G + (active ? unit % G : 0);
  const int row = tile * 32 + col;
  const bool valid = active && row < a.n_q;
  const int pos = valid ? a.qpos[row] : -1;

  // key range of the block: up to its largest query position
  int mx = pos;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  int bmax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  bmax = min(bmax, T - 1);
  const int nkb = bmax < 0 ? 0 : bmax / BK + 1;

  // Rotated query as bf16 hi + lo fragments (B operand): d = 16*s + 8*g + t.
  u32x4_t qh[NS], ql[NS];
  {
    const size_t qb = ((size_t)row * Hq + hq) * D;
    const double fpos = (double)max(pos, 0);
    auto put = [&](int s, int t, double y) {
      uint32_t hi = bf16_from_f64(y);
      double r = y - (double)__uint_as_float(hi << 16);
      uint32_t lo = bf16_from_f64(r);
      int w = t >> 1, sh = 16 * (t & 1);
      qh[s][w] |= hi << sh;
      ql[s][w] |= lo << sh;
    };
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int w = 0; w < 4; ++w) { qh[s][w] = 0u; ql[s][w] = 0u; }
    if (a.style == CT_ROPE_HALF) {
#pragma unroll
      for (int s = 0; s < NS / 2; ++s)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int j = 16 * s + 8 * g + t;  // pair (j, j + D/2): steps s and s + NS/2
          double u = valid ? ld_q<DT>(a.q, qb + j) : 0.0;
          double w = valid ? ld_q<DT>(a.q, qb + j + D / 2) : 0.0;
          double sn, cs;
          sincos(fpos * a.inv_freq[j], &sn, &cs);
          put(s, t, u * cs - w * sn);
          put(s + NS / 2, t, u * sn + w * cs);
        }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const int d = 16 * s + 8 * g + t;  // pair (d, d + 1), frequency index d/2
          double u = valid ? ld_q<DT>(a.q, qb + d) : 0.0;
          double w = valid ? ld_q<DT>(a.q, qb + d + 1) : 0.0;
          double sn, cs;
          sincos(fpos * a.inv_freq[d / 2], &sn, &cs);
          put(s, t, u * cs - w * sn);
          put(s, t + 1, u * sn + w * cs);
        }
    }
  }

  f32x16_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * BK;
    __syncthreads();
    // K block -> Ks[plane][key][d]
    for (int item = tid; item < BK * (D / 8); item += 256) {
      int key = item / (D / 8), c = item % (D / 8);
      u32x4_t hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
      if (k0 + key < T) ld8_split<DT>(a.k, ((size_t)(k0 + key) * H + kvh) * D + 8 * c, &hi, &lo);
      *reinterpret_cast<u32x4_t*>(&Ks[0][key * KS + 8 * c]) = hi;
      if constexpr (NPL == 2) *reinterpret_cast<u32x4_t*>(&Ks[NPL - 1][key * KS + 8 * c]) = lo;
    }
    // V block -> Vt[plane][d][key], two keys packed per 32-bit store
    for (int item = tid; item < (BK / 2) * (D / 8); item += 256) {
      int pr = item / (D / 8), c = item % (D / 8);
      int key0 = k0 + 2 * pr;
      u32x4_t h0 = {0u, 0u, 0u, 0u}, l0 = h0, h1 = h0, l1 = h0;
      if (key0 < T) ld8_split<DT>(a.v, ((size_t)key0 * H + kvh) * D + 8 * c, &h0, &l0);
      if (key0 + 1 < T) ld8_split<DT>(a.v, ((size_t)(key0 + 1) * H + kvh) * D + 8 * c, &h1, &l1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        uint32_t x0 = (h0[e >> 1] >> sh) & 0xffffu, x1 = (h1[e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint32_t*>(&Vt[0][(8 * c + e) * VTS + 2 * pr]) = x0 | (x1 << 16);
        if constexpr (NPL == 2) {
          uint32_t y0 = (l0[e >> 1] >> sh) & 0xffffu, y1 = (l1[e >> 1] >> sh) & 0xffffu;
          *reinterpret_cast<uint32_t*>(&Vt[NPL - 1][(8 * c + e) * VTS + 2 * pr]) = y0 | (y1 << 16);
        }
      }
    }
    __syncthreads();
    if (!active) continue;

    // S^T = K . Q^T for 64 keys (two 32-key tiles)
    f32x16_t st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[kt][v] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int ofs = (kt * 32 + col) * KS + 16 * s + 8 * g;
        bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&Ks[0][ofs]);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, __builtin_bit_cast(bf16x8_t, qh[s]), st[kt], 0, 0, 0);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, __builtin_bit_cast(bf16x8_t, ql[s]), st[kt], 0, 0, 0);
        if constexpr (NPL == 2) {
          bf16x8_t kl = *reinterpret_cast<const bf16x8_t*>(&Ks[NPL - 1][ofs]);
          st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, __builtin_bit_cast(bf16x8_t, qh[s]), st[kt], 0, 0, 0);
        }
      }
    }
    // scale, causal mask, block max
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int key = k0 + kt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        float z = key <= pos ? st[kt][v] * sl2 : -INFINITY;
        st[kt][v] = z;
        bm = fmaxf(bm, z);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = st[kt][v] == -INFINITY ? 0.f : exp2f(st[kt][v] - m_new);
        st[kt][v] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][v] *= alpha;

    // O^T += V^T . P^T ; k-step (kt, h2): keys kt*32 + 16*h2 + 4*g + {0..3, 8..11}
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4_t ph, pl;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          float p0 = st[kt][8 * h2 + 2 * h], p1 = st[kt][8 * h2 + 2 * h + 1];
          uint32_t a0 = bf16_bits_rne(p0), a1 = bf16_bits_rne(p1);
          float r0 = p0 - __uint_as_float(a0 << 16), r1 = p1 - __uint_as_float(a1 << 16);
          ph[h] = a0 | (a1 << 16);
          pl[h] = bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16);
        }
        const bf16x8_t pfh = __builtin_bit_cast(bf16x8_t, ph);
        const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, pl);
        const int kofs = kt * 32 + 16 * h2 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int ofs = (dt * 32 + col) * VTS + kofs;
          u32x2_t lo = *reinterpret_cast<const u32x2_t*>(&Vt[0][ofs]);
          u32x2_t hi = *reinterpret_cast<const u32x2_t*>(&Vt[0][ofs + 8]);
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, (u32x4_t){lo[0], lo[1], hi[0], hi[1]});
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pfh, o[dt], 0, 0, 0);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pfl, o[dt], 0, 0, 0);
          if constexpr (NPL == 2) {
            u32x2_t lo2 = *reinterpret_cast<const u32x2_t*>(&Vt[NPL - 1][ofs]);
            u32x2_t hi2 = *reinterpret_cast<const u32x2_t*>(&Vt[NPL - 1][ofs + 8]);
            const bf16x8_t vl = __builtin_bit_cast(bf16x8_t, (u32x4_t){lo2[0], lo2[1], hi2[0], hi2[1]});
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, pfh, o[dt], 0, 0, 0);
          }
        }
      }
  }

  if (!valid) return;
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const size_t obase = ((size_t)row * Hq + hq) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      int d0 = dt * 32 + 8 * v4 + 4 * g;
      float r0 = o[dt][4 * v4] * inv_l, r1 = o[dt][4 * v4 + 1] * inv_l;
      float r2 = o[dt][4 * v4 + 2] * inv_l, r3 = o[dt][4 * v4 + 3] * inv_l;
      if constexpr (DT == CT_BF16) {
        u32x2_t w = {bf16_bits_rne(r0) | (bf16_bits_rne(r1) << 16), bf16_bits_rne(r2) | (bf16_bits_rne(r3) << 16)};
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) = w;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + obase + d0) = make_float4(r0, r1, r2, r3);
      }
    }
  if (a.lse && g == 0)
    a.lse[(size_t)row * Hq + hq] = l_run > 0.f ? 0.6931471805599453f * (m_run + log2f(l_run)) : -INFINITY;
}

template <int DT, int D>
ct_status launch(const AttnArgs& a, hipStream_t stream) {
  const int ntiles = (a.n_q + 31) / 32;
  const int units = ntiles * a.group;
  dim3 grid((units + 3) / 4, a.H);
  {
    TimedLaunch tl_("attention", stream);
    hipLaunchKernelGGL((k_attn<DT, D>), grid, dim3(256), 0, stream, a);
  }
  return check_launch("attention");
}

}  // namespace

ct_status attn_f32_run(const AttnArgs& a, hipStream_t stream) {
  if (a.n_q == 0) return CT_OK;
  return a.D == 128 ? launch<CT_F32, 128>(a, stream) : launch<CT_F32, 64>(a, stream);
}

}  // namespace ct

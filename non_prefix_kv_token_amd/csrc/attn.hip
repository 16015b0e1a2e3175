// Selected-query causal GQA attention, bf16 storage -- "Adaptive KV Cache
// Reuse for Fast Long-Context LLM Serving" (CacheTune), Sec. 4.1
// "Recomputing in the new context" and App. B.2 (check layer: the selected
// positions' queries attend over the complete assembled layer under the
// causal mask).
//
// Flash-style kernel on the gfx950 matrix cores, computed transposed so that a
// query's softmax row lives in the two lanes (lane, lane ^ 32) of one wave:
//   S^T (keys x queries) = K . Q^T    A = K rows from LDS,   B = Q (registers)
//   O^T (dims x queries) += V^T . P^T A = V^T from LDS,      B = P (registers)
// MFMA layouts (32x32x16): A lane -> row lane%32, k-group lane/32 (8 values);
// B lane -> col lane%32, k-group lane/32; D lane -> col lane%32, rows
// 8*(v/4) + 4*(lane/32) + v%4.  The contraction index inside a k-group only has
// to agree between A and B, which lets P stay in the accumulator layout: V^T is
// written to LDS with its keys permuted so that each lane's 8 keys of a k-step
// are contiguous (one 16-byte read).
//
// Work decomposition.  A block of 8 waves shares one KV head and one 64-key
// K/V block in LDS (double-buffered, next block prefetched into registers
// while the current one is consumed).  Each wave owns 32 query rows of one
// query head of the group (grouped-query attention: the 4 query heads of a KV
// head and 2 row tiles for a group of 4).  The causal key range of such a
// tile group is cut into segments of S keys (split-KV) so that long rows do
// not serialise the launch; a row whose keys span several segments gets
// partial results (normalised output and log2-sum-exp) that k_attn_merge
// combines.  The grid is persistent: one block per CU, block b serving KV
// head b % H (blocks are dealt round-robin over the 8 XCDs, so each XCD's L2
// holds one head's keys), taking (tile group, segment) items from a per-head
// counter in the order the set-up launch computed from the query positions,
// longest first.
//
// Precision.  The recomputed query is stored rotated, like a rotated key: the
// set-up launch rotates it to its position in fp64 and rounds it once to bf16,
// and the products take that stored value (bf16 x bf16 exact in fp32, fp32
// accumulation).  The softmax scale (times log2 e) is applied to the fp32
// logits inside the exponent, exp2(s * c - m), one fused multiply-add.
// Probabilities and V enter the PV product as fp16 (11 bits): bf16 V converts
// to fp16 exactly whenever |v| < 65536 (values below 2^-14 land on the fp16
// subnormal grid, an absolute change below 2^-25).  A 64-key block holding a
// larger or non-finite V falls back to bf16 V with P as a bf16 hi + lo pair.
// Softmax runs in fp32 with exp2; the running maximum is only raised when a
// block's maximum exceeds it by more than 8 (log2 units), so probabilities stay
// below 2^8 and most blocks skip the accumulator rescale.
#include <climits>
#include <mutex>

#include "ct_device.h"
#include "ct_internal.h"

namespace ct {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int BK = 64;              // keys per LDS block
constexpr int VTS = BK + 8;         // V^T row stride (16-bit elements): 144 B
constexpr float kLazyThr = 8.f;     // running-max slack before a rescale (log2 units)

__device__ inline float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack_f16(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Column of key u (0..63) in the permuted V^T layout: inside each group of 16
// keys, keys {4h+i, 8+4h+i} (h = 0, 1; i < 4) go to columns 8h+i and 8h+4+i.
__device__ inline int vt_col(int u) {
  int w = u & 15;
  return (u & ~15) + 8 * ((w & 7) >> 2) + (w & 3) + 4 * (w >> 3);
}

// Preparation of V for the fp16 PV product, one (64-key tile, KV head) per
// call: V^T tiles of 64 keys, fp16, keys permuted inside each group of 16
// (vt_col), laid out exactly as the attention kernel keeps them in LDS, plus
// one flag per tile that is set when a value does not fit fp16 (|v| >= 65536,
// or not finite).  Keys at and beyond T are zero.  The tile passes through
// LDS with rows padded by one 32-bit word, so that the column reads of the
// transpose fall in distinct banks.
template <int D>
__device__ void prep_v_tile(const AttnArgs& a, int kb, int h, uint16_t* tile) {
  constexpr int TS = D + 2;       // padded row (16-bit elements)
  constexpr int CH = BK * D / 8;  // 16-byte chunks per tile
  const int tid = threadIdx.x;
  const int H = a.H, T = a.T;
  const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v);
#pragma unroll
  for (int c = tid; c < CH; c += 256) {
    const int key = kb * BK + c / (D / 8), part = c % (D / 8);
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (key < T) w = *reinterpret_cast<const u32x4_t*>(Vg + ((size_t)key * H + h) * D + 8 * part);
    uint32_t* t = reinterpret_cast<uint32_t*>(&tile[(c / (D / 8)) * TS + 8 * part]);
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = w[i];  // 4-byte aligned only (padded rows)
  }
  __syncthreads();
  uint32_t wide = 0u;
  uint16_t* dst = a.vt16 + ((size_t)h * a.nblk + kb) * D * BK;
#pragma unroll
  for (int c = tid; c < CH; c += 256) {
    const int d = c / (BK / 8), q0 = 8 * (c % (BK / 8));
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qa = q0 + 2 * e, qb = qa + 1;
      // key at column q: bits 2 and 3 of its index inside the group swapped
      const int ua = (qa & ~15) | ((qa & 4) << 1) | ((qa & 8) >> 1) | (qa & 3);
      const int ub = (qb & ~15) | ((qb & 4) << 1) | ((qb & 8) >> 1) | (qb & 3);
      const uint32_t xa = tile[ua * TS + d], xb = tile[ub * TS + d];
      wide = max(wide, max(xa & 0x7fffu, xb & 0x7fffu));
      w[e] = pack_f16(__uint_as_float(xa << 16), __uint_as_float(xb << 16));
    }
    *reinterpret_cast<u32x4_t*>(dst + (size_t)d * BK + q0) = w;
  }
  // 0x4780 is 65536 in bf16: the first magnitude fp16 cannot hold
  const int any_wide = __syncthreads_or((int)(wide >= 0x4780u));
  if (tid == 0) a.vflag[h * a.nblk + kb] = any_wide;
}

// Per-layer rotation of the queries: every selected row's query, turned to
// the row's position in fp64 (angle, sine, cosine and rotation) and rounded
// once to bf16 -- the stored rotated query, as the assembly stores rotated
// keys.  kQRows rows per call: the sines and cosines of a row's D/2 angles are
// formed once into LDS and shared by its Hq heads; a thread then rotates 8
// pairs of one head (two 16-byte loads and stores), with the loads of all its
// items issued before the arithmetic.
constexpr int kQRows = 4;
template <int D>
__device__ void prep_q_rows(const AttnArgs& a, int row0, char* smem) {
  constexpr int NP = D / 2;   // rotation pairs per head
  constexpr int NG = NP / 8;  // groups of 8 pairs per head
  double2* sc = reinterpret_cast<double2*>(smem);  // [kQRows][NP]: sine, cosine
  const int tid = threadIdx.x;
  for (int i = tid; i < kQRows * NP; i += 256) {
    const int row = row0 + i / NP, j = i % NP;
    double sn = 0.0, cs = 1.0;
    if (row < a.n_q) rope_sincos((double)min(a.qpos[row], a.T - 1) * a.inv_freq[j], &sn, &cs);
    sc[i] = make_double2(sn, cs);
  }
  __syncthreads();
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const bool half = a.style == CT_ROPE_HALF;
  const int per_row = a.Hq * NG;
  // Hq is at most a few hundred: per_row * kQRows items, up to kIt per thread
  constexpr int kIt = 4;
  for (int it0 = tid; it0 < kQRows * per_row; it0 += 256 * kIt) {
    u32x4_t xa[kIt], xb[kIt];
    size_t off_a[kIt], off_b[kIt];
    bool ok[kIt];
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      const int it = it0 + 256 * u;
      const int rr = it / per_row, h = (it % per_row) / NG, gq = it % NG;
      ok[u] = it < kQRows * per_row && row0 + rr < a.n_q;
      const size_t base = ((size_t)(ok[u] ? row0 + rr : 0) * a.Hq + (ok[u] ? h : 0)) * D;
      // half: dims 8gq.. (first of each pair) and NP + 8gq.. (second);
      // interleaved: dims 16gq .. 16gq + 15 (pairs side by side)
      off_a[u] = base + (half ? 8 * gq : 16 * gq);
      off_b[u] = base + (half ? NP + 8 * gq : 16 * gq + 8);
      xa[u] = *reinterpret_cast<const u32x4_t*>(q + off_a[u]);
      xb[u] = *reinterpret_cast<const u32x4_t*>(q + off_b[u]);
    }
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      if (!ok[u]) continue;
      const int it = it0 + 256 * u;
      const int rr = it / per_row, gq = it % NG;
      const double2* scr = sc + rr * NP + 8 * gq;  // pairs 8gq .. 8gq + 7
      auto el = [](const u32x4_t& w, int t) {
        return (double)((t & 1) ? bf16_hi_to_f32(w[t >> 1]) : bf16_lo_to_f32(w[t >> 1]));
      };
      u32x4_t ya = {0u, 0u, 0u, 0u}, yb = {0u, 0u, 0u, 0u};
      auto rot = [&](int t, double& r0, double& r1) {
        const double2 c = scr[t];
        double x0, x1;
        if (half) {
          x0 = el(xa[u], t);
          x1 = el(xb[u], t);
        } else {
          x0 = t < 4 ? el(xa[u], 2 * t) : el(xb[u], 2 * t - 8);
          x1 = t < 4 ? el(xa[u], 2 * t + 1) : el(xb[u], 2 * t - 7);
        }
        r0 = x0 * c.y - x1 * c.x;
        r1 = x0 * c.x + x1 * c.y;
      };
      // Rounded to fp32 and then to bf16 (both to nearest even): the one
      // rounding of the fp64 value unless the fp32 result lies exactly on a
      // bf16 midpoint (fp32 holds every bf16 midpoint, so otherwise the two
      // lie on the same side of each); a lane that meets one rounds its 16
      // values once from the fp64 bits instead.
      uint32_t f0[8], f1[8];
      bool mid = false;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        double r0, r1;
        rot(t, r0, r1);
        f0[t] = __float_as_uint((float)r0);
        f1[t] = __float_as_uint((float)r1);
        mid |= ((f0[t] & 0xffffu) == 0x8000u) | ((f1[t] & 0xffffu) == 0x8000u);
      }
      if (__builtin_expect(mid, 0)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          double r0, r1;
          rot(t, r0, r1);
          f0[t] = (uint32_t)bf16_from_f64(r0) << 16;  // a bf16 value: the rounding below keeps it
          f1[t] = (uint32_t)bf16_from_f64(r1) << 16;
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t y0 = bf16_bits_rne(__uint_as_float(f0[t])), y1 = bf16_bits_rne(__uint_as_float(f1[t]));
        if (half) {
          ya[t >> 1] |= y0 << (16 * (t & 1));
          yb[t >> 1] |= y1 << (16 * (t & 1));
        } else if (t < 4) {
          ya[t] = y0 | (y1 << 16);
        } else {
          yb[t - 4] = y0 | (y1 << 16);
        }
      }
      *reinterpret_cast<u32x4_t*>(a.qrot + off_a[u]) = ya;
      *reinterpret_cast<u32x4_t*>(a.qrot + off_b[u]) = yb;
    }
  }
}

// Maximum of a lane's 16 logits with the 3-input maximum (no canonicalising
// moves; NaN propagates).
__device__ inline float max16(const f32x16_t& s) {
  auto mx3 = [](float x, float y, float z) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
  };
  const float m0 = mx3(s[0], s[1], s[2]), m1 = mx3(s[3], s[4], s[5]), m2 = mx3(s[6], s[7], s[8]);
  const float m3 = mx3(s[9], s[10], s[11]), m4 = mx3(s[12], s[13], s[14]);
  return __builtin_elementwise_maximum(mx3(mx3(m0, m1, m2), m3, m4), s[15]);
}

// NW waves per block; each wave owns QT tiles of 32 query rows of one query
// head.  QT = 2 runs one wave per SIMD with the whole register file, so every
// K / V^T fragment read from LDS feeds two tiles; QT = 1 runs two waves per
// SIMD.
template <int D, int NW, int QT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 2 : 1, QT == 1 ? 2 : 1)))
void k_attn_bf16(AttnArgs a) {
  constexpr int NT = 64 * NW;        // threads per block
  constexpr int KS = D + 8;          // K row stride (bf16): 16-byte reads conflict-free
  constexpr int NS = D / 16;         // k-steps over the head dimension
  constexpr int NDT = D / 32;        // output tiles over the head dimension
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int KIT = BK * KCH / NT; // K chunks staged per thread
  constexpr int NDG = NT / 32;       // V staging: 32 key pairs x NDG dim groups
  constexpr int DPG = D / NDG;       // V dims per thread (2 keys x DPG dims)
  static_assert(KIT >= 1 && BK * KCH == KIT * NT, "K staging split");
  static_assert(DPG >= 4 && DPG % 4 == 0, "V staging split");
  // K and V^T rings of four 64-key blocks: blocks are staged two ahead, so
  // one barrier every other block orders both the writes before their reads
  // and the reads before the slot is written again.
  __shared__ __attribute__((aligned(16))) uint16_t Ks[4][BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[4][D * VTS];  // V^T: fp16 (bf16 when redone)
  __shared__ int s_wmax[NW];
  __shared__ int s_item;

  const int H = a.H, G = a.group, T = a.T, Hq = a.Hq, S = a.seg_keys;

  // ---- persistent blocks: block b serves KV head b % H (blocks are dealt
  // round-robin over the XCDs, so each XCD's L2 holds one head's keys) and
  // takes that head's work items -- (tile group, segment) pairs in the order
  // k_attn_sched wrote, longest first, times the head chunks -- from a
  // counter until none are left.
  const int kvh = blockIdx.x % H;
  const int n_work = a.sched_n[0] * a.n_hc;
  for (;;) {
  // Lane indices pass through an empty asm once per item: address arithmetic
  // that depends on them is then formed inside the item, not hoisted out of
  // this loop, where it would hold registers across the whole kernel.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  __syncthreads();  // the previous item's LDS reads and s_item are done
  if (tid == 0) s_item = atomicAdd(&a.sched_cnt[kvh], 1);
  __syncthreads();
  const int item = s_item;
  if (item >= n_work) break;
  const int e_ = a.sched_order[item / a.n_hc];
  const int tg = e_ / a.nseg, seg = e_ % a.nseg;
  const int hc = item % a.n_hc;
  const int wt = wave / a.hpb, wh = wave % a.hpb;
  const int tile0 = (tg * a.tpb + wt) * QT;  // first 32-row tile of the wave
  const int hig = hc * a.hpb + wh;           // head inside the group
  const bool wave_on = wt < a.tpb && hig < G && tile0 * 32 < a.n_q;
  const int hq = kvh * G + hig;
  int row[QT], pos[QT];
  bool valid[QT];
  int wmax = -1, wmin = INT_MAX;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    row[qt] = (tile0 + qt) * 32 + col;
    valid[qt] = wave_on && row[qt] < a.n_q;
    pos[qt] = valid[qt] ? min(a.qpos[row[qt]], T - 1) : -1;
    wmax = max(wmax, pos[qt]);
    if (valid[qt]) wmin = min(wmin, pos[qt]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, o));
    wmin = min(wmin, __shfl_xor(wmin, o));
  }
  if (lane == 0) s_wmax[wave] = wmax;
  __syncthreads();
  int bmax = -1;
#pragma unroll
  for (int w = 0; w < NW; ++w) bmax = max(bmax, s_wmax[w]);
  const int nkeys = bmax + 1;
  const int seg_lo = seg * S;
  if (seg_lo >= nkeys) continue;  // uniform over the block
  const int seg_hi = min(seg_lo + S, nkeys);
  const int kb0 = seg_lo / BK, kb1 = (seg_hi + BK - 1) / BK;

  // ---- the stored rotated query (B operand, bf16, written by the set-up
  // launch).  The lane's dims of k-step s are 16*s + 8*g + t (t < 8).
  // (Loaded by prep_q, which is called once the first K/V block's loads are
  // out, so that their latencies overlap.)
  u32x4_t qh[QT][NS];
  auto prep_q = [&]() {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const uint16_t* qp = a.qrot + ((size_t)(valid[qt] ? row[qt] : 0) * Hq + hq) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qh[qt][s] = *reinterpret_cast<const u32x4_t*>(qp + 16 * s);
        if (!valid[qt]) qh[qt][s] = (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
  };

  // ---- staging: K rows as 16-byte chunks; V as 2 keys x DPG dims per thread
  const uint16_t* Kg = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v);
  const int kp = tid & 31, dg = tid >> 5;  // V: key pair, dim group
  u32x4_t kreg[KIT];
  uint32_t vreg[2][DPG / 2];

  auto load = [&](int kb) {
    const int k0 = kb * BK;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int item = tid + it * NT;
      const int key = k0 + item / KCH, ch = item % KCH;
      kreg[it] = (u32x4_t){0u, 0u, 0u, 0u};
      if (key < T) kreg[it] = *reinterpret_cast<const u32x4_t*>(Kg + ((size_t)key * H + kvh) * D + 8 * ch);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = k0 + 2 * kp + e;
      const uint16_t* src = Vg + ((size_t)key * H + kvh) * D + dg * DPG;
      if constexpr (DPG >= 8) {
#pragma unroll
        for (int c8 = 0; c8 < DPG / 8; ++c8) {
          u32x4_t w = {0u, 0u, 0u, 0u};
          if (key < T) w = *reinterpret_cast<const u32x4_t*>(src + 8 * c8);
#pragma unroll
          for (int i = 0; i < 4; ++i) vreg[e][4 * c8 + i] = w[i];
        }
      } else {
        u32x2_t w = {0u, 0u};
        if (key < T) w = *reinterpret_cast<const u32x2_t*>(src);
        vreg[e][0] = w[0];
        vreg[e][1] = w[1];
      }
    }
  };

  // main pass: the V^T tile prepared by k_attn_prep, copied as it is
  constexpr int VIT = D * BK / 8 / NT;  // 16-byte V^T chunks per thread
  u32x4_t vtreg[VIT];
  // K rows through a buffer resource based at key k0 of this head whose range
  // ends at the end of K: rows at and past T read as zero without a branch
  // (the whole offset is in the VGPR operand, so the range check covers it).
  auto load_fast = [&](int kb) {
    const int k0 = kb * BK;
    const long long rem = ((long long)(T - k0) * H - kvh) * D * 2;
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Kg + ((size_t)k0 * H + kvh) * D), 0,
        (int)(rem < 0x7fffffffLL ? rem : 0x7fffffffLL), 0x00020000);
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int item = tid + it * NT;
      const int voff = ((item / KCH) * H * D + 8 * (item % KCH)) * 2;
      kreg[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(kres, voff, 0, 0));
    }
    const u32x4_t* vt = reinterpret_cast<const u32x4_t*>(a.vt16 + ((size_t)kvh * a.nblk + kb) * D * BK);
#pragma unroll
    for (int it = 0; it < VIT; ++it) vtreg[it] = vt[tid + it * NT];
  };
  auto store_fast = [&](int kbuf_i, int buf) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int item = tid + it * NT;
      *reinterpret_cast<u32x4_t*>(&Ks[kbuf_i][(item / KCH) * KS + 8 * (item % KCH)]) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int c = tid + it * NT;
      *reinterpret_cast<u32x4_t*>(&Vs[buf][(c / (BK / 8)) * VTS + 8 * (c % (BK / 8))]) = vtreg[it];
    }
  };

  // fallback pass: V^T transposed here, as bf16
  auto store = [&](int kbuf_i, int buf) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int item = tid + it * NT;
      *reinterpret_cast<u32x4_t*>(&Ks[kbuf_i][(item / KCH) * KS + 8 * (item % KCH)]) = kreg[it];
    }
    const int cpos = vt_col(2 * kp);
#pragma unroll
    for (int i = 0; i < DPG / 2; ++i) {
      const uint32_t w0 = vreg[0][i], w1 = vreg[1][i];  // dims 2i, 2i+1 of keys 2kp, 2kp+1
      const int d0 = dg * DPG + 2 * i;
      *reinterpret_cast<uint32_t*>(&Vs[buf][d0 * VTS + cpos]) = (w0 & 0xffffu) | (w1 << 16);
      *reinterpret_cast<uint32_t*>(&Vs[buf][(d0 + 1) * VTS + cpos]) = (w0 >> 16) | (w1 & 0xffff0000u);
    }
  };

  f32x16_t o[QT][NDT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[qt][i][v] = 0.f;
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  // S^T = K . Q^T for the 64 keys of a buffer: each K fragment feeds all QT
  // tiles; causal mask where the block reaches past the wave's first row.
  auto scores = [&](const uint16_t* kbuf, int k0, f32x16_t (*st)[2]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[qt][kt][v] = 0.f;
    // fragments of the next k-step are read before the MFMAs of this one
    const uint16_t* kb_ = kbuf + col * KS + 8 * g;
    bf16x8_t ka[2], kn[2];
    ka[0] = *reinterpret_cast<const bf16x8_t*>(kb_);
    ka[1] = *reinterpret_cast<const bf16x8_t*>(kb_ + 32 * KS);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + 1 < NS) {
        kn[0] = *reinterpret_cast<const bf16x8_t*>(kb_ + 16 * (s + 1));
        kn[1] = *reinterpret_cast<const bf16x8_t*>(kb_ + 32 * KS + 16 * (s + 1));
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, qh[qt][s]);
        st[qt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], bh, st[qt][0], 0, 0, 0);
        st[qt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[1], bh, st[qt][1], 0, 0, 0);
      }
      if (s + 1 < NS) {
        ka[0] = kn[0];
        ka[1] = kn[1];
      }
    }
    if (k0 + BK - 1 > wmin) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + kt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
            if (key > pos[qt]) st[qt][kt][v] = -INFINITY;
          }
    }
  };

  // Online softmax of one 32-key tile of tile qt (16 logits per lane): lazy
  // maximum, probabilities exp2(s - m) in place.
  const float cq = a.scale_log2;  // > 0: the scale commutes with the maximum
  auto softmax_tile = [&](int qt, f32x16_t& st) {
    const float bm = max16(st) * cq;
    if (__any(bm > m_run[qt] + kLazyThr)) {
      const float m_new = fmaxf(m_run[qt], fmaxf(bm, __shfl_xor(bm, 32)));
      const float alpha = m_run[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qt] - m_new);
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[qt][i][v] *= alpha;
      l_run[qt] *= alpha;
      m_run[qt] = m_new;
    }
    const float mu = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], cq, -mu));
  };

  // P^T . V^T for one 64-key block (probabilities in st, fp16), row sums from
  // the rounded probabilities.
  const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  // One lazy-maximum decision covers the whole 64-key block, so that the
  // exponentials of the second 32-key tile and the products of the first sit
  // in one scheduling region (no branch between them) and can interleave.
  auto pv = [&](const uint16_t* vbuf, f32x16_t (*st)[2]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float bm = __builtin_elementwise_maximum(max16(st[qt][0]), max16(st[qt][1])) * cq;
      if (__any(bm > m_run[qt] + kLazyThr)) {
        const float m_new = fmaxf(m_run[qt], fmaxf(bm, __shfl_xor(bm, 32)));
        const float alpha = m_run[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qt] - m_new);
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[qt][i][v] *= alpha;
        l_run[qt] *= alpha;
        m_run[qt] = m_new;
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mu = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
#pragma unroll
        for (int v = 0; v < 16; ++v) st[qt][kt][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[qt][kt][v], cq, -mu));
      }
      // O^T += V^T . P^T ; k-step (kt, h2) covers keys kt*32 + 16*h2 + [0, 16)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        // (the dot product takes the converted pair itself: hipcc reads the
        // wrong register when it is given a bit-cast element of pw)
        f16x8_t pf[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          u32x4_t pw;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const f32x2_t pv2 = {st[qt][kt][8 * h2 + 2 * h], st[qt][kt][8 * h2 + 2 * h + 1]};
            const f16x2_t ph = __builtin_convertvector(pv2, f16x2_t);
            l_run[qt] = __builtin_amdgcn_fdot2(ph, ones, l_run[qt], false);
            pw[h] = __builtin_bit_cast(uint32_t, ph);
          }
          pf[qt] = __builtin_bit_cast(f16x8_t, pw);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f16x8_t va = *reinterpret_cast<const f16x8_t*>(
              &vbuf[(dt * 32 + col) * VTS + 32 * kt + 16 * h2 + 8 * g]);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[qt], o[qt][dt], 0, 0, 0);
        }
      }
    }
  };

  // Main pass: P and V^T as fp16.  A segment with a V tile that does not fit
  // fp16 takes the pass below instead: bf16 V and P as a bf16 pair.
  // the fp16 path needs every V tile of the segment to fit fp16
  // (the segment's flags are read by the lanes in parallel and combined)
  bool wide_v = false;
  for (int kb = kb0 + lane; kb < kb1; kb += 64) wide_v |= a.vflag[kvh * a.nblk + kb] != 0;
  // The first block's loads go out before the flags are known (they stay in
  // bounds either way; the bf16 pass reloads), then the query's.
  load_fast(kb0);
  prep_q();
  const bool redo = __any(wide_v);
  f32x16_t st[QT][2];
  if (!redo) {
    store_fast(0, 0);
    if (kb0 + 1 < kb1) {
      load_fast(kb0 + 1);
      store_fast(1, 1);
    }
  }
  // The query operands are complete before the loop: the compiler's wait
  // counting would otherwise treat them as pending inside the loop and make
  // every k-block wait for the next block's prefetch.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(qh[qt][s]));
  for (int kb = kb0; kb < kb1 && !redo; ++kb) {
    const int i = kb - kb0, c = i & 3;
    const bool more = kb + 2 < kb1;
    // Block kb + 2 goes to slot (i + 2) & 3, last read at block i - 2.  A
    // barrier at the start of every even block lies between each store
    // (block i) and its reads (block i + 2), and between the reads of a slot
    // (block i - 2) and its next store (block i).
    if ((i & 1) == 0) __syncthreads();
    if (more) load_fast(kb + 2);
    const int k0 = kb * BK;
    if (wave_on && k0 <= wmax) {
      // The score products run at raised wave priority: of the two waves
      // sharing a SIMD, the one in its matrix phase gets the issue slots, and
      // the other drifts into the complementary (softmax) phase.
      __builtin_amdgcn_s_setprio(2);
      scores(Ks[c], k0, st);
      __builtin_amdgcn_s_setprio(0);
      pv(Vs[c], st);
    }
    if (more) store_fast((i + 2) & 3, (i + 2) & 3);
  }

  if (redo) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[qt][i][v] = 0.f;
      m_run[qt] = -INFINITY;
      l_run[qt] = 0.f;
    }
    for (int kb = kb0; kb < kb1; ++kb) {
      __syncthreads();  // previous readers of buffer 0 are done
      load(kb);
      store(0, 0);
      __syncthreads();
      const int k0 = kb * BK;
      if (wave_on && k0 <= wmax) {
        f32x16_t st[QT][2];
        scores(Ks[0], k0, st);
#pragma unroll 1
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            softmax_tile(qt, st[qt][kt]);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              u32x4_t ph, pl;
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                const float p0 = st[qt][kt][8 * h2 + 2 * h], p1 = st[qt][kt][8 * h2 + 2 * h + 1];
                l_run[qt] += p0 + p1;
                const uint32_t a0 = bf16_bits_rne(p0), a1 = bf16_bits_rne(p1);
                ph[h] = a0 | (a1 << 16);
                pl[h] = bf16_bits_rne(p0 - __uint_as_float(a0 << 16)) |
                        (bf16_bits_rne(p1 - __uint_as_float(a1 << 16)) << 16);
              }
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(
                    &Vs[0][(dt * 32 + col) * VTS + 32 * kt + 16 * h2 + 8 * g]);
                o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, __builtin_bit_cast(bf16x8_t, ph), o[qt][dt], 0, 0, 0);
                o[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, __builtin_bit_cast(bf16x8_t, pl), o[qt][dt], 0, 0, 0);
              }
            }
          }
        }
      }
    }
  }

  if (!wave_on) continue;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float l_tot = l_run[qt] + __shfl_xor(l_run[qt], 32);
    if (!valid[qt] || pos[qt] < seg_lo) continue;
    const float inv_l = 1.f / l_tot;
    const float lse2 = m_run[qt] + __log2f(l_tot);
    if (seg == 0 && pos[qt] < S) {  // every key of this row lies in segment 0
      const size_t obase = ((size_t)row[qt] * Hq + hq) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d0 = dt * 32 + 8 * v4 + 4 * g;
          const f32x16_t& oo = o[qt][dt];
          u32x2_t w = {bf16_bits_rne(oo[4 * v4] * inv_l) | (bf16_bits_rne(oo[4 * v4 + 1] * inv_l) << 16),
                       bf16_bits_rne(oo[4 * v4 + 2] * inv_l) | (bf16_bits_rne(oo[4 * v4 + 3] * inv_l) << 16)};
          *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) = w;
        }
      if (a.lse && g == 0) a.lse[(size_t)row[qt] * Hq + hq] = 0.6931471805599453f * lse2;
    } else {
      // A partial is a convex combination of V rows: with every V of the
      // segment inside the fp16 range it is stored as fp16 (half the bytes
      // for this kernel and the merge), else as fp32.
      const size_t pb = (((size_t)seg * a.n_q + row[qt]) * Hq + hq);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const int d0 = dt * 32 + 8 * v4 + 4 * g;
          const f32x16_t& oo = o[qt][dt];
          if (!redo)
            *reinterpret_cast<u32x2_t*>(a.part_o16 + pb * D + d0) =
                (u32x2_t){pack_f16(oo[4 * v4] * inv_l, oo[4 * v4 + 1] * inv_l),
                          pack_f16(oo[4 * v4 + 2] * inv_l, oo[4 * v4 + 3] * inv_l)};
          else
            *reinterpret_cast<float4*>(a.part_o + pb * D + d0) =
                make_float4(oo[4 * v4] * inv_l, oo[4 * v4 + 1] * inv_l, oo[4 * v4 + 2] * inv_l,
                            oo[4 * v4 + 3] * inv_l);
        }
      if (g == 0) {
        a.part_lse[pb] = lse2;
        a.part_fmt[pb] = redo ? 1 : 0;
      }
    }
  }
  }  // work items
}

// Work list of the persistent attention blocks (one block): the key range
// of each tile group (its rows' largest position), the number of 64-key
// blocks each (tile group, segment) pair covers, and the pairs that have
// work, sorted longest first: each KV head's blocks take the long items
// before the short ones, which keeps the tail of the launch short.  Lists
// longer than kSchedMax pairs keep the natural order (segment by segment,
// latest rows first) with the empty pairs included.  Also resets the
// per-head item counters.
constexpr int kSchedMax = 2048;
__device__ void build_schedule(const AttnArgs& a, char* smem) {
  unsigned long long* s_key = reinterpret_cast<unsigned long long*>(smem);
  int* s_bmax = reinterpret_cast<int*>(smem + kSchedMax * 8);
  int* s_n = s_bmax + kSchedMax;
  const int tid = threadIdx.x;
  const int n_tg = a.n_tg, nseg = a.nseg, S = a.seg_keys;
  const int n_items = n_tg * nseg;
  for (int h = tid; h < a.H; h += 256) a.sched_cnt[h] = 0;
  if (n_items > kSchedMax) {
    for (int i = tid; i < n_items; i += 256) {
      const int seg = i / n_tg, tg = n_tg - 1 - i % n_tg;
      a.sched_order[i] = tg * nseg + seg;
    }
    if (tid == 0) a.sched_n[0] = n_items;
    return;
  }
  for (int t = tid; t < n_tg; t += 256) s_bmax[t] = -1;
  if (tid == 0) *s_n = 0;
  __syncthreads();
  const int rows_per_tg = 32 * a.tpb * a.qt;
  for (int r0 = 0; r0 < a.n_q; r0 += 256 * 8) {
    int p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // eight loads in flight per thread
      const int r = r0 + u * 256 + tid;
      p[u] = r < a.n_q ? a.qpos[r] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * 256 + tid;
      if (r < a.n_q) atomicMax(&s_bmax[r / rows_per_tg], min(p[u], a.T - 1));
    }
  }
  __syncthreads();
  int N = 1;
  while (N < n_items) N <<= 1;
  for (int i = tid; i < N; i += 256) {
    unsigned long long key = 0ull;
    if (i < n_items) {
      const int tg = i / nseg, seg = i % nseg;
      const int lo = seg * S, nkeys = s_bmax[tg] + 1;
      const int work = lo < nkeys ? (min(lo + S, nkeys) + BK - 1) / BK - lo / BK : 0;
      key = ((unsigned long long)work << 32) | (0xffffffffu - (unsigned)i);
    }
    s_key[i] = key;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < N; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long x = s_key[i], y = s_key[l];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            s_key[i] = y;
            s_key[l] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < N; i += 256) {
    const bool has = (s_key[i] >> 32) != 0;
    if (has) a.sched_order[i] = (int)(0xffffffffu - (unsigned)(s_key[i] & 0xffffffffu));
    if (has && (i + 1 == N || (s_key[i + 1] >> 32) == 0)) *s_n = i + 1;
  }
  __syncthreads();
  if (tid == 0) a.sched_n[0] = *s_n;
}

// Per-layer set-up of the attention, one launch: block 0 builds the work
// list, then one block per (64-key V tile, KV head) and one per kQRows query
// rows (their rotated bf16 queries).
template <int D>
constexpr int setup_lds_bytes() {
  return BK * (D + 2) * 2 > kSchedMax * 12 + 4 ? BK * (D + 2) * 2 : kSchedMax * 12 + 4;
}
static_assert(kQRows * 64 * 16 <= kSchedMax * 12 + 4, "query rotation tables fit the set-up LDS");
template <int D>
__global__ __launch_bounds__(256) void k_attn_setup(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[setup_lds_bytes<D>()];
  const int nv = a.nblk * a.H;
  const int b = (int)blockIdx.x - 1;
  if (b < 0)
    build_schedule(a, smem);
  else if (b < nv)
    prep_v_tile<D>(a, b % a.nblk, b / a.nblk, reinterpret_cast<uint16_t*>(smem));
  else
    prep_q_rows<D>(a, (b - nv) * kQRows, smem);
}

// Combine the per-segment results of rows whose keys span several segments:
// out = sum_s 2^(lse2_s - M) o_s / sum_s 2^(lse2_s - M).  One wave per
// (row, group of kMergeHeads query heads), 16 lanes per head holding D/16
// dims each (16-byte fp16 loads); rows in segment 0 only were written by
// k_attn_bf16.  Lanes work independently (no cross-lane operations).
constexpr int kMergeHeads = 4;
template <int D>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  constexpr int PER = D / 16;
  constexpr int U = 4;  // segments whose loads are in flight together
  typedef float fv_t __attribute__((ext_vector_type(PER)));
  typedef _Float16 hv_t __attribute__((ext_vector_type(PER)));
  const int hgroups = (a.Hq + kMergeHeads - 1) / kMergeHeads;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= a.n_q * hgroups) return;
  const int row = w / hgroups, hq = (w % hgroups) * kMergeHeads + lane / 16;
  const int dl = (lane % 16) * PER;  // this lane's first dim
  if (hq >= a.Hq) return;
  const int pos = min(a.qpos[row], a.T - 1);
  const int S = a.seg_keys;
  if (pos < S) return;
  const int ns = pos / S + 1;
  // online combination over groups of U segments: running maximum M, weight
  // sum and weighted output
  float M = -INFINITY, wsum = 0.f;
  fv_t acc = {};
  for (int s0 = 0; s0 < ns; s0 += U) {
    float ls[U];
    fv_t os[U];
    hv_t hs[U];
    int fm[U];
    // the fp16 record is loaded with the format and the lse (one round
    // trip); a record stored as fp32 (wide V, rare) is loaded after
    // (segments past the row's last read its last record, with weight 0:
    // every load is unconditional)
    int any_fp32 = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      const size_t pb = ((size_t)min(s, ns - 1) * a.n_q + row) * a.Hq + hq;
      const float lv = a.part_lse[pb];
      ls[u] = s < ns ? lv : -INFINITY;
      fm[u] = a.part_fmt[pb];
      hs[u] = *reinterpret_cast<const hv_t*>(a.part_o16 + pb * D + dl);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      os[u] = __builtin_convertvector(hs[u], fv_t);
      any_fp32 |= fm[u];
    }
    if (any_fp32) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t pb = ((size_t)min(s0 + u, ns - 1) * a.n_q + row) * a.Hq + hq;
        if (fm[u]) os[u] = *reinterpret_cast<const fv_t*>(a.part_o + pb * D + dl);
      }
    }
    float mg = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mg = fmaxf(mg, ls[u]);
    const float c = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mg);
    wsum *= c;
    acc *= c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = ls[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[u] - mg);
      wsum += wgt;
      acc += wgt * os[u];
    }
    M = mg;
  }
  const float inv = 1.f / wsum;
  typedef uint32_t uv_t __attribute__((ext_vector_type(PER / 2)));
  uv_t ov;
#pragma unroll
  for (int i = 0; i < PER / 2; ++i)
    ov[i] = bf16_bits_rne(acc[2 * i] * inv) | (bf16_bits_rne(acc[2 * i + 1] * inv) << 16);
  *reinterpret_cast<uv_t*>(reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * a.Hq + hq) * D + dl) = ov;
  if (a.lse && lane % 16 == 0) a.lse[(size_t)row * a.Hq + hq] = 0.6931471805599453f * (M + __log2f(wsum));
}

template <int D>
ct_status launch(const AttnArgs& a, hipStream_t stream) {
  {
    TimedLaunch tl_("attention_setup", stream);
    constexpr int rpb = kQRows;  // query rows per set-up block
    hipLaunchKernelGGL((k_attn_setup<D>), dim3(1 + a.nblk * a.H + (a.n_q + rpb - 1) / rpb), dim3(256), 0,
                       stream, a);
  }
  if (ct_status s = check_launch("attention set-up")) return s;
  const int blocks = a.H * a.blocks_per_head;
  {
    TimedLaunch tl_("attention", stream);
    hipLaunchKernelGGL((k_attn_bf16<D, 8, 1>), dim3(blocks), dim3(512), 0, stream, a);
  }
  if (ct_status s = check_launch("attention")) {
    set_error(std::string(cachetune_last_error()) + " [grid " + std::to_string(blocks) + ", segments " +
              std::to_string(a.nseg) + "]");
    return s;
  }
  if (a.nseg > 1) {
    const long long waves = (long long)a.n_q * ((a.Hq + kMergeHeads - 1) / kMergeHeads);
    {
      TimedLaunch tl_("attention_merge", stream);
      hipLaunchKernelGGL((k_attn_merge<D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
    }
    if (ct_status s = check_launch("attention merge")) return s;
  }
  return CT_OK;
}

}  // namespace

void attn_plan(AttnArgs* a, int n_cu) {
  const int G = a->group;
  // Block shape: 8 waves with one 32-row tile each (two waves per SIMD).
  a->nw = 8;
  a->qt = 1;
  a->hpb = G < a->nw ? G : a->nw;
  a->tpb = a->nw / a->hpb;
  a->n_hc = (G + a->hpb - 1) / a->hpb;
  const int ntiles = (a->n_q + 31) / 32;
  a->n_tg = (ntiles + a->tpb * a->qt - 1) / (a->tpb * a->qt);
  // Segment length: the causal triangle (about units * T / 2 keys of block
  // work) spread over about 1.8 items per CU (longer items mean fewer
  // partial results and merges; with the longest-first order of the work
  // list this keeps the tail short), at least 1024 keys, a multiple of the
  // LDS block.
  const long long units = (long long)a->H * a->n_tg * a->n_hc;
  long long s = units * (long long)a->T * 5 / (18LL * (n_cu > 0 ? n_cu : 256));
  if (const char* env = getenv("CACHETUNE_ATTN_SEG")) s = atoll(env);
  if (s < 1024) s = 1024;
  s = (s + BK - 1) / BK * BK;
  if (s > a->T) s = (a->T + BK - 1) / BK * BK;
  a->seg_keys = (int32_t)s;
  a->nseg = (a->T + a->seg_keys - 1) / a->seg_keys;
  a->nblk = (a->T + BK - 1) / BK;
  // persistent grid: one block per compute unit, the same number per KV head
  const int ncu = n_cu > 0 ? n_cu : 256;
  a->blocks_per_head = ncu / a->H > 0 ? ncu / a->H : 1;
}

// Workspace: [partial outputs fp32][partial outputs fp16][record formats]
// [partial log2-sum-exp][V^T fp16 tiles][tile flags][rotated bf16 queries]
// [work list, per-head counters, list length]
struct AttnWs { size_t o16, fmt, lse, vt, flag, q, sched, total; };
static AttnWs ws_layout(const AttnArgs& a) {
  AttnWs w{};
  const size_t rows = a.nseg > 1 ? (size_t)a.nseg * a.n_q * a.Hq : 0;
  size_t off = align256(rows * a.D * 4);
  w.o16 = off;
  off += align256(rows * a.D * 2);
  w.fmt = off;
  off += align256(rows);
  w.lse = off;
  off += align256(rows * 4);
  w.vt = off;
  off += align256((size_t)a.H * a.nblk * a.D * BK * 2);
  w.flag = off;
  off += align256((size_t)a.H * a.nblk * 4);
  w.q = off;
  off += align256((size_t)a.n_q * a.Hq * a.D * 2);
  w.sched = off;
  off += align256(((size_t)a.n_tg * a.nseg + a.H + 1) * 4);
  w.total = off;
  return w;
}

size_t attn_ws_bytes(const AttnArgs& a) {
  if (a.dtype != CT_BF16) return 0;
  return ws_layout(a).total;
}

ct_status attn_run(AttnArgs a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a.n_q == 0) return CT_OK;
  if (a.dtype == CT_F32) return attn_f32_run(a, stream);
  const AttnWs L = ws_layout(a);
  if (!ws || ws_bytes < L.total)
    return fail(CT_E_WORKSPACE, "attention workspace of " + std::to_string(L.total) + " bytes required");
  char* w = reinterpret_cast<char*>(ws);
  a.part_o = reinterpret_cast<float*>(w);
  a.part_o16 = reinterpret_cast<uint16_t*>(w + L.o16);
  a.part_fmt = reinterpret_cast<uint8_t*>(w + L.fmt);
  a.part_lse = reinterpret_cast<float*>(w + L.lse);
  a.vt16 = reinterpret_cast<uint16_t*>(w + L.vt);
  a.vflag = reinterpret_cast<int32_t*>(w + L.flag);
  a.qrot = reinterpret_cast<uint16_t*>(w + L.q);
  a.sched_order = reinterpret_cast<int32_t*>(w + L.sched);
  a.sched_cnt = a.sched_order + (size_t)a.n_tg * a.nseg;
  a.sched_n = a.sched_cnt + a.H;
  return a.D == 128 ? launch<128>(a, stream) : launch<64>(a, stream);
}

// ---- the variant that allocates nothing ------------------------------------
// A file-scope device array serves as the workspace of
// cachetune_recompute_attn_noalloc.  Each device the library runs on holds its
// own copy (kNoAllocScratchBytes) until the process ends.  In host code the
// array's name is not a device address: the address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// pointer is handed to the kernels.  Every call on a device shares the array,
// so calls that overlap on one device race.  Nothing in it has to start at
// zero: the set-up launch writes the work list, its counters, the V^T tiles,
// their flags and the rotated queries, and every partial record read by the
// merge is written first by the attention kernel.
namespace {
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ct_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CT_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(CT_E_UNSUPPORTED, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CT_E_HIP, std::string("hipGetSymbolAddress of the attention scratch: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CT_OK;
}
}  // namespace

ct_status attn_run_noalloc(const AttnArgs& a, hipStream_t stream) {
  if (a.n_q == 0) return CT_OK;
  const size_t need = attn_ws_bytes(a);
  if (need > kNoAllocScratchBytes)
    return fail(CT_E_WORKSPACE, "these shapes need " + std::to_string(need) + " bytes of attention workspace, above the " +
                                    std::to_string(kNoAllocScratchBytes) + "-byte scratch of the no-alloc entry point");
  void* ws = nullptr;
  if (need > 0)
    if (ct_status s = scratch_ptr(&ws)) return s;
  return attn_run(a, ws, kNoAllocScratchBytes, stream);
}

}  // namespace ct

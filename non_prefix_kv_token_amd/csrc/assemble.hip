// Per-layer working-buffer assembly with deferred RoPE -- "Adaptive KV Cache
// Reuse for Fast Long-Context LLM Serving" (CacheTune), App. B.2 (fusion:
// reused rows written by position, recomputed rows scattered into the selected
// positions, uncached rows added) and App. B.3 (keys are cached before RoPE and
// rotated at their global position when reused).
//
// One pass over HBM: every output row is read once from its source (cache,
// recomputation buffer or suffix) and written once.  One wave per token row;
// a lane owns 8 RoPE pairs of one head (two 16-byte bf16 vectors, or two
// 32-byte fp32 vectors), so all loads and stores are full vectors and a row's
// H*D elements move in one or two passes of the wave.  The rotation angle and
// its sine and cosine are formed in fp64, the rotated value is rounded once to
// the storage type (for bf16 through fp32 where that is the same rounding).
#include "ct_device.h"
#include "ct_internal.h"

namespace ct {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 8 consecutive stored elements <-> 8 doubles.
template <int DT> struct Vec8;
template <> struct Vec8<CT_BF16> {
  u32x4_t w;
  __device__ void load(const void* p, size_t i) { w = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(p) + i); }
  __device__ void store(void* p, size_t i) const { *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(p) + i) = w; }
  __device__ double get(int t) const {
    const uint32_t x = w[t >> 1];
    return (double)__uint_as_float((t & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  __device__ void set(int t, double v) {
    const uint32_t b = bf16_from_f64(v);
    const int i = t >> 1;
    w[i] = (t & 1) ? ((w[i] & 0xffffu) | (b << 16)) : ((w[i] & 0xffff0000u) | b);
  }
};
template <> struct Vec8<CT_F32> {
  float4 a, b;
  __device__ void load(const void* p, size_t i) {
    const float4* f = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    a = f[0];
    b = f[1];
  }
  __device__ void store(void* p, size_t i) const {
    float4* f = reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i);
    f[0] = a;
    f[1] = b;
  }
  __device__ double get(int t) const {
    const float4& v = t < 4 ? a : b;
    const int k = t & 3;
    return (double)(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
  }
  __device__ void set(int t, double x) {
    float4& v = t < 4 ? a : b;
    const int k = t & 3;
    const float f = (float)x;
    if (k == 0) v.x = f; else if (k == 1) v.y = f; else if (k == 2) v.z = f; else v.w = f;
  }
};

template <int DT, int D>
__global__ __launch_bounds__(256) void k_assemble(AsmLaunch al, void* k_out, void* v_out) {
  constexpr int CPH = D / 16;  // 8-pair chunks per head
  // sine and cosine of the row's D/2 rotation angles, shared by its heads
  __shared__ double s_sc[4][D / 2][2];
  const AsmPlace& pl = al.p[blockIdx.y];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = blockIdx.x * 4 + wv;
  if (r >= pl.n) return;
  const int H = al.H;

  // resolve source row and global position
  const void *ks, *vs;
  int local, srow;
  if (pl.pad_ == 1) {  // plain rows (uncached suffix)
    local = r;
    srow = r;
    ks = pl.k_src;
    vs = pl.v_src;
  } else if (r < pl.n - pl.k) {  // reused row
    if (pl.src_rows) {
      local = pl.src_rows[r];
      srow = r;
    } else {
      local = pl.comp[r];
      srow = local;
    }
    ks = pl.k_src;
    vs = pl.v_src;
  } else {  // recomputed row
    const int t = r - (pl.n - pl.k);
    local = pl.sel[t];
    srow = t;
    ks = pl.k_rec;
    vs = pl.v_rec;
  }
  const long long gpos = (long long)pl.offset + local;
  const size_t src_base = (size_t)srow * H * D;
  const size_t dst_base = (size_t)gpos * H * D;
  const bool half = al.style == CT_ROPE_HALF;
  // one angle per lane (frequency index j), then read back by every head
  // (the wave's own LDS slice: no barrier beyond the wave)
  for (int j = lane; j < D / 2; j += 64) rope_sincos((double)gpos * al.inv_freq[j], &s_sc[wv][j][0], &s_sc[wv][j][1]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  for (int item = lane; item < H * CPH; item += 64) {
    const int h = item / CPH, c = item % CPH;
    // element offsets (within the head) of the two 8-element vectors
    const int ea = half ? 8 * c : 16 * c;
    const int eb = half ? D / 2 + 8 * c : 16 * c + 8;
    const size_t so = src_base + (size_t)h * D, dof = dst_base + (size_t)h * D;
    Vec8<DT> xa, xb, va, vb;
    xa.load(ks, so + ea);
    xb.load(ks, so + eb);
    va.load(vs, so + ea);
    vb.load(vs, so + eb);
    Vec8<DT> ya = xa, yb = xb;
    // pair t of this lane (frequency index 8c + t) rotated in fp64; y0 and y1
    // go to output elements s0(t) and s1(t) of the 16 (0..7 in ya, 8..15 in yb)
    auto rot = [&](const Vec8<DT>& va_, const Vec8<DT>& vb_, int t, double& y0, double& y1) {
      const double sn = s_sc[wv][8 * c + t][0], cs = s_sc[wv][8 * c + t][1];
      double x0, x1;
      if (half) {
        x0 = va_.get(t);
        x1 = vb_.get(t);
      } else {  // interleaved: pairs (2t', 2t'+1) of the 16 elements
        x0 = t < 4 ? va_.get(2 * t) : vb_.get(2 * t - 8);
        x1 = t < 4 ? va_.get(2 * t + 1) : vb_.get(2 * t - 7);
      }
      y0 = x0 * cs - x1 * sn;
      y1 = x0 * sn + x1 * cs;
    };
    auto s0 = [&](int t) { return half ? t : 2 * t; };
    auto s1 = [&](int t) { return half ? 8 + t : 2 * t + 1; };
    if constexpr (DT == CT_BF16) {
      // Round to fp32 (RNE), then to bf16 (RNE).  The two roundings give the
      // one rounding of the fp64 value unless the fp32 result lies exactly on
      // a bf16 midpoint (low 16 bits 0x8000): fp32 holds every bf16 midpoint,
      // so otherwise the fp32 result and the fp64 value are on the same side
      // of every midpoint.  A wave in which some lane meets a midpoint forms
      // its 16 values again and rounds them once, on the fp64 bits.
      uint32_t fb[16];
      bool mid = false;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        double y0, y1;
        rot(xa, xb, t, y0, y1);
        const uint32_t f0 = __float_as_uint((float)y0), f1 = __float_as_uint((float)y1);
        mid |= ((f0 & 0xffffu) == 0x8000u) | ((f1 & 0xffffu) == 0x8000u);
        fb[s0(t)] = f0;
        fb[s1(t)] = f1;
      }
      if (__builtin_expect(__any(mid), 0)) {
        // the inputs pass through an empty asm, so the rotation is formed again
        // here instead of its fp64 results being held from above
        Vec8<DT> xa2 = xa, xb2 = xb;
        asm volatile("" : "+v"(xa2.w), "+v"(xb2.w));
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          double y0, y1;
          rot(xa2, xb2, t, y0, y1);
          fb[s0(t)] = (uint32_t)bf16_from_f64(y0) << 16;  // a bf16 value: the rounding below keeps it
          fb[s1(t)] = (uint32_t)bf16_from_f64(y1) << 16;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ya.w[i] = bf16_bits_rne(__uint_as_float(fb[2 * i])) | (bf16_bits_rne(__uint_as_float(fb[2 * i + 1])) << 16);
        yb.w[i] = bf16_bits_rne(__uint_as_float(fb[8 + 2 * i])) | (bf16_bits_rne(__uint_as_float(fb[9 + 2 * i])) << 16);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        double y0, y1;
        rot(xa, xb, t, y0, y1);
        const int e0 = s0(t), e1 = s1(t);
        if (e0 < 8) ya.set(e0, y0); else yb.set(e0 - 8, y0);
        if (e1 < 8) ya.set(e1, y1); else yb.set(e1 - 8, y1);
      }
    }
    ya.store(k_out, dof + ea);
    yb.store(k_out, dof + eb);
    va.store(v_out, dof + ea);
    vb.store(v_out, dof + eb);
  }
}

template <int DT, int D>
ct_status launch(const AsmLaunch& al, void* k_out, void* v_out, hipStream_t stream) {
  dim3 grid((al.max_rows + 3) / 4, al.n_places);
  {
    TimedLaunch tl_("assemble", stream);
    hipLaunchKernelGGL((k_assemble<DT, D>), grid, dim3(256), 0, stream, al, k_out, v_out);
  }
  return check_launch("assemble");
}

}  // namespace

ct_status assemble_run(const AsmLaunch& al, void* k_out, void* v_out, hipStream_t stream) {
  if (al.max_rows <= 0 || al.n_places <= 0) return CT_OK;
  if (al.dtype == CT_BF16)
    return al.D == 128 ? launch<CT_BF16, 128>(al, k_out, v_out, stream)
                       : launch<CT_BF16, 64>(al, k_out, v_out, stream);
  return al.D == 128 ? launch<CT_F32, 128>(al, k_out, v_out, stream)
                     : launch<CT_F32, 64>(al, k_out, v_out, stream);
}

}  // namespace ct

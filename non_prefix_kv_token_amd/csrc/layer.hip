// The rest of the selective-recompute layer -- "Adaptive KV Cache Reuse for
// Fast Long-Context LLM Serving" (CacheTune), Sec. 4.1 and App. B.2: the
// selected tokens (and the uncached suffix) run through every layer in the new
// context, so besides assembly and attention each layer normalises their
// hidden rows, projects them to q / k / v, projects the attention output back
// with a residual, and applies the gated MLP of the models of Sec. 5.1.
//
// RMSNorm and the gated activation are HBM-bound row kernels; the projections
// are bf16 GEMMs on the matrix cores with the residual added before the single
// rounding of each output.
#include "ct_internal.h"

namespace ct {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline uint32_t pack2(float a, float b) { return bf16_rne(a) | (bf16_rne(b) << 16); }

constexpr int kNormThreads = 256;

// y = x / sqrt(mean(x^2) + eps) * g, one block per row.  The sum of squares
// is accumulated in fp32 per thread over 8-element vectors, then reduced in a
// fixed order (deterministic); the row is read a second time (from cache) to
// scale it, and each output is rounded once to bf16.
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const uint16_t* x, const uint16_t* g,
                                                          int dim, float eps, uint16_t* y) {
  __shared__ float red[kNormThreads];
  const size_t base = (size_t)blockIdx.x * dim;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int c = 8 * tid; c < dim; c += 8 * kNormThreads) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + base + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_lo(v[i]), b = bf16_hi(v[i]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  red[tid] = ss;
  __syncthreads();
  for (int s = kNormThreads / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / (float)dim + eps);
  for (int c = 8 * tid; c < dim; c += 8 * kNormThreads) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + base + c);
    const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(g + c);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack2(bf16_lo(v[i]) * inv * bf16_lo(gv[i]), bf16_hi(v[i]) * inv * bf16_hi(gv[i]));
    *reinterpret_cast<u32x4_t*>(y + base + c) = o;
  }
}

// out[m][j] = silu(gu[m][j]) * gu[m][ff + j], silu(g) = g / (1 + exp(-g)) in
// fp32, rounded once to bf16.  One thread per 8 outputs.
__global__ __launch_bounds__(256) void k_silu_mul(const uint16_t* gu, int rows, int ff, uint16_t* out) {
  const long long per_row = ff / 8;
  const long long item = (long long)blockIdx.x * 256 + threadIdx.x;
  if (item >= (long long)rows * per_row) return;
  const long long m = item / per_row, j = 8 * (item % per_row);
  const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(gu + m * 2 * ff + j);
  const u32x4_t uv = *reinterpret_cast<const u32x4_t*>(gu + m * 2 * ff + ff + j);
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g0 = bf16_lo(gv[i]), g1 = bf16_hi(gv[i]);
    const float s0 = g0 / (1.0f + expf(-g0)), s1 = g1 / (1.0f + expf(-g1));
    o[i] = pack2(s0 * bf16_lo(uv[i]), s1 * bf16_hi(uv[i]));
  }
  *reinterpret_cast<u32x4_t*>(out + m * ff + j) = o;
}

// ---- projections on the matrix cores ---------------------------------------------
// out[m][n] = sum_k x[m][k] w[n][k] (+ res[m][n]), bf16 operands (products exact
// in fp32), fp32 accumulation, one rounding to bf16 at the end (after the
// residual is added).  Block tile 128 (m) x 256 (n), four waves of 64 x 128
// (2 x 4 tiles of v_mfma_f32_32x32x16_bf16), k in stages of 32: each stage's
// x and w slabs are loaded into registers one stage ahead with buffer loads
// (rows past m or n and k past K read as zeros), written to the other of two
// padded LDS buffers after the current stage's products, one barrier per stage.
constexpr int kGBM = 128, kGBN = 256, kGBK = 32;
constexpr int kGLD = kGBK + 8;  // LDS row stride in bf16 (80 bytes: conflict-free 16-byte reads)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                 const uint16_t* res, uint16_t* out, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][kGBM * kGLD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][kGBN * kGLD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const int m0 = blockIdx.y * kGBM, n0 = blockIdx.x * kGBN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;
  const int mrows = min(kGBM, M - m0), nrows = min(kGBN, N - n0);
  // resources start at the block's first row; a load at or past num_records reads 0
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (size_t)m0 * K), 0, mrows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w + (size_t)n0 * K), 0, nrows * K * 2, 0x00020000);
  const int xlim = mrows * K * 2, wlim = nrows * K * 2;
  // staging: the x slab is 128 rows x 4 vectors of 8, the w slab 256 x 4
  int xo[2], wo[4], xl[2], wl[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = tid + 256 * i, r = v >> 2, q = v & 3;
    xo[i] = (r * K + 8 * q) * 2;
    xl[i] = r * kGLD + 8 * q;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = tid + 256 * i, r = v >> 2, q = v & 3;
    wo[i] = (r * K + 8 * q) * 2;
    wl[i] = r * kGLD + 8 * q;
  }
  u32x4_t xs[2], ws[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = (tid + 256 * i) & 3;
      const int off = k0 + 8 * q < K ? xo[i] + k0 * 2 : xlim;  // k past K: zeros
      xs[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = (tid + 256 * i) & 3;
      const int off = k0 + 8 * q < K ? wo[i] + k0 * 2 : wlim;
      ws[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4_t*>(&sa[buf][xl[i]]) = xs[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(&sb[buf][wl[i]]) = ws[i];
  };
  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kGBK / 16; ++ks) {
      bf16x8_t a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(&sa[buf][(wm + 32 * i + col) * kGLD + 16 * ks + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(&sb[buf][(wn + 32 * j + col) * kGLD + 16 * ks + 8 * g]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (K + kGBK - 1) / kGBK;
  load(0);
  store(0);
  if (nk > 1) load(kGBK);
  for (int s = 0; s < nk; ++s) {
    __syncthreads();
    compute(s & 1);
    if (s + 1 < nk) {
      store((s + 1) & 1);
      if (s + 2 < nk) load((s + 2) * kGBK);
    }
  }

  // lane holds n = n0 + wn + 32 j + col and m = m0 + wm + 32 i + 8 (v / 4) + 4 g + v % 4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 32 * j + col;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m >= M) continue;
        float val = acc[i][j][v];
        if (res) val += __uint_as_float(((uint32_t)res[(size_t)m * N + n]) << 16);
        out[(size_t)m * N + n] = (uint16_t)bf16_rne(val);
      }
    }
}

}  // namespace

ct_status rmsnorm_run(const void* x, const void* g, int rows, int dim, float eps, void* y,
                      hipStream_t stream) {
  if (rows == 0) return CT_OK;
  TimedLaunch tl_("rmsnorm", stream);
  hipLaunchKernelGGL(k_rmsnorm, dim3(rows), dim3(kNormThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(g), dim, eps,
                     reinterpret_cast<uint16_t*>(y));
  return check_launch("rmsnorm");
}

ct_status silu_mul_run(const void* gu, int rows, int ff, void* out, hipStream_t stream) {
  const long long items = (long long)rows * (ff / 8);
  if (items == 0) return CT_OK;
  TimedLaunch tl_("silu_mul", stream);
  hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(gu), rows, ff, reinterpret_cast<uint16_t*>(out));
  return check_launch("silu_mul");
}

ct_status linear_run(const void* x, const void* w, const void* residual, int m, int n, int k, void* out,
                     hipStream_t stream) {
  if (m == 0) return CT_OK;
  TimedLaunch tl_("linear", stream);
  dim3 grid((n + kGBN - 1) / kGBN, (m + kGBM - 1) / kGBM);
  hipLaunchKernelGGL(k_gemm_bf16, grid, dim3(256), 0, stream, reinterpret_cast<const uint16_t*>(x),
                     reinterpret_cast<const uint16_t*>(w), reinterpret_cast<const uint16_t*>(residual),
                     reinterpret_cast<uint16_t*>(out), m, n, k);
  return check_launch("linear");
}

}  // namespace ct

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
#include "ct_device.h"
#include "ct_internal.h"

namespace ct {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t pack2(float a, float b) { return bf16_bits_rne(a) | (bf16_bits_rne(b) << 16); }

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
// residual is added).  A block computes a BM x BN tile with WGM x WGN waves,
// each a (BM / WGM) x (BN / WGN) tile of v_mfma_f32_32x32x16_bf16 tiles; k
// advances in stages of BK (32 or 64).  Each stage's x and w slabs are loaded into
// registers two stages ahead (two register sets, alternating) with buffer
// loads (rows past m or n and k past K read as zeros) and written to the other
// of two LDS buffers after the current stage's products: one barrier per
// stage, and two stages of products to cover each load's latency.  An LDS row is BK k (BK / 8
// 16-byte chunks); chunk c of row r sits at chunk c ^ ((r / R) % (BK / 8)),
// R = 128 / BK rows per pass over the 64 banks, so that both the row-major
// slab writes and the operand reads (one row per lane) hit 16 distinct 4-bank
// groups per 16 lanes.  The output columns may be split over
// three destinations (q | k | v of the fused projection): columns [0, n1) go
// to out0 (row length n1), [n1, n2) to out1, [n2, N) to out2.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int BM, int BN, int WGM, int WGN, int BK>
__global__ __launch_bounds__(64 * WGM * WGN)
__attribute__((amdgpu_waves_per_eu((BM / WGM) * (BN / WGN) > 64 * 128 ? 1 : 2,
                                   (BM / WGM) * (BN / WGN) > 64 * 128 ? 1 : 2)))
void k_gemm_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                 const uint16_t* res, uint16_t* out0, uint16_t* out1, uint16_t* out2, int n1, int n2,
                 int M, int N, int K) {
  constexpr int NT = 64 * WGM * WGN;                        // threads
  constexpr int TI = BM / WGM / 32, TJ = BN / WGN / 32;     // MFMA tiles per wave
  constexpr int CPR = BK / 8;                               // 16-byte chunks per LDS row
  constexpr int RPC = 128 / BK;                             // LDS rows per 64-bank cycle
  constexpr int NX = BM * CPR / NT, NW = BN * CPR / NT;     // 16-byte vectors per thread and stage
  static_assert(NX * NT == BM * CPR && NW * NT == BN * CPR && NT % CPR == 0, "slab split");
  static_assert(BK == 32 || BK == 64, "stage depth");
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN * BK];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int wm = (wave / WGN) * (BM / WGM), wn = (wave % WGN) * (BN / WGN);
  const int mrows = min(BM, M - m0), nrows = min(BN, N - n0);
  // resources start at the block's first row; a load at or past num_records reads 0
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (size_t)m0 * K), 0, mrows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w + (size_t)n0 * K), 0, nrows * K * 2, 0x00020000);
  const int xlim = mrows * K * 2, wlim = nrows * K * 2;
  int xo[NX], wo[NW], xl[NX], wl[NW];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int v = tid + NT * i, r = v / CPR, q = v % CPR;
    xo[i] = (r * K + 8 * q) * 2;
    xl[i] = r * BK + 8 * (q ^ ((r / RPC) % CPR));
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = tid + NT * i, r = v / CPR, q = v % CPR;
    wo[i] = (r * K + 8 * q) * 2;
    wl[i] = r * BK + 8 * (q ^ ((r / RPC) % CPR));
  }
  const int q8 = 8 * (tid % CPR);  // k offset of this thread's vectors within a stage
  u32x4_t xa[NX], wa[NW], xb[NX], wb[NW];
  auto load = [&](int k0, u32x4_t* xs, u32x4_t* ws) {
    const bool in = k0 + q8 < K;  // k past K: zeros
#pragma unroll
    for (int i = 0; i < NX; ++i)
      xs[i] = __builtin_bit_cast(u32x4_t,
                                 __builtin_amdgcn_raw_buffer_load_b128(xr, in ? xo[i] + k0 * 2 : xlim, 0, 0));
#pragma unroll
    for (int i = 0; i < NW; ++i)
      ws[i] = __builtin_bit_cast(u32x4_t,
                                 __builtin_amdgcn_raw_buffer_load_b128(wr, in ? wo[i] + k0 * 2 : wlim, 0, 0));
  };
  auto store = [&](int buf, const u32x4_t* xs, const u32x4_t* ws) {
#pragma unroll
    for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4_t*>(&sa[buf][xl[i]]) = xs[i];
#pragma unroll
    for (int i = 0; i < NW; ++i) *reinterpret_cast<u32x4_t*>(&sb[buf][wl[i]]) = ws[i];
  };
  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int sw = (col / RPC) % CPR;  // rows read by this lane are col mod 32
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[TI], b[TJ];
      const int ch = 8 * ((2 * ks + g) ^ sw);
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(&sa[buf][(wm + 32 * i + col) * BK + ch]);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(&sb[buf][(wn + 32 * j + col) * BK + ch]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (K + BK - 1) / BK;
  // stages two ahead in registers (sets a and b alternate), two LDS buffers
  load(0, xa, wa);
  store(0, xa, wa);
  if (nk > 1) load(BK, xa, wa);
  if (nk > 2) load(2 * BK, xb, wb);
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    __syncthreads();
    compute(0);
    store(1, xa, wa);
    if (s + 3 < nk) load((s + 3) * BK, xa, wa);
    __syncthreads();
    compute(1);
    if (s + 2 < nk) {
      store(0, xb, wb);
      if (s + 4 < nk) load((s + 4) * BK, xb, wb);
    }
  }
  if (s < nk) {
    __syncthreads();
    compute(0);
  }

  // lane holds n = n0 + wn + 32 j + col and m = m0 + wm + 32 i + 8 (v / 4) + 4 g + v % 4
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int n = n0 + wn + 32 * j + col;
    if (n >= N) continue;
    uint16_t* dst = out0;
    int ld = n1, c = n;
    if (n >= n2) {
      dst = out2; ld = N - n2; c = n - n2;
    } else if (n >= n1) {
      dst = out1; ld = n2 - n1; c = n - n1;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m >= M) continue;
        float val = acc[i][j][v];
        if (res) val += __uint_as_float(((uint32_t)res[(size_t)m * N + n]) << 16);
        dst[(size_t)m * ld + c] = (uint16_t)bf16_bits_rne(val);
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

template <int BM, int BN, int WGM, int WGN, int BK>
static void gemm_go(const void* x, const void* w, const void* residual, void* out0, void* out1, void* out2,
                    int n1, int n2, int m, int n, int k, hipStream_t stream) {
  dim3 grid((n + BN - 1) / BN, (m + BM - 1) / BM);
  hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WGM, WGN, BK>), grid, dim3(64 * WGM * WGN), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                     reinterpret_cast<const uint16_t*>(residual), reinterpret_cast<uint16_t*>(out0),
                     reinterpret_cast<uint16_t*>(out1), reinterpret_cast<uint16_t*>(out2), n1, n2, m, n, k);
}

// Tile choice by waves of blocks: a 256 x 256 block (8 waves, one per CU)
// moves half the LDS bytes per product of a 128 x 256 block (4 waves, two per
// CU), and one round of small blocks was measured at about 1.15 rounds of big
// ones; the configuration with the fewer (weighted) rounds is taken, so a
// product whose big-block count just passes a multiple of the CU count (the
// fused q/k/v projection of 2584 rows: 264 blocks) uses small blocks.
static ct_status gemm_launch(const void* x, const void* w, const void* residual, void* out0, void* out1,
                             void* out2, int n1, int n2, int m, int n, int k, hipStream_t stream) {
  if (m == 0) return CT_OK;
  TimedLaunch tl_("linear", stream);
  const long long ncu = device_cu_count();
  const long long big = (long long)((m + 255) / 256) * ((n + 255) / 256);
  const long long small = (long long)((m + 127) / 128) * ((n + 255) / 256);
  const double r_big = (double)((big + ncu - 1) / ncu), r_small = 1.15 * (double)((small + 2 * ncu - 1) / (2 * ncu));
  if (r_big <= r_small)
    gemm_go<256, 256, 4, 2, 32>(x, w, residual, out0, out1, out2, n1, n2, m, n, k, stream);
  else
    gemm_go<128, 256, 2, 2, 32>(x, w, residual, out0, out1, out2, n1, n2, m, n, k, stream);
  return check_launch("linear");
}

ct_status linear_run(const void* x, const void* w, const void* residual, int m, int n, int k, void* out,
                     hipStream_t stream) {
  return gemm_launch(x, w, residual, out, out, out, n, n, m, n, k, stream);
}

ct_status qkv_run(const void* x, const void* w_qkv, int m, int d, int nq, int nkv, void* q, void* k, void* v,
                  hipStream_t stream) {
  return gemm_launch(x, w_qkv, nullptr, q, k, v, nq, nq + nkv, m, nq + 2 * nkv, d, stream);
}

}  // namespace ct

// The rest of the selective-recompute layer -- "Adaptive KV Cache Reuse for
// Fast Long-Context LLM Serving" (CacheTune), Sec. 4.1 and App. B.2: the
// selected tokens (and the uncached suffix) run through every layer in the new
// context, so besides assembly and attention each layer normalises their
// hidden rows, projects them to q / k / v, projects the attention output back
// with a residual, and applies the gated MLP of the models of Sec. 5.1.
//
// RMSNorm and the gated activation are HBM-bound row kernels written here.
// The projections are plain bf16 GEMMs with fp32 accumulation; they go to
// hipBLASLt (one handle per device, created on first use and kept until the
// process ends), with the residual folded in as D = X W^T + R (beta = 1).
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

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

// ---- projections on hipBLASLt ---------------------------------------------------
// Row-major Y[m][n] = X[m][k] W[n][k]^T (+ R[m][n]) is, in hipBLASLt's
// column-major terms, Y^T (n x m) = op_T(W as k x n) * (X as k x m): a "TN"
// product with leading dimensions k, k and n.
struct Plan {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws_need = 0;
};

std::mutex g_blas_mu;
hipblasLtHandle_t g_handle[64] = {};
std::map<std::tuple<int, int, int, int, size_t>, Plan> g_plans[64];

ct_status blas_fail(hipblasStatus_t st, const char* what) {
  return fail(CT_E_HIP, std::string("hipBLASLt ") + what + " failed (status " + std::to_string((int)st) + ")");
}

ct_status get_plan(int dev, int m, int n, int k, size_t ws_bytes, const Plan** out) {
  std::lock_guard<std::mutex> lock(g_blas_mu);
  if (!g_handle[dev]) {
    hipblasStatus_t st = hipblasLtCreate(&g_handle[dev]);
    if (st != HIPBLAS_STATUS_SUCCESS) {
      g_handle[dev] = nullptr;
      return blas_fail(st, "handle creation");
    }
  }
  auto key = std::make_tuple(m, n, k, 0, ws_bytes);
  auto it = g_plans[dev].find(key);
  if (it != g_plans[dev].end()) {
    *out = &it->second;
    return CT_OK;
  }
  Plan p;
  hipblasStatus_t st = hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F);
  if (st != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "descriptor");
  const hipblasOperation_t tA = HIPBLAS_OP_T, tB = HIPBLAS_OP_N;
  hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &tA, sizeof(tA));
  hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tB, sizeof(tB));
  if ((st = hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, k, n, k)) != HIPBLAS_STATUS_SUCCESS ||
      (st = hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, k, m, k)) != HIPBLAS_STATUS_SUCCESS ||
      (st = hipblasLtMatrixLayoutCreate(&p.c, HIP_R_16BF, n, m, n)) != HIPBLAS_STATUS_SUCCESS)
    return blas_fail(st, "layout");
  hipblasLtMatmulPreference_t pref = nullptr;
  if ((st = hipblasLtMatmulPreferenceCreate(&pref)) != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "preference");
  const uint64_t cap = ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
  hipblasLtMatmulHeuristicResult_t res[1];
  int got = 0;
  st = hipblasLtMatmulAlgoGetHeuristic(g_handle[dev], p.op, p.a, p.b, p.c, p.c, pref, 1, res, &got);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS || got < 1) return blas_fail(st, "algorithm selection");
  p.algo = res[0].algo;
  p.ws_need = res[0].workspaceSize;
  auto ins = g_plans[dev].emplace(key, p);
  *out = &ins.first->second;
  return CT_OK;
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
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (m == 0) return CT_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(CT_E_HIP, "no current device");
  const Plan* p = nullptr;
  if (ct_status s = get_plan(dev, m, n, k, ws_bytes, &p)) return s;
  const float alpha = 1.0f, beta = residual ? 1.0f : 0.0f;
  TimedLaunch tl_("linear", stream);
  hipblasStatus_t st = hipblasLtMatmul(g_handle[dev], p->op, &alpha, w, p->a, x, p->b, &beta,
                                       residual ? residual : out, p->c, out, p->c, &p->algo, ws,
                                       ws_bytes, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "matmul");
  return check_launch("linear");
}

}  // namespace ct

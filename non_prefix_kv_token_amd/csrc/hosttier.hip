// Host-tier sparse loading -- "Adaptive KV Cache Reuse for Fast Long-Context
// LLM Serving" (CacheTune), App. B.1 (the ranking is stored with the chunk when
// the cache is generated; another r only moves the cut) and App. B.2 (only the
// reuse complement is loaded from the external pool, layer by layer).
//
// Offline, the rows of every chunk layer are stored in rank order, so that for
// any r the reuse complement of a (chunk, layer) is the contiguous tail of
// that layer: one DMA copy per (chunk, layer, K|V) instead of one per run of
// rows.  k_rank_order is that gather on the device; the copies themselves are
// hipMemcpyAsync calls issued by cachetune_stage_complement.
#include "ct_internal.h"

namespace ct {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// dst[l][j] = src[l][ranking[j]]: one wave per destination row, 16-byte vectors.
__global__ __launch_bounds__(256) void k_rank_order(const char* ksrc, const char* vsrc,
                                                    const int32_t* ranking, int32_t n,
                                                    int32_t row_bytes, char* kdst, char* vdst) {
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (j >= n) return;
  const size_t l = blockIdx.y;
  const int i = ranking[j];
  const size_t so = (l * n + i) * (size_t)row_bytes, dof = (l * n + j) * (size_t)row_bytes;
  for (int c = lane; c < row_bytes / 16; c += 64) {
    *reinterpret_cast<u32x4_t*>(kdst + dof + 16 * c) = *reinterpret_cast<const u32x4_t*>(ksrc + so + 16 * c);
    *reinterpret_cast<u32x4_t*>(vdst + dof + 16 * c) = *reinterpret_cast<const u32x4_t*>(vsrc + so + 16 * c);
  }
}

}  // namespace

ct_status rank_order_run(const void* k_src, const void* v_src, const int32_t* ranking, int32_t n,
                         int32_t L, int32_t row_bytes, void* k_dst, void* v_dst, hipStream_t stream) {
  dim3 grid((n + 3) / 4, L);
  {
    TimedLaunch tl_("rank_order", stream);
    hipLaunchKernelGGL(k_rank_order, grid, dim3(256), 0, stream, reinterpret_cast<const char*>(k_src),
                       reinterpret_cast<const char*>(v_src), ranking, n, row_bytes,
                       reinterpret_cast<char*>(k_dst), reinterpret_cast<char*>(v_dst));
  }
  return check_launch("rank order");
}

}  // namespace ct

// Top-r selection -- "Adaptive KV Cache Reuse for Fast Long-Context LLM
// Serving" (CacheTune), App. B.1: the top-ranked rN positions of a chunk form
// the recomputation set, the rest its reuse complement; the full ranking is
// stored so that another r only moves the cut.
//
// One block (1024 threads) per chunk.  Each score becomes a 64-bit key
//   high word: bitwise complement of an order-preserving image of the fp32
//              score (so ascending key = descending score; -0 == +0; NaN last)
//   low word:  local index (so equal scores rank by lower index)
// sorted ascending by a bitonic network in LDS (n <= 8192).  The ascending
// recomputation set and complement come from a block-wide prefix count over
// the membership flags in index order.
#include "ct_internal.h"

namespace ct {
namespace {

constexpr int kThreads = 1024;

__device__ inline uint32_t score_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;               // -0 -> +0
  uint32_t ord;
  if ((u & 0x7fffffffu) > 0x7f800000u) ord = 0u;     // NaN: lowest score
  else ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ord;
}

__global__ __launch_bounds__(kThreads) void k_topr(TopRLaunch tl, const float* score,
                                                   int32_t* ranking, int32_t* sel,
                                                   int32_t* comp) {
  __shared__ unsigned long long key[kMaxN];
  __shared__ unsigned char flag[kMaxN];
  __shared__ int cnt[kThreads];
  const TopRChunk& c = tl.c[blockIdx.x];
  const int n = c.n, k = c.k, tid = threadIdx.x;
  int p2 = 1;
  while (p2 < n) p2 <<= 1;

  for (int i = tid; i < p2; i += kThreads) {
    key[i] = i < n ? ((unsigned long long)score_order_key(score[c.tok_off + i]) << 32) | (uint32_t)i
                   : ~0ull;
  }
  __syncthreads();
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < p2 / 2; i += kThreads) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool up = (lo & size) == 0;
        unsigned long long a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < n; r += kThreads) {
    int idx = (int)(key[r] & 0xffffffffull);
    if (ranking) ranking[c.tok_off + r] = idx;
    flag[idx] = r < k ? 1 : 0;
  }
  __syncthreads();

  // ascending membership lists: each thread owns a contiguous index range
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += flag[i];
  cnt[tid] = mine;
  __syncthreads();
  for (int s = 1; s < kThreads; s <<= 1) {  // inclusive Hillis-Steele scan
    int v = tid >= s ? cnt[tid - s] : 0;
    __syncthreads();
    cnt[tid] += v;
    __syncthreads();
  }
  int before = cnt[tid] - mine;  // selected indices below i0
  for (int i = i0; i < i1; ++i) {
    if (flag[i]) {
      sel[c.sel_off + before] = i;
      ++before;
    } else if (comp) {
      comp[c.comp_off + (i - before)] = i;
    }
  }
}

}  // namespace

ct_status topr_run(const TopRLaunch& tl, const float* score, int32_t* ranking, int32_t* sel,
                   int32_t* comp, hipStream_t stream) {
  {
    TimedLaunch tl_("topr", stream);
    hipLaunchKernelGGL(k_topr, dim3(tl.n_chunks), dim3(kThreads), 0, stream, tl, score, ranking,
                     sel, comp);
  }
  return check_launch("top-r");
}

}  // namespace ct

// Top-r selection -- "Adaptive KV Cache Reuse for Fast Long-Context LLM
// Serving" (CacheTune), App. B.1.  Per chunk: sort the positions by score,
// take the first floor(r * n) as the positions to recompute and keep the
// others for reuse; the whole order is written out once, so a different r
// later only changes where it is cut.
//
// Each score becomes a 64-bit key
//   high word: bitwise complement of an order-preserving image of the fp32
//              score (so ascending key = descending score; -0 == +0; NaN last)
//   low word:  local index (so equal scores rank by lower index)
// and the ranking is the ascending order of the keys.  When the caller stores
// the ranking, every element's rank is counted in parallel (below), then one
// block per chunk forms the lists.  Otherwise one block (1024 threads) per
// chunk sorts the keys ascending by a bitonic network (n <= 8192).  Stages whose stride is
// at least 128 pair elements across waves and run in LDS with a block barrier;
// the others stay inside one wave's 128-element segments and run in registers
// (lane-pair exchanges), two elements per lane.  The ascending recomputation
// set and complement come from a block-wide prefix count over the membership
// flags in index order (wave scans, then the wave totals).
#include <algorithm>

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

// Ascending membership lists from the per-index flags (in LDS): each thread
// owns a contiguous index range; a block prefix count places its entries.
__device__ void compact(const TopRChunk& c, const unsigned char* flag, int* cnt, int32_t* sel,
                        int32_t* comp) {
  const int n = c.n, tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += flag[i];
  int incl = mine;  // inclusive scan over the wave's lanes
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += t;
  }
  if ((tid & 63) == 63) cnt[tid >> 6] = incl;  // wave totals
  __syncthreads();
  int before = incl - mine;  // selected indices below i0
  for (int w = 0; w < (tid >> 6); ++w) before += cnt[w];
  for (int i = i0; i < i1; ++i) {
    if (flag[i]) {
      sel[c.sel_off + before] = i;
      ++before;
    } else if (comp) {
      comp[c.comp_off + (i - before)] = i;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_topr(TopRLaunch tl, const float* score,
                                                   int32_t* ranking, int32_t* sel,
                                                   int32_t* comp) {
  __shared__ unsigned long long key[kMaxN];
  __shared__ unsigned char flag[kMaxN];
  __shared__ int cnt[kThreads / 64];
  const TopRChunk& c = tl.c[blockIdx.x];
  const int n = c.n, k = c.k, tid = threadIdx.x;
  int p2 = 1;
  while (p2 < n) p2 <<= 1;

  for (int i = tid; i < p2; i += kThreads) {
    key[i] = i < n ? ((unsigned long long)score_order_key(score[c.tok_off + i]) << 32) | (uint32_t)i
                   : ~0ull;
  }
  __syncthreads();
  // one compare-exchange stage in LDS: pairs (lo, lo + stride), ascending
  // where bit `size` of lo is clear
  auto lds_stage = [&](int size, int stride) {
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
  };
  if (p2 < 128) {
    for (int size = 2; size <= p2; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) lds_stage(size, stride);
  } else {
    // Stages of stride <= 64 pair positions inside one 128-element segment:
    // lane l holds positions x = base + l (a) and x + 64 (b).  At stride 64
    // the pair is (a, b); below it, the partner of position x is x ^ s, in
    // lane l ^ s.  The lower position of a pair keeps the smaller key where
    // bit `size` of the position is clear, the larger one elsewhere.
    const int wave = tid >> 6, lane = tid & 63, nseg = p2 >> 7;
    auto wave_stages = [&](int size_lo, int size_hi, int s_first) {
      for (int seg = wave; seg < nseg; seg += kThreads / 64) {
        const int x = seg * 128 + lane;
        unsigned long long a = key[x], b = key[x + 64];
        for (int size = size_lo; size <= size_hi; size <<= 1)
          for (int st = min(s_first, size >> 1); st > 0; st >>= 1) {
            if (st == 64) {
              if ((a > b) == ((x & size) == 0)) {
                const unsigned long long t = a;
                a = b;
                b = t;
              }
            } else {
              const unsigned long long pa = __shfl_xor(a, st), pb = __shfl_xor(b, st);
              const bool lower = (x & st) == 0;
              const bool min_a = lower == ((x & size) == 0), min_b = lower == (((x + 64) & size) == 0);
              a = (min_a == (pa < a)) ? pa : a;
              b = (min_b == (pb < b)) ? pb : b;
            }
          }
        key[x] = a;
        key[x + 64] = b;
      }
      __syncthreads();
    };
    wave_stages(2, 128, 64);  // every stage of the sizes up to 128
    for (int size = 256; size <= p2; size <<= 1) {
      for (int stride = size >> 1; stride >= 128; stride >>= 1) lds_stage(size, stride);
      wave_stages(size, size, 64);
    }
  }
  for (int r = tid; r < n; r += kThreads) {
    int idx = (int)(key[r] & 0xffffffffull);
    if (ranking) ranking[c.tok_off + r] = idx;
    flag[idx] = r < k ? 1 : 0;
  }
  __syncthreads();
  compact(c, flag, cnt, sel, comp);
}

// ---- when the ranking is stored: ranks by counting ----------------------------
// The keys are distinct (the index is part of them), so an element's rank is
// the number of keys of its chunk below its own.  kRankSlices threads share an
// element, each counting over every kRankSlices-th key (consecutive lanes read
// consecutive keys: no bank conflicts), and the chunk's keys sit in LDS once
// per block.  Every chunk is spread over n / kRankElems blocks, so the whole
// GPU takes part instead of one block per chunk.
constexpr int kRankThreads = 256;
constexpr int kRankSlices = 8;
constexpr int kRankElems = kRankThreads / kRankSlices;

__global__ __launch_bounds__(kRankThreads) void k_topr_rank(TopRLaunch tl, const float* score,
                                                            int32_t* ranking) {
  extern __shared__ unsigned long long skey[];  // [n]
  const TopRChunk& c = tl.c[blockIdx.y];
  const int n = c.n, tid = threadIdx.x;
  const int e = blockIdx.x * kRankElems + tid / kRankSlices, sl = tid % kRankSlices;
  if (blockIdx.x * kRankElems >= n) return;  // uniform over the block
  for (int i = tid; i < n; i += kRankThreads)
    skey[i] = ((unsigned long long)score_order_key(score[c.tok_off + i]) << 32) | (uint32_t)i;
  __syncthreads();
  const unsigned long long mine = e < n ? skey[e] : 0ull;
  int below = 0;
#pragma unroll 8
  for (int j = sl; j < n; j += kRankSlices) below += skey[j] < mine ? 1 : 0;
#pragma unroll
  for (int o = 1; o < kRankSlices; o <<= 1) below += __shfl_xor(below, o);
  if (sl == 0 && e < n) ranking[c.tok_off + below] = e;
}

// The ascending set and complement from the stored ranking: its first k
// entries are the selected indices.
__global__ __launch_bounds__(kThreads) void k_topr_compact(TopRLaunch tl, const int32_t* ranking,
                                                           int32_t* sel, int32_t* comp) {
  __shared__ unsigned char flag[kMaxN];
  __shared__ int cnt[kThreads / 64];
  const TopRChunk& c = tl.c[blockIdx.x];
  const int n = c.n, k = c.k, tid = threadIdx.x;
  for (int i = tid; i < n; i += kThreads) flag[i] = 0;
  __syncthreads();
  for (int r = tid; r < k; r += kThreads) flag[ranking[c.tok_off + r]] = 1;
  __syncthreads();
  compact(c, flag, cnt, sel, comp);
}

}  // namespace

// ---- checking a device index array ------------------------------------------
// The array is only read; a value out of range is counted, never followed.
namespace {
__global__ __launch_bounds__(64) void k_check_clear(int32_t* bad) {
  if (threadIdx.x == 0) bad[0] = 0;
}
__global__ __launch_bounds__(256) void k_check_indices(const int32_t* idx, int32_t count, int32_t bound,
                                                       int32_t ascending, int32_t* bad) {
  int n_bad = 0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count; i += (long long)gridDim.x * 256) {
    const int32_t v = idx[i];
    bool b = v < 0 || v >= bound;
    if (ascending && i > 0) b = b || v <= idx[i - 1];
    n_bad += b;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n_bad += __shfl_xor(n_bad, o);
  if ((threadIdx.x & 63) == 0 && n_bad) atomicAdd(bad, n_bad);
}
}  // namespace

ct_status check_indices_run(const int32_t* idx, int32_t count, int32_t bound, bool ascending, int32_t* bad,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_check_clear, dim3(1), dim3(64), 0, stream, bad);
  if (ct_status s = check_launch("index check")) return s;
  if (count == 0) return CT_OK;
  const int blocks = (int)std::min<long long>(((long long)count + 255) / 256, 1024);
  hipLaunchKernelGGL(k_check_indices, dim3(blocks), dim3(256), 0, stream, idx, count, bound, (int32_t)ascending, bad);
  return check_launch("index check");
}

ct_status topr_run(const TopRLaunch& tl, const float* score, int32_t* ranking, int32_t* sel,
                   int32_t* comp, hipStream_t stream) {
  if (!ranking) {  // one sort per chunk, the ranking kept in LDS only
    TimedLaunch tl_("topr", stream);
    hipLaunchKernelGGL(k_topr, dim3(tl.n_chunks), dim3(kThreads), 0, stream, tl, score, ranking,
                       sel, comp);
    return check_launch("top-r");
  }
  int max_n = 0;
  for (int i = 0; i < tl.n_chunks; ++i) max_n = std::max(max_n, (int)tl.c[i].n);
  if (max_n <= 0) return CT_OK;
  {
    TimedLaunch tl_("topr", stream);
    hipLaunchKernelGGL(k_topr_rank, dim3((max_n + kRankElems - 1) / kRankElems, tl.n_chunks),
                       dim3(kRankThreads), (size_t)max_n * sizeof(unsigned long long), stream, tl, score,
                       ranking);
  }
  if (ct_status s = check_launch("top-r ranks")) return s;
  {
    TimedLaunch tl_("topr", stream);
    hipLaunchKernelGGL(k_topr_compact, dim3(tl.n_chunks), dim3(kThreads), 0, stream, tl, ranking, sel,
                       comp);
  }
  return check_launch("top-r lists");
}

}  // namespace ct

// Per-layer working-buffer assembly with deferred RoPE -- "Adaptive KV Cache
// Reuse for Fast Long-Context LLM Serving" (CacheTune), App. B.2 (fusion:
// reused rows written by position, recomputed rows scattered into the selected
// positions, uncached rows added) and App. B.3 (keys are cached before RoPE and
// rotated at their global position when reused).
//
// One pass over HBM: every output row is read once from its source (cache,
// recomputation buffer or suffix) and written once.  A group of D/8 threads
// handles one row: thread q owns RoPE pairs 4q..4q+3 of every head, so the
// four angles (fp64 sincos) are formed once per row and reused for all H heads.
// The rotation is done in fp64 and rounded once to the storage type.
#include "ct_internal.h"

namespace ct {
namespace {

__device__ inline double ld_elem(const void* p, size_t i, int dt) {
  if (dt == CT_F32) return (double)reinterpret_cast<const float*>(p)[i];
  return (double)__uint_as_float(((uint32_t)reinterpret_cast<const uint16_t*>(p)[i]) << 16);
}

__device__ inline uint16_t bf16_from_f64(double d) {
  float f = __double2float_rz(d);
  uint32_t u = __float_as_uint(f);
  if ((double)f != d) u |= 1u;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <int DT>
__device__ inline void st_elem(void* p, size_t i, double v) {
  if constexpr (DT == CT_F32) reinterpret_cast<float*>(p)[i] = (float)v;
  else reinterpret_cast<uint16_t*>(p)[i] = bf16_from_f64(v);
}

template <int DT, int D>
__global__ __launch_bounds__(256) void k_assemble(AsmLaunch al, void* k_out, void* v_out) {
  constexpr int TPR = D / 8;            // threads per row
  constexpr int RPB = 256 / TPR;        // rows per block
  const AsmPlace& pl = al.p[blockIdx.y];
  const int q = threadIdx.x % TPR;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
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
    int t = r - (pl.n - pl.k);
    local = pl.sel[t];
    srow = t;
    ks = pl.k_rec;
    vs = pl.v_rec;
  }
  const long long gpos = (long long)pl.offset + local;

  double cs[4], sn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double ang = (double)gpos * al.inv_freq[4 * q + i];
    sincos(ang, &sn[i], &cs[i]);
  }

  const size_t src_base = (size_t)srow * H * D;
  const size_t dst_base = (size_t)gpos * H * D;
  for (int h = 0; h < H; ++h) {
    const size_t so = src_base + (size_t)h * D, dof = dst_base + (size_t)h * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = 4 * q + i;
      int e0 = al.style == CT_ROPE_HALF ? j : 2 * j;
      int e1 = al.style == CT_ROPE_HALF ? j + D / 2 : 2 * j + 1;
      double a = ld_elem(ks, so + e0, DT), b = ld_elem(ks, so + e1, DT);
      st_elem<DT>(k_out, dof + e0, a * cs[i] - b * sn[i]);
      st_elem<DT>(k_out, dof + e1, a * sn[i] + b * cs[i]);
      if constexpr (DT == CT_F32) {
        reinterpret_cast<float*>(v_out)[dof + e0] = reinterpret_cast<const float*>(vs)[so + e0];
        reinterpret_cast<float*>(v_out)[dof + e1] = reinterpret_cast<const float*>(vs)[so + e1];
      } else {
        reinterpret_cast<uint16_t*>(v_out)[dof + e0] = reinterpret_cast<const uint16_t*>(vs)[so + e0];
        reinterpret_cast<uint16_t*>(v_out)[dof + e1] = reinterpret_cast<const uint16_t*>(vs)[so + e1];
      }
    }
  }
}

template <int DT, int D>
ct_status launch(const AsmLaunch& al, void* k_out, void* v_out, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  dim3 grid((al.max_rows + RPB - 1) / RPB, al.n_places);
  hipLaunchKernelGGL((k_assemble<DT, D>), grid, dim3(256), 0, stream, al, k_out, v_out);
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

// Internal declarations of the gfx950 CacheTune library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "cachetune.h"

namespace ct {

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
ct_status fail(ct_status s, const std::string& msg);
ct_status check_launch(const char* what);

// ------------------------------------------------------------ timing
// Brackets one kernel launch with HIP events when timing is enabled
// (cachetune_timing_enable); a no-op otherwise.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t stream);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  hipStream_t stream_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  std::string name_;
};

// ------------------------------------------------------- shared constants
constexpr int kMaxChunksPerLaunch = 32;  // descriptors passed by value in kernel arguments
constexpr int kMaxN = 8192;              // tokens per chunk
constexpr int kPTile = 128;              // band rows per projection block

// Retained bins and transform length (App. B.1).
int fft_len(int n, ct_fftlen mode);
int kkeep(int nf, int a_num, int a_den);
inline int band_rows_padded(int kk) { return ((2 * kk + 31) / 32) * 32; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// -------------------------------------------------------------- score path
// Descriptor of one chunk in a score launch.  Byte offsets are into the
// caller's workspace.
struct ScoreChunkDesc {
  const void* k;
  const void* v;
  int32_t n;         // tokens
  int32_t nf;        // transform length
  int32_t kk;        // retained bins
  int32_t ppad;      // padded band rows (multiple of 32, >= 2*kk)
  int32_t ntok_pad;  // twiddle table row length (multiple of 32, >= n)
  int32_t tw_owner;  // 1: this launch writes the chunk's tables (not held by a context)
  int64_t tw_off;    // workspace offsets of the tables when they live there
  int64_t tw16_off;
  int64_t trig_off;
  uint16_t* tw;      // bf16 twiddle planes [3][ppad][ntok_pad] (device; set by score_bind)
  uint16_t* tw16;    // fp16 twiddle planes [2][ppad][ntok_pad]
  double2* trig;     // fp64 (cos, sin) of 2*pi*m/nf, m < nf
  int64_t y_off;     // fp32 band coefficients [L][2][ppad][C]
  int64_t e_off;     // fp64 low-pass energies [L][2][n]
  int64_t tok_off;   // first token of this chunk in the concatenated score vector
};

struct ScoreLaunch {
  ScoreChunkDesc c[kMaxChunksPerLaunch];
  int32_t n_chunks;
  int32_t L, H, D, C;  // C = H * D
  int32_t dtype;
  int32_t norm;
  int32_t max_ppad;
  int32_t n_slots;     // Gram scratch slots
  int32_t slot_p2;     // rows of the largest Gram handled (2 * max kk)
  int64_t slot_off;    // byte offset of the Gram slots
  int64_t slot_bytes;  // bytes per slot
  int64_t total_tokens;
  int32_t variant;     // ct_score_variant
};


// Twiddle and trigonometric tables of one (transform length, retained bins,
// padded token count), device memory.
struct ScoreTables {
  uint16_t* tw;
  uint16_t* tw16;
  double2* trig;
};
// Per-device context (cachetune_create): device ordinal, compute units and the
// scoring tables built by cachetune_prepare_scoring.
struct Context;
bool context_find_tables(const Context* ctx, int nf, int kk, int ntp, ScoreTables* out);
int context_cu_count(const Context* ctx);  // the current device's when ctx is NULL

// The plan of a score call.  Tables found in `ctx` are taken from there; the
// others get a region of the workspace and are written by the call.
ct_status score_plan(const int32_t* n_per_chunk, int32_t n_chunks, int32_t L, int32_t H,
                     int32_t D, int32_t a_num, int32_t a_den, ct_fftlen fftlen, size_t* bytes,
                     std::vector<ScoreLaunch>* launches, int32_t variant = CT_SCORE_LOWPASS,
                     const Context* ctx = nullptr);
// Points the descriptors' workspace tables at `ws` (context tables are set by
// score_plan already).
void score_bind(std::vector<ScoreLaunch>* launches, char* ws);
// Writes one table set (k_twiddle) on `stream`.
ct_status score_tables_build(int nf, int kk, int ntp, int dtype, const ScoreTables& t, hipStream_t stream);
size_t score_tables_bytes(int nf, int kk, int ntp, size_t* tw16_off, size_t* trig_off);
ct_status score_run(const std::vector<ScoreLaunch>& launches, char* ws, float* score,
                    float* layer_score, hipStream_t stream);
// Band projection of every bin (plan with alpha = 1 and this variant: no Gram
// slots), then the energy fractions of n_bands equal bands of the bins.
constexpr int32_t kVariantBandEnergy = 100;
ct_status band_energy_run(const std::vector<ScoreLaunch>& launches, char* ws, int n_bands,
                          double* fraction, double* total, hipStream_t stream);

// ------------------------------------------------------------- selection
struct TopRChunk {
  int32_t n, k;
  int64_t tok_off, sel_off, comp_off;
};
struct TopRLaunch {
  TopRChunk c[kMaxChunksPerLaunch];
  int32_t n_chunks;
};
// Index-array check (topr.hip): *bad = entries outside [0, bound), plus
// (ascending) entries not above their predecessor.
ct_status check_indices_run(const int32_t* idx, int32_t count, int32_t bound, bool ascending, int32_t* bad,
                            hipStream_t stream);
ct_status topr_run(const TopRLaunch& tl, const float* score, int32_t* ranking, int32_t* sel,
                   int32_t* comp, hipStream_t stream);

// -------------------------------------------------------------- assembly
struct AsmPlace {
  const void* k_src;
  const void* v_src;
  const int32_t* src_rows;
  const void* k_rec;
  const void* v_rec;
  const int32_t* sel;
  const int32_t* comp;
  int32_t n, k, offset, pad_;
};
constexpr int kMaxPlacesPerLaunch = 32;
struct AsmLaunch {
  AsmPlace p[kMaxPlacesPerLaunch];
  int32_t n_places;
  int32_t max_rows;
  int32_t H, D, dtype, style;
  double inv_freq[64];
};
ct_status assemble_run(const AsmLaunch& al, void* k_out, void* v_out, hipStream_t stream);

// ------------------------------------------------------------- attention
struct AttnArgs {
  const void* q;
  const int32_t* qpos;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int32_t n_q, Hq, T, H, D, dtype, style, group;
  float scale_log2;  // softmax_scale * log2(e)
  float scale;
  double inv_freq[64];
  // bf16 path: launch plan (attn_plan) and split-KV partials in the workspace
  int32_t seg_keys;  // keys per segment (multiple of 64)
  int32_t nseg;      // segments covering [0, T)
  int32_t nw;        // waves per block (8)
  int32_t qt;        // 32-row tiles per wave (1)
  int32_t hpb, tpb;  // query heads and 32-row tiles per block (hpb * tpb <= nw)
  int32_t n_hc;      // head chunks per group
  int32_t n_tg;      // tile groups (tpb * qt tiles each)
  float* part_o;     // [nseg][n_q][Hq][D] normalised partial outputs, fp32 (segments with wide V)
  uint16_t* part_o16;  // [nseg][n_q][Hq][D] the same as fp16 (every other segment)
  uint8_t* part_fmt;   // [nseg][n_q][Hq] 1: the record is in part_o, 0: in part_o16
  float* part_lse;   // [nseg][n_q][Hq] log2-sum-exp of the partials
  int32_t nblk;      // 64-key tiles covering [0, T)
  uint16_t* vt16;    // [H][nblk][D][64] V^T tiles as fp16 (keys permuted)
  int32_t* vflag;    // [H][nblk] tile holds a V outside the fp16 range
  uint16_t* qrot;    // [n_q][Hq][D] queries rotated to their positions, bf16
  int32_t blocks_per_head;  // persistent blocks serving each KV head
  int32_t* sched_order;     // [n_tg * nseg] work items (tg * nseg + seg), longest first
  int32_t* sched_cnt;       // [H] items taken so far by each head's blocks
  int32_t* sched_n;         // [1] items in sched_order
};
void attn_plan(AttnArgs* a, int n_cu);
size_t attn_ws_bytes(const AttnArgs& a);
ct_status attn_run(AttnArgs a, void* ws, size_t ws_bytes, hipStream_t stream);
// The same with the library's own per-device scratch array as the workspace
// (no allocation; shapes needing more than kNoAllocScratchBytes are refused).
constexpr size_t kNoAllocScratchBytes = size_t(256) << 20;
ct_status attn_run_noalloc(const AttnArgs& a, hipStream_t stream);
ct_status attn_f32_run(const AttnArgs& a, hipStream_t stream);
int device_cu_count();

// ------------------------------------------------------ recompute layer
ct_status rmsnorm_run(const void* x, const void* g, int rows, int dim, float eps, void* y,
                      hipStream_t stream);
ct_status silu_mul_run(const void* gu, int rows, int ff, void* out, hipStream_t stream);
ct_status linear_run(const void* x, const void* w, const void* residual, int m, int n, int k, void* out,
                     hipStream_t stream);
ct_status qkv_run(const void* x, const void* w_qkv, int m, int d, int nq, int nkv, void* q, void* k, void* v,
                  hipStream_t stream);

// ------------------------------------------------------------- host tier
ct_status rank_order_run(const void* k_src, const void* v_src, const int32_t* ranking, int32_t n,
                         int32_t L, int32_t row_bytes, void* k_dst, void* v_dst, hipStream_t stream);

}  // namespace ct

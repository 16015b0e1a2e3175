// C ABI entry points: argument validation, launch planning, error reporting.
// The operations themselves are defined in the header (include/cachetune.h)
// with their citations; this file only checks arguments and enqueues kernels.
#include <cmath>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "ct_internal.h"

namespace ct {

// Per-device context behind a ct_handle: the device, its compute units, and
// the scoring tables cachetune_prepare_scoring built (device memory owned by
// the context, freed by cachetune_destroy).
struct Context {
  int device = 0;
  int cu = 256;
  mutable std::mutex mu;
  struct Entry {
    int nf, kk, ntp;
    ScoreTables t;
    void* mem;
  };
  std::vector<Entry> tables;
};

bool context_find_tables(const Context* ctx, int nf, int kk, int ntp, ScoreTables* out) {
  if (!ctx) return false;
  std::lock_guard<std::mutex> lock(ctx->mu);
  for (const Context::Entry& e : ctx->tables)
    if (e.nf == nf && e.kk == kk && e.ntp == ntp) {
      *out = e.t;
      return true;
    }
  return false;
}

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

ct_status fail(ct_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

ct_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(CT_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return CT_OK;
}

static bool dtype_ok(int dt) { return dt == CT_F32 || dt == CT_BF16; }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

int context_cu_count(const Context* ctx) { return ctx ? ctx->cu : device_cu_count(); }

static void fill_inv_freq(double* f, int D, double theta) {
  for (int j = 0; j < 64; ++j) f[j] = 0.0;
  for (int j = 0; j < D / 2; ++j) f[j] = std::pow(theta, -2.0 * (double)j / (double)D);
}

}  // namespace ct

struct ct_ctx {
  ct::Context c;
};

using namespace ct;

#define CT_GUARD_BEGIN try {
#define CT_GUARD_END                                                   \
  }                                                                    \
  catch (const std::exception& e) {                                    \
    return fail(CT_E_INVALID, std::string("internal error: ") + e.what()); \
  }                                                                    \
  catch (...) {                                                        \
    return fail(CT_E_INVALID, "internal error");                       \
  }

extern "C" {

const char* cachetune_status_string(int32_t s) {
  switch (s) {
    case CT_OK: return "ok";
    case CT_E_INVALID: return "invalid argument";
    case CT_E_UNSUPPORTED: return "unsupported configuration";
    case CT_E_WORKSPACE: return "workspace missing or too small";
    case CT_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* cachetune_last_error(void) { return g_last_error.c_str(); }

int32_t cachetune_version(void) { return 2; }

// A handle's calls must run with its device current.
static ct_status ctx_of(ct_handle h, const Context** out) {
  *out = nullptr;
  if (!h) return CT_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CT_E_HIP, "hipGetDevice failed");
  if (dev != h->c.device)
    return fail(CT_E_INVALID, "the handle belongs to device " + std::to_string(h->c.device) +
                                  ", the current device is " + std::to_string(dev));
  *out = &h->c;
  return CT_OK;
}

ct_status cachetune_create(int32_t device, ct_handle* out) {
  CT_GUARD_BEGIN
  if (!out) return fail(CT_E_INVALID, "out is NULL");
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) return fail(CT_E_HIP, "hipGetDeviceCount failed");
  if (device < 0 || device >= n) return fail(CT_E_INVALID, "no device " + std::to_string(device));
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cu <= 0)
    return fail(CT_E_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
  ct_ctx* h = new ct_ctx();
  h->c.device = device;
  h->c.cu = cu;
  *out = h;
  return CT_OK;
  CT_GUARD_END
}

void cachetune_destroy(ct_handle h) {
  if (!h) return;
  for (Context::Entry& e : h->c.tables) (void)hipFree(e.mem);
  delete h;
}

ct_status cachetune_prepare_scoring(ct_handle h, const int32_t* n_per_chunk, int32_t n_chunks,
                                    int32_t alpha_num, int32_t alpha_den, ct_fftlen fftlen,
                                    hipStream_t stream) {
  CT_GUARD_BEGIN
  if (!h) return fail(CT_E_INVALID, "handle is NULL");
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  if (!n_per_chunk) return fail(CT_E_INVALID, "n_per_chunk is NULL");
  if (n_chunks < 1 || n_chunks > 4096) return fail(CT_E_INVALID, "n_chunks must be in [1, 4096]");
  if (alpha_den <= 0 || alpha_num <= 0 || alpha_num > alpha_den)
    return fail(CT_E_INVALID, "alpha = alpha_num/alpha_den must lie in (0, 1]");
  if (fftlen != CT_FFT_EXACT_N && fftlen != CT_FFT_ZEROPAD_POW2) return fail(CT_E_INVALID, "unknown fftlen mode");
  for (int b = 0; b < n_chunks; ++b) {
    const int n = n_per_chunk[b];
    if (n < 2 || n > kMaxN) return fail(CT_E_INVALID, "chunk length must be in [2, 8192]");
    if (fft_len(n, fftlen) > kMaxN) return fail(CT_E_UNSUPPORTED, "transform length above 8192");
  }
  Context& c = h->c;
  bool built = false;
  for (int b = 0; b < n_chunks; ++b) {
    const int n = n_per_chunk[b];
    const int nf = fft_len(n, fftlen), kk = kkeep(nf, alpha_num, alpha_den), ntp = (n + 31) / 32 * 32;
    ScoreTables t;
    if (context_find_tables(&c, nf, kk, ntp, &t)) continue;
    size_t o16 = 0, otr = 0;
    const size_t bytes = score_tables_bytes(nf, kk, ntp, &o16, &otr);
    void* mem = nullptr;
    if (hipMalloc(&mem, bytes) != hipSuccess) return fail(CT_E_HIP, "hipMalloc of the scoring tables failed");
    t.tw = reinterpret_cast<uint16_t*>(mem);
    t.tw16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(mem) + o16);
    t.trig = reinterpret_cast<double2*>(reinterpret_cast<char*>(mem) + otr);
    if (ct_status s = score_tables_build(nf, kk, ntp, CT_BF16, t, stream)) {
      (void)hipFree(mem);
      return s;
    }
    {
      std::lock_guard<std::mutex> lock(c.mu);
      c.tables.push_back(Context::Entry{nf, kk, ntp, t, mem});
    }
    built = true;
  }
  // later calls may run on other streams: the tables are complete on return
  if (built && hipStreamSynchronize(stream) != hipSuccess) return fail(CT_E_HIP, "hipStreamSynchronize failed");
  return CT_OK;
  CT_GUARD_END
}

static ct_status check_score_shapes(const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                    int32_t H, int32_t D, int32_t a_num, int32_t a_den,
                                    int32_t fftlen) {
  if (!n_per_chunk) return fail(CT_E_INVALID, "n_per_chunk is NULL");
  if (n_chunks < 1 || n_chunks > 4096) return fail(CT_E_INVALID, "n_chunks must be in [1, 4096]");
  if (L < 1 || L > 256) return fail(CT_E_INVALID, "L must be in [1, 256]");
  if (H < 1 || D < 1) return fail(CT_E_INVALID, "H and D must be positive");
  long long C = (long long)H * D;
  if (C % 64 != 0 || C > 8192) return fail(CT_E_UNSUPPORTED, "H*D must be a multiple of 64, at most 8192");
  if (a_den <= 0 || a_num <= 0 || a_num > a_den)
    return fail(CT_E_INVALID, "alpha = alpha_num/alpha_den must lie in (0, 1]");
  if (fftlen != CT_FFT_EXACT_N && fftlen != CT_FFT_ZEROPAD_POW2)
    return fail(CT_E_INVALID, "unknown fftlen mode");
  for (int b = 0; b < n_chunks; ++b) {
    int n = n_per_chunk[b];
    if (n < 2 || n > kMaxN) return fail(CT_E_INVALID, "chunk length must be in [2, 8192]");
    if (fft_len(n, (ct_fftlen)fftlen) > kMaxN) return fail(CT_E_UNSUPPORTED, "transform length above 8192");
  }
  return CT_OK;
}

ct_status cachetune_score_variant_ws(ct_handle h, const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                     int32_t H, int32_t D, int32_t alpha_num, int32_t alpha_den,
                                     ct_fftlen fftlen, ct_score_variant variant, size_t* bytes) {
  CT_GUARD_BEGIN
  if (!bytes) return fail(CT_E_INVALID, "bytes is NULL");
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  if (variant != CT_SCORE_LOWPASS && variant != CT_SCORE_L2 && variant != CT_SCORE_HIGHPASS)
    return fail(CT_E_INVALID, "unknown variant");
  if (variant == CT_SCORE_L2) {  // no transform: the cutoff and length are not used
    alpha_num = alpha_den = 1;
    fftlen = CT_FFT_EXACT_N;
  }
  if (ct_status s = check_score_shapes(n_per_chunk, n_chunks, L, H, D, alpha_num, alpha_den, fftlen))
    return s;
  return score_plan(n_per_chunk, n_chunks, L, H, D, alpha_num, alpha_den, fftlen, bytes, nullptr,
                    variant, cc);
  CT_GUARD_END
}

ct_status cachetune_score_chunk_ws(ct_handle h, const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                   int32_t H, int32_t D, int32_t alpha_num, int32_t alpha_den,
                                   ct_fftlen fftlen, size_t* bytes) {
  return cachetune_score_variant_ws(h, n_per_chunk, n_chunks, L, H, D, alpha_num, alpha_den, fftlen,
                                    CT_SCORE_LOWPASS, bytes);
}

ct_status cachetune_score_chunk(ct_handle h, const ct_chunk* chunks, int32_t n_chunks, int32_t L, int32_t H,
                                int32_t D, ct_dtype dtype, int32_t alpha_num, int32_t alpha_den,
                                ct_fftlen fftlen, ct_norm norm, float* score, float* layer_score,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  return cachetune_score_variant(h, chunks, n_chunks, L, H, D, dtype, alpha_num, alpha_den, fftlen, norm,
                                 CT_SCORE_LOWPASS, score, layer_score, ws, ws_bytes, stream);
}

ct_status cachetune_score_variant(ct_handle h, const ct_chunk* chunks, int32_t n_chunks, int32_t L, int32_t H,
                                  int32_t D, ct_dtype dtype, int32_t alpha_num, int32_t alpha_den,
                                  ct_fftlen fftlen, ct_norm norm, ct_score_variant variant,
                                  float* score, float* layer_score, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  CT_GUARD_BEGIN
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  if (variant != CT_SCORE_LOWPASS && variant != CT_SCORE_L2 && variant != CT_SCORE_HIGHPASS)
    return fail(CT_E_INVALID, "unknown variant");
  if (variant == CT_SCORE_L2) {  // no transform: the cutoff and length are not used
    alpha_num = alpha_den = 1;
    fftlen = CT_FFT_EXACT_N;
  }
  if (!chunks) return fail(CT_E_INVALID, "chunks is NULL");
  if (n_chunks < 1 || n_chunks > 4096) return fail(CT_E_INVALID, "n_chunks must be in [1, 4096]");
  if (!dtype_ok(dtype)) return fail(CT_E_INVALID, "unknown dtype");
  if (norm < CT_NORM_SUM || norm > CT_NORM_NONE) return fail(CT_E_INVALID, "unknown norm");
  if (!score) return fail(CT_E_INVALID, "score is NULL");
  std::vector<int32_t> ns(n_chunks);
  for (int b = 0; b < n_chunks; ++b) {
    if (!chunks[b].k || !chunks[b].v) return fail(CT_E_INVALID, "chunk K or V pointer is NULL");
    ns[b] = chunks[b].n;
  }
  if (ct_status s = check_score_shapes(ns.data(), n_chunks, L, H, D, alpha_num, alpha_den, fftlen))
    return s;
  size_t need = 0;
  std::vector<ScoreLaunch> launches;
  if (ct_status s = score_plan(ns.data(), n_chunks, L, H, D, alpha_num, alpha_den, fftlen, &need,
                               &launches, variant, cc))
    return s;
  if (!ws || ws_bytes < need)
    return fail(CT_E_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(CT_E_INVALID, "workspace must be 256-byte aligned");
  score_bind(&launches, reinterpret_cast<char*>(ws));
  int b0 = 0;
  for (ScoreLaunch& sl : launches) {
    sl.dtype = dtype;
    sl.norm = norm;
    for (int i = 0; i < sl.n_chunks; ++i) {
      sl.c[i].k = chunks[b0 + i].k;
      sl.c[i].v = chunks[b0 + i].v;
    }
    b0 += sl.n_chunks;
  }
  return score_run(launches, reinterpret_cast<char*>(ws), score, layer_score, stream);
  CT_GUARD_END
}

ct_status cachetune_band_energy_ws(const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                  int32_t H, int32_t D, ct_fftlen fftlen, size_t* bytes) {
  CT_GUARD_BEGIN
  if (!bytes) return fail(CT_E_INVALID, "bytes is NULL");
  if (ct_status s = check_score_shapes(n_per_chunk, n_chunks, L, H, D, 1, 1, fftlen)) return s;
  return score_plan(n_per_chunk, n_chunks, L, H, D, 1, 1, fftlen, bytes, nullptr, kVariantBandEnergy);
  CT_GUARD_END
}

ct_status cachetune_band_energy(const ct_chunk* chunks, int32_t n_chunks, int32_t L, int32_t H,
                                int32_t D, ct_dtype dtype, ct_fftlen fftlen, int32_t n_bands,
                                double* fraction, double* total, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  CT_GUARD_BEGIN
  if (!chunks) return fail(CT_E_INVALID, "chunks is NULL");
  if (n_chunks < 1 || n_chunks > 4096) return fail(CT_E_INVALID, "n_chunks must be in [1, 4096]");
  if (!dtype_ok(dtype)) return fail(CT_E_INVALID, "unknown dtype");
  if (!fraction) return fail(CT_E_INVALID, "fraction is NULL");
  std::vector<int32_t> ns(n_chunks);
  for (int b = 0; b < n_chunks; ++b) {
    if (!chunks[b].k || !chunks[b].v) return fail(CT_E_INVALID, "chunk K or V pointer is NULL");
    ns[b] = chunks[b].n;
  }
  if (ct_status s = check_score_shapes(ns.data(), n_chunks, L, H, D, 1, 1, fftlen)) return s;
  if (n_bands < 1 || n_bands > 1024) return fail(CT_E_INVALID, "n_bands must be in [1, 1024]");
  for (int b = 0; b < n_chunks; ++b)
    if (n_bands > fft_len(ns[b], fftlen) / 2 + 1)
      return fail(CT_E_INVALID, "n_bands above the bin count of a chunk");
  size_t need = 0;
  std::vector<ScoreLaunch> launches;
  if (ct_status s = score_plan(ns.data(), n_chunks, L, H, D, 1, 1, fftlen, &need, &launches,
                               kVariantBandEnergy))
    return s;
  if (!ws || ws_bytes < need)
    return fail(CT_E_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(CT_E_INVALID, "workspace must be 256-byte aligned");
  score_bind(&launches, reinterpret_cast<char*>(ws));
  int b0 = 0;
  for (ScoreLaunch& sl : launches) {
    sl.dtype = dtype;
    for (int i = 0; i < sl.n_chunks; ++i) {
      sl.c[i].k = chunks[b0 + i].k;
      sl.c[i].v = chunks[b0 + i].v;
    }
    b0 += sl.n_chunks;
  }
  return band_energy_run(launches, reinterpret_cast<char*>(ws), n_bands, fraction, total, stream);
  CT_GUARD_END
}

ct_status cachetune_rmsnorm(const void* x, const void* gain, int32_t rows, int32_t dim, float eps,
                            ct_dtype dtype, void* out, hipStream_t stream) {
  CT_GUARD_BEGIN
  if (dtype != CT_BF16) return fail(CT_E_UNSUPPORTED, "rmsnorm takes bf16 rows");
  if (rows < 0) return fail(CT_E_INVALID, "rows must be non-negative");
  if (dim < 8 || dim % 8 != 0 || dim > 65536) return fail(CT_E_INVALID, "dim must be a multiple of 8 in [8, 65536]");
  if (!(eps >= 0.0f)) return fail(CT_E_INVALID, "eps must be non-negative");
  if (rows > 0 && (!x || !gain || !out)) return fail(CT_E_INVALID, "NULL argument");
  if (rows > 0 && (!aligned16(x) || !aligned16(gain) || !aligned16(out)))
    return fail(CT_E_INVALID, "rows and gain must be 16-byte aligned");
  return rmsnorm_run(x, gain, rows, dim, eps, out, stream);
  CT_GUARD_END
}

ct_status cachetune_silu_mul(const void* gate_up, int32_t rows, int32_t ff, ct_dtype dtype, void* out,
                             hipStream_t stream) {
  CT_GUARD_BEGIN
  if (dtype != CT_BF16) return fail(CT_E_UNSUPPORTED, "silu_mul takes bf16 rows");
  if (rows < 0) return fail(CT_E_INVALID, "rows must be non-negative");
  if (ff < 8 || ff % 8 != 0) return fail(CT_E_INVALID, "ff must be a positive multiple of 8");
  if (rows > 0 && (!gate_up || !out)) return fail(CT_E_INVALID, "NULL argument");
  if (rows > 0 && (!aligned16(gate_up) || !aligned16(out)))
    return fail(CT_E_INVALID, "rows must be 16-byte aligned");
  return silu_mul_run(gate_up, rows, ff, out, stream);
  CT_GUARD_END
}

ct_status cachetune_linear(const void* x, const void* w, const void* residual, int32_t m, int32_t n,
                           int32_t k, ct_dtype dtype, void* out, hipStream_t stream) {
  CT_GUARD_BEGIN
  if (dtype != CT_BF16) return fail(CT_E_UNSUPPORTED, "linear takes bf16 operands");
  if (m < 0 || n < 1 || k < 1) return fail(CT_E_INVALID, "m must be non-negative, n and k positive");
  if (n % 8 != 0 || k % 8 != 0) return fail(CT_E_INVALID, "n and k must be multiples of 8");
  if ((long long)k * 256 * 2 >= (1LL << 31)) return fail(CT_E_UNSUPPORTED, "k above 4 194 303");
  if (m > 0 && (!x || !w || !out)) return fail(CT_E_INVALID, "NULL argument");
  if (m > 0 && (!aligned16(x) || !aligned16(w) || !aligned16(out) || (residual && !aligned16(residual))))
    return fail(CT_E_INVALID, "operands must be 16-byte aligned");
  if ((long long)(m + 127) / 128 > 65535) return fail(CT_E_UNSUPPORTED, "m above 8 388 480");
  return linear_run(x, w, residual, m, n, k, out, stream);
  CT_GUARD_END
}

ct_status cachetune_qkv_proj(const void* x, const void* w_qkv, int32_t m, int32_t d, int32_t nq,
                             int32_t nkv, ct_dtype dtype, void* q_out, void* k_out, void* v_out,
                             hipStream_t stream) {
  CT_GUARD_BEGIN
  if (dtype != CT_BF16) return fail(CT_E_UNSUPPORTED, "qkv_proj takes bf16 operands");
  if (m < 0 || d < 1 || nq < 1 || nkv < 1) return fail(CT_E_INVALID, "m must be non-negative, d, nq, nkv positive");
  if (d % 8 != 0 || nq % 8 != 0 || nkv % 8 != 0) return fail(CT_E_INVALID, "d, nq and nkv must be multiples of 8");
  if ((long long)d * 256 * 2 >= (1LL << 31)) return fail(CT_E_UNSUPPORTED, "d above 4 194 303");
  if ((long long)nq + 2LL * nkv > (1LL << 30)) return fail(CT_E_UNSUPPORTED, "nq + 2 nkv too large");
  if ((long long)(m + 127) / 128 > 65535) return fail(CT_E_UNSUPPORTED, "m above 8 388 480");
  if (m > 0 && (!x || !w_qkv || !q_out || !k_out || !v_out)) return fail(CT_E_INVALID, "NULL argument");
  if (m > 0 && (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out)))
    return fail(CT_E_INVALID, "operands must be 16-byte aligned");
  return qkv_run(x, w_qkv, m, d, nq, nkv, q_out, k_out, v_out, stream);
  CT_GUARD_END
}

static ct_status topr_counts(const int32_t* n_per_chunk, int32_t n_chunks, int32_t r_num, int32_t r_den,
                             int32_t* ks) {
  if (!n_per_chunk || !ks) return fail(CT_E_INVALID, "NULL argument");
  if (n_chunks < 1 || n_chunks > 65536) return fail(CT_E_INVALID, "n_chunks must be in [1, 65536]");
  if (r_den <= 0 || r_num < 0 || r_num > r_den) return fail(CT_E_INVALID, "r must lie in [0, 1]");
  for (int b = 0; b < n_chunks; ++b) {
    const int n = n_per_chunk[b];
    if (n < 1 || n > kMaxN) return fail(CT_E_INVALID, "chunk length must be in [1, 8192]");
    ks[b] = (int32_t)(((long long)r_num * n) / r_den);
  }
  return CT_OK;
}

ct_status cachetune_check_indices(const int32_t* idx, int32_t count, int32_t bound, int32_t ascending,
                                  int32_t* bad, hipStream_t stream) {
  CT_GUARD_BEGIN
  if (!bad) return fail(CT_E_INVALID, "bad is NULL");
  if (count < 0 || bound < 0) return fail(CT_E_INVALID, "count and bound must be >= 0");
  if (count > 0 && !idx) return fail(CT_E_INVALID, "idx is NULL");
  return check_indices_run(idx, count, bound, ascending != 0, bad, stream);
  CT_GUARD_END
}

ct_status cachetune_select_topr_counts(const int32_t* n_per_chunk, int32_t n_chunks, int32_t r_num,
                                       int32_t r_den, int32_t* k_per_chunk) {
  CT_GUARD_BEGIN
  return topr_counts(n_per_chunk, n_chunks, r_num, r_den, k_per_chunk);
  CT_GUARD_END
}

ct_status cachetune_select_topr(ct_handle h, const float* score, const int32_t* n_per_chunk, int32_t n_chunks,
                                int32_t r_num, int32_t r_den, int32_t* ranking, int32_t* sel,
                                int32_t* comp, int32_t* k_per_chunk, hipStream_t stream) {
  CT_GUARD_BEGIN
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  if (!score || !n_per_chunk || !k_per_chunk) return fail(CT_E_INVALID, "NULL argument");
  std::vector<int32_t> ks((size_t)std::max(n_chunks, 1));
  if (ct_status s = topr_counts(n_per_chunk, n_chunks, r_num, r_den, ks.data())) return s;
  long long tok = 0, sk = 0, sc = 0;
  bool any_sel = false;
  for (int b = 0; b < n_chunks; ++b) any_sel |= ks[b] > 0;
  if (any_sel && !sel) return fail(CT_E_INVALID, "sel is NULL");
  for (int b0 = 0; b0 < n_chunks; b0 += kMaxChunksPerLaunch) {
    TopRLaunch tl{};
    tl.n_chunks = std::min(kMaxChunksPerLaunch, n_chunks - b0);
    for (int i = 0; i < tl.n_chunks; ++i) {
      int b = b0 + i;
      tl.c[i].n = n_per_chunk[b];
      tl.c[i].k = ks[b];
      tl.c[i].tok_off = tok;
      tl.c[i].sel_off = sk;
      tl.c[i].comp_off = sc;
      tok += n_per_chunk[b];
      sk += ks[b];
      sc += n_per_chunk[b] - ks[b];
    }
    if (ct_status s = topr_run(tl, score, ranking, sel, comp, stream)) return s;
  }
  for (int b = 0; b < n_chunks; ++b) k_per_chunk[b] = ks[b];
  return CT_OK;
  CT_GUARD_END
}

ct_status cachetune_assemble_rope(ct_handle h, const ct_place* places, int32_t n_places, const void* k_sfx,
                                  const void* v_sfx, int32_t n_sfx, int32_t sfx_offset, int32_t H,
                                  int32_t D, ct_dtype dtype, double rope_theta, ct_rope style,
                                  void* k_out, void* v_out, int32_t T, hipStream_t stream) {
  CT_GUARD_BEGIN
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  if (!dtype_ok(dtype)) return fail(CT_E_INVALID, "unknown dtype");
  if (D != 64 && D != 128) return fail(CT_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (H < 1) return fail(CT_E_INVALID, "H must be positive");
  if (style != CT_ROPE_HALF && style != CT_ROPE_INTERLEAVED) return fail(CT_E_INVALID, "unknown RoPE style");
  if (!(rope_theta > 1.0) || !std::isfinite(rope_theta)) return fail(CT_E_INVALID, "rope_theta must be > 1");
  if (!k_out || !v_out) return fail(CT_E_INVALID, "output is NULL");
  if (T < 1) return fail(CT_E_INVALID, "T must be positive");
  if (n_places < 0 || (n_places > 0 && !places)) return fail(CT_E_INVALID, "places invalid");
  if (n_sfx < 0) return fail(CT_E_INVALID, "n_sfx must be >= 0");
  if (n_sfx > 0) {
    if (!k_sfx || !v_sfx) return fail(CT_E_INVALID, "suffix pointers are NULL");
    if (sfx_offset < 0 || (long long)sfx_offset + n_sfx > T) return fail(CT_E_INVALID, "suffix rows outside [0, T)");
  }
  for (int i = 0; i < n_places; ++i) {
    const ct_place& p = places[i];
    if (p.n < 1 || p.k < 0 || p.k > p.n) return fail(CT_E_INVALID, "place: need 0 <= k <= n, n >= 1");
    if (p.offset < 0 || (long long)p.offset + p.n > T) return fail(CT_E_INVALID, "place rows outside [0, T)");
    if (p.k < p.n && (!p.k_src || !p.v_src)) return fail(CT_E_INVALID, "place: cached rows are NULL");
    if (p.k < p.n && !p.src_rows && !p.comp) return fail(CT_E_INVALID, "place: comp and src_rows are both NULL");
    if (p.k > 0 && (!p.k_rec || !p.v_rec || !p.sel)) return fail(CT_E_INVALID, "place: recomputed rows are NULL");
  }
  bool al_ok = aligned16(k_out) && aligned16(v_out) && aligned16(k_sfx) && aligned16(v_sfx);
  for (int i = 0; i < n_places; ++i)
    al_ok = al_ok && aligned16(places[i].k_src) && aligned16(places[i].v_src) &&
            aligned16(places[i].k_rec) && aligned16(places[i].v_rec);
  if (!al_ok) return fail(CT_E_INVALID, "row buffers must be 16-byte aligned");
  std::vector<AsmPlace> all;
  for (int i = 0; i < n_places; ++i) {
    const ct_place& p = places[i];
    AsmPlace a{p.k_src, p.v_src, p.src_rows, p.k_rec, p.v_rec, p.sel, p.comp, p.n, p.k, p.offset, 0};
    all.push_back(a);
  }
  if (n_sfx > 0) {
    AsmPlace a{k_sfx, v_sfx, nullptr, nullptr, nullptr, nullptr, nullptr, n_sfx, 0, sfx_offset, 1};
    all.push_back(a);
  }
  for (size_t i0 = 0; i0 < all.size(); i0 += kMaxPlacesPerLaunch) {
    AsmLaunch al{};
    al.n_places = (int32_t)std::min<size_t>(kMaxPlacesPerLaunch, all.size() - i0);
    al.max_rows = 0;
    for (int i = 0; i < al.n_places; ++i) {
      al.p[i] = all[i0 + i];
      al.max_rows = std::max(al.max_rows, al.p[i].n);
    }
    al.H = H;
    al.D = D;
    al.dtype = dtype;
    al.style = style;
    fill_inv_freq(al.inv_freq, D, rope_theta);
    if (ct_status s = assemble_run(al, k_out, v_out, stream)) return s;
  }
  return CT_OK;
  CT_GUARD_END
}

static ct_status attn_args(const Context* cc, const void* q_pre, const int32_t* q_pos, int32_t n_q, int32_t Hq,
                           const void* k, const void* v, int32_t T, int32_t H, int32_t D,
                           int32_t dtype, float softmax_scale, double rope_theta, int32_t style,
                           void* out, float* lse, bool need_ptrs, AttnArgs* a) {
  if (!dtype_ok(dtype)) return fail(CT_E_INVALID, "unknown dtype");
  if (D != 64 && D != 128) return fail(CT_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (H < 1 || Hq < 1 || Hq % H != 0) return fail(CT_E_INVALID, "need Hq % H == 0");
  if (style != CT_ROPE_HALF && style != CT_ROPE_INTERLEAVED) return fail(CT_E_INVALID, "unknown RoPE style");
  if (!(rope_theta > 1.0) || !std::isfinite(rope_theta)) return fail(CT_E_INVALID, "rope_theta must be > 1");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CT_E_INVALID, "softmax_scale must be positive and finite");
  if (n_q < 0 || T < 1) return fail(CT_E_INVALID, "need n_q >= 0, T >= 1");
  if (need_ptrs && n_q > 0 && (!q_pre || !q_pos || !k || !v || !out)) return fail(CT_E_INVALID, "NULL argument");
  if (need_ptrs && !(aligned16(q_pre) && aligned16(k) && aligned16(v) && aligned16(out)))
    return fail(CT_E_INVALID, "q_pre, k, v and out must be 16-byte aligned");
  if ((long long)(n_q + 31) / 32 * Hq > (long long)INT32_MAX / 64)
    return fail(CT_E_UNSUPPORTED, "too many query rows");
  *a = AttnArgs{};
  a->q = q_pre;
  a->qpos = q_pos;
  a->k = k;
  a->v = v;
  a->out = out;
  a->lse = lse;
  a->n_q = n_q;
  a->Hq = Hq;
  a->T = T;
  a->H = H;
  a->D = D;
  a->dtype = dtype;
  a->style = style;
  a->group = Hq / H;
  a->scale = softmax_scale;
  a->scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  fill_inv_freq(a->inv_freq, D, rope_theta);
  attn_plan(a, context_cu_count(cc));
  return CT_OK;
}

ct_status cachetune_recompute_attn_ws(ct_handle h, int32_t n_q, int32_t Hq, int32_t T, int32_t H, int32_t D,
                                      ct_dtype dtype, size_t* bytes) {
  CT_GUARD_BEGIN
  if (!bytes) return fail(CT_E_INVALID, "bytes is NULL");
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  AttnArgs a;
  if (ct_status s = attn_args(cc, nullptr, nullptr, n_q, Hq, nullptr, nullptr, T, H, D, dtype, 1.f,
                              10000.0, CT_ROPE_HALF, nullptr, nullptr, false, &a))
    return s;
  *bytes = attn_ws_bytes(a);
  return CT_OK;
  CT_GUARD_END
}

ct_status cachetune_recompute_attn(ct_handle h, const void* q_pre, const int32_t* q_pos, int32_t n_q,
                                   int32_t Hq, const void* k, const void* v, int32_t T,
                                   int32_t H, int32_t D, ct_dtype dtype, float softmax_scale,
                                   double rope_theta, ct_rope style, void* out, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  CT_GUARD_BEGIN
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  AttnArgs a;
  if (ct_status s = attn_args(cc, q_pre, q_pos, n_q, Hq, k, v, T, H, D, dtype, softmax_scale,
                              rope_theta, style, out, lse, true, &a))
    return s;
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(CT_E_INVALID, "workspace must be 256-byte aligned");
  return attn_run(a, ws, ws_bytes, stream);
  CT_GUARD_END
}

ct_status cachetune_recompute_attn_noalloc(ct_handle h, const void* q_pre, const int32_t* q_pos, int32_t n_q,
                                           int32_t Hq, const void* k, const void* v, int32_t T,
                                           int32_t H, int32_t D, ct_dtype dtype, float softmax_scale,
                                           double rope_theta, ct_rope style, void* out, float* lse,
                                           hipStream_t stream) {
  CT_GUARD_BEGIN
  const Context* cc = nullptr;
  if (ct_status s = ctx_of(h, &cc)) return s;
  AttnArgs a;
  if (ct_status s = attn_args(cc, q_pre, q_pos, n_q, Hq, k, v, T, H, D, dtype, softmax_scale,
                              rope_theta, style, out, lse, true, &a))
    return s;
  return attn_run_noalloc(a, stream);
  CT_GUARD_END
}

ct_status cachetune_rank_order(const void* k_src, const void* v_src, const int32_t* ranking,
                               int32_t n, int32_t L, int32_t H, int32_t D, ct_dtype dtype,
                               void* k_dst, void* v_dst, hipStream_t stream) {
  CT_GUARD_BEGIN
  if (!dtype_ok(dtype)) return fail(CT_E_INVALID, "unknown dtype");
  if (n < 1 || n > kMaxN || L < 1 || H < 1 || D < 1) return fail(CT_E_INVALID, "bad shape");
  const long long row_bytes = (long long)H * D * (dtype == CT_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || row_bytes > (1LL << 30)) return fail(CT_E_UNSUPPORTED, "H*D*element size must be a multiple of 16 bytes");
  if (!k_src || !v_src || !ranking || !k_dst || !v_dst) return fail(CT_E_INVALID, "NULL argument");
  if (!(aligned16(k_src) && aligned16(v_src) && aligned16(k_dst) && aligned16(v_dst)))
    return fail(CT_E_INVALID, "row buffers must be 16-byte aligned");
  if (k_src == k_dst || v_src == v_dst || k_src == v_dst || v_src == k_dst)
    return fail(CT_E_INVALID, "destination must not alias the source");
  return rank_order_run(k_src, v_src, ranking, n, L, (int32_t)row_bytes, k_dst, v_dst, stream);
  CT_GUARD_END
}

ct_status cachetune_stage_complement(const ct_ranked_chunk* chunks, int32_t n_chunks, int32_t layer,
                                     int32_t H, int32_t D, ct_dtype dtype,
                                     const int32_t* k_per_chunk, void* k_stage, void* v_stage,
                                     hipStream_t stream) {
  CT_GUARD_BEGIN
  if (!dtype_ok(dtype)) return fail(CT_E_INVALID, "unknown dtype");
  if (!chunks || !k_per_chunk || n_chunks < 1) return fail(CT_E_INVALID, "NULL argument or no chunks");
  if (layer < 0 || H < 1 || D < 1) return fail(CT_E_INVALID, "bad shape");
  const size_t row_bytes = (size_t)H * D * (dtype == CT_BF16 ? 2 : 4);
  size_t rows = 0;
  for (int b = 0; b < n_chunks; ++b) {
    const ct_ranked_chunk& c = chunks[b];
    if (c.n < 1 || c.n > kMaxN || layer >= c.L) return fail(CT_E_INVALID, "chunk: bad n or layer");
    if (k_per_chunk[b] < 0 || k_per_chunk[b] > c.n) return fail(CT_E_INVALID, "k outside [0, n]");
    if (k_per_chunk[b] < c.n && (!c.k || !c.v)) return fail(CT_E_INVALID, "chunk rows are NULL");
    rows += (size_t)(c.n - k_per_chunk[b]);
  }
  if (rows > 0 && (!k_stage || !v_stage)) return fail(CT_E_INVALID, "staging buffers are NULL");
  size_t at = 0;
  for (int b = 0; b < n_chunks; ++b) {
    const ct_ranked_chunk& c = chunks[b];
    const size_t tail = (size_t)(c.n - k_per_chunk[b]);
    if (tail == 0) continue;
    const size_t src = ((size_t)layer * c.n + k_per_chunk[b]) * row_bytes;
    const size_t dst = at * row_bytes;
    if (hipMemcpyAsync(reinterpret_cast<char*>(k_stage) + dst, reinterpret_cast<const char*>(c.k) + src,
                       tail * row_bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipMemcpyAsync(reinterpret_cast<char*>(v_stage) + dst, reinterpret_cast<const char*>(c.v) + src,
                       tail * row_bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
      return fail(CT_E_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(hipGetLastError()));
    at += tail;
  }
  return CT_OK;
  CT_GUARD_END
}

}  // extern "C"

/*
 * cachetune.h -- C ABI of the MI355X (gfx950) CacheTune hot path.
 *
 * The four calls follow the problem statement of "Adaptive KV Cache Reuse for
 * Fast Long-Context LLM Serving" (CacheTune):
 *   cachetune_score_chunk     App. B.1: frequency-domain importance score of
 *                             each independently encoded chunk
 *   cachetune_select_topr     App. B.1: stored ranking and the top-rN
 *                             recomputation set / reuse complement
 *   cachetune_assemble_rope   App. B.2 and B.3: per-layer working buffer
 *                             assembled from reused and recomputed rows, keys
 *                             rotated at their global positions
 *   cachetune_recompute_attn  Sec. 4.1 "Recomputing in the new context" and
 *                             App. B.2 "check layer": the selected queries
 *                             attend causally over the assembled layer
 *
 * Conventions shared by every call:
 *  - Memory: the caller owns all buffers.  "device" pointers are HIP device
 *    memory of the current device; "host" pointers are ordinary host memory
 *    read before the call returns.  The library allocates device memory only
 *    in cachetune_prepare_scoring (constant tables kept by a handle, freed by
 *    cachetune_destroy).
 *  - Handle: the four calls take a ct_handle (cachetune_create) as their first
 *    argument; NULL is accepted everywhere and makes each call self-contained
 *    (the scoring tables are then rebuilt in the caller's workspace by every
 *    call).  A handle's calls must run with its device current.
 *  - Asynchrony: arguments are validated synchronously; work is then enqueued
 *    on `stream` and the call returns without synchronising.  A call that
 *    fails validation enqueues nothing.
 *  - Errors: every call returns a ct_status; no exception crosses the ABI.
 *    cachetune_last_error() gives a message for the calling thread's last
 *    failure.  CT_E_HIP means a HIP launch failed (the stream may hold work
 *    enqueued by earlier launches of the same call).
 *  - Storage types: CT_F32 (IEEE binary32) and CT_BF16 (bfloat16).  Results
 *    are rounded once, to nearest even.
 *  - Layout: per-layer tensors are row-major [rows][H][D] (token-major, the
 *    H*D channels of one token contiguous).  Chunk tensors are [L][n][H][D].
 *    Row-data pointers (keys, values, queries, outputs) must be 16-byte
 *    aligned; a misaligned one is rejected with CT_E_INVALID.
 *  - Determinism: identical inputs give bit-identical outputs (no floating
 *    point atomics, fixed reduction orders).
 *  - Concurrency: calls on different streams may run concurrently as long as
 *    their output and workspace buffers do not overlap.
 *  - Positions and indices are 0-based: chunk b placed at global offset o_b
 *    maps its local row i to o_b + i (App. B.1 writes this 1-based as
 *    o_b + i - 1).
 */
#ifndef CACHETUNE_H
#define CACHETUNE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
/* C++ gives the enums a fixed 32-bit underlying type, so that any int32 value a
 * C caller passes is a value of the type (and is then rejected by the call's
 * validation) rather than undefined behaviour; C sees int-sized enums. */
#define CT_ENUM_BASE : int32_t
#else
#define CT_ENUM_BASE
#endif

typedef enum CT_ENUM_BASE {
  CT_OK = 0,
  CT_E_INVALID = -1,     /* bad argument (null pointer, size, ratio ...) */
  CT_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim) */
  CT_E_WORKSPACE = -3,   /* workspace missing or smaller than required */
  CT_E_HIP = -4          /* a HIP runtime call or kernel launch failed */
} ct_status;

typedef enum CT_ENUM_BASE { CT_F32 = 0, CT_BF16 = 1 } ct_dtype;

/* Per-layer normalisation of the chunk scores (App. B.1 states only that the
 * scores are normalised within each layer).  CT_NORM_SUM divides by the layer
 * sum (a layer whose sum is 0 becomes uniform 1/n); CT_NORM_MAX divides by the
 * layer maximum; CT_NORM_MINMAX maps [min, max] to [0, 1]; CT_NORM_NONE keeps
 * the raw values.  Degenerate MAX / MINMAX layers become 0. */
typedef enum CT_ENUM_BASE { CT_NORM_SUM = 0, CT_NORM_MAX = 1, CT_NORM_MINMAX = 2, CT_NORM_NONE = 3 } ct_norm;

/* RoPE pairing: rotate-half pairs (j, j + D/2); interleaved pairs (2j, 2j+1).
 * Pair j turns by pos * theta^(-2j/D). */
typedef enum CT_ENUM_BASE { CT_ROPE_HALF = 0, CT_ROPE_INTERLEAVED = 1 } ct_rope;

/* Transform length of a chunk of n tokens: the exact length n (App. B.1), or
 * the next power of two with the chunk zero-padded (the retained-bin count is
 * then taken over that length's bins and positions [0, n) are scored). */
typedef enum CT_ENUM_BASE { CT_FFT_EXACT_N = 0, CT_FFT_ZEROPAD_POW2 = 1 } ct_fftlen;

/* One independently encoded chunk: pre-RoPE keys and values, [L][n][H][D],
 * device memory.  n in [2, 8192]. */
typedef struct {
  const void* k;
  const void* v;
  int32_t n;
} ct_chunk;

/* One chunk placed in a request, for ONE layer (App. B.2 fusion).
 *  k_src, v_src  cached pre-RoPE rows of the layer (device):
 *                src_rows == NULL: the full chunk layer [n][H][D], indexed by
 *                                  local row; the reused rows are comp[0..n-k)
 *                src_rows != NULL: a packed buffer [n-k][H][D] whose row j holds
 *                                  local row src_rows[j] (device array)
 *  k_rec, v_rec  recomputed pre-RoPE rows [k][H][D] (device); row t belongs to
 *                local row sel[t]
 *  sel           device, k ascending local indices of the recomputation set
 *  comp          device, n-k ascending local indices of the reuse complement
 *                (only read when src_rows == NULL)
 *  n, k, offset  rows of the chunk, recomputed rows, global start o_b
 * The output rows offset .. offset+n-1 are written. */
typedef struct {
  const void* k_src;
  const void* v_src;
  const int32_t* src_rows;
  const void* k_rec;
  const void* v_rec;
  const int32_t* sel;
  const int32_t* comp;
  int32_t n;
  int32_t k;
  int32_t offset;
} ct_place;

const char* cachetune_status_string(int32_t status);
const char* cachetune_last_error(void);
int32_t cachetune_version(void);

/* ---- context handle --------------------------------------------------------
 * A per-device context holding what the calls would otherwise recompute:
 * the device's compute-unit count (launch planning of the attention) and the
 * scoring path's constant tables -- the twiddle planes of the retained band
 * (cos and sin of 2*pi*j*n/m for bins j < K_keep and tokens n) and the
 * trigonometric table of each transform length m -- which App. B.1 treats as
 * preprocessing amortised over every chunk of that length.
 *
 * cachetune_create: a context for HIP device `device`; *out receives it.
 *   Allocates no device memory.  CT_E_INVALID for a device that does not
 *   exist.
 * cachetune_destroy: frees the context and its tables (NULL is ignored).  All
 *   work enqueued with the handle must have completed.
 * cachetune_prepare_scoring: builds, in device memory owned by the context,
 *   the tables that score calls with these chunk lengths, alpha and fftlen
 *   use (tables already held are kept); then synchronises `stream`, so the
 *   tables are complete for calls on any stream.  Later score calls with the
 *   handle use them instead of rebuilding them in the workspace (and their
 *   workspace query no longer counts them).  Arguments and errors as
 *   cachetune_score_chunk_ws; CT_E_HIP if an allocation fails. */
typedef struct ct_ctx* ct_handle;
ct_status cachetune_create(int32_t device, ct_handle* out);
void cachetune_destroy(ct_handle h);
ct_status cachetune_prepare_scoring(ct_handle h, const int32_t* n_per_chunk, int32_t n_chunks,
                                    int32_t alpha_num, int32_t alpha_den, ct_fftlen fftlen,
                                    hipStream_t stream);

/* ---- scoring (App. B.1) ---------------------------------------------------
 * For each chunk and layer: along the token axis of every (head, channel)
 * sequence, a real DFT; bins at and above K_keep = max(1, floor(alpha * (m/2+1)))
 * are zeroed (m = transform length, alpha = alpha_num / alpha_den in (0, 1]);
 * the inverse transform with output length m gives the low-frequency tensor
 * at the original positions.  Per token: a = L2 norm of the low-passed K over
 * its H*D channels, b = the same for V; s = a/2 + b/2; s is normalised within
 * the layer (`norm`); the chunk score is the mean over the L layers.
 *
 * Workspace query: writes the required workspace size for these shapes.
 *   n_per_chunk: host, n_chunks entries. */
ct_status cachetune_score_chunk_ws(ct_handle h, const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                   int32_t H, int32_t D, int32_t alpha_num, int32_t alpha_den,
                                   ct_fftlen fftlen, size_t* bytes);

/* chunks: host array of n_chunks descriptors (1 <= n_chunks <= 4096).
 * H*D must be a multiple of 64 and at most 8192; L in [1, 256].
 * score:       device float[sum n], chunk scores concatenated in the order of
 *              `chunks` (fp32, computed through fp64 reductions)
 * layer_score: device float[L][sum n] normalised per-layer scores, or NULL
 * ws/ws_bytes: device workspace of at least cachetune_score_chunk_ws bytes,
 *              256-byte aligned; its contents are scratch. */
ct_status cachetune_score_chunk(ct_handle h, const ct_chunk* chunks, int32_t n_chunks, int32_t L, int32_t H,
                                int32_t D, ct_dtype dtype, int32_t alpha_num, int32_t alpha_den,
                                ct_fftlen fftlen, ct_norm norm, float* score, float* layer_score,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- scoring variants the pages compare (§5.4, App. E.2, App. E.4) ----------
 *   CT_SCORE_LOWPASS  the score of cachetune_score_chunk.
 *   CT_SCORE_L2       the same joint K/V magnitudes, layer normalisation and
 *                     layer mean without the frequency analysis: a = L2 norm
 *                     of K over the token's H*D channels, b the same for V
 *                     (the alpha = 1 score of App. E.4, which keeps every bin;
 *                     alpha_num / alpha_den and fftlen are ignored).
 *   CT_SCORE_HIGHPASS the high-frequency-guided strategy of Sec. 5.4 and
 *                     App. E.2 (Table 3, Figure 1): the same magnitudes of
 *                     the reconstruction from the bins at and above the
 *                     low-pass cutoff (bins >= kk for the same alpha and
 *                     fftlen), i.e. of x - xlow at the stored positions.
 *                     Needs the workspace of the low-pass score.
 * Random selection needs no score of its own: cachetune_select_topr over
 * caller-supplied seeded uniform scores selects a uniformly random set.
 * Arguments, layouts and errors are those of cachetune_score_chunk(_ws); an
 * unknown variant is CT_E_INVALID. */
typedef enum CT_ENUM_BASE { CT_SCORE_LOWPASS = 0, CT_SCORE_L2 = 1, CT_SCORE_HIGHPASS = 2 } ct_score_variant;
ct_status cachetune_score_variant_ws(ct_handle h, const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                     int32_t H, int32_t D, int32_t alpha_num, int32_t alpha_den,
                                     ct_fftlen fftlen, ct_score_variant variant, size_t* bytes);
ct_status cachetune_score_variant(ct_handle h, const ct_chunk* chunks, int32_t n_chunks, int32_t L, int32_t H,
                                  int32_t D, ct_dtype dtype, int32_t alpha_num, int32_t alpha_den,
                                  ct_fftlen fftlen, ct_norm norm, ct_score_variant variant,
                                  float* score, float* layer_score, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---- frequency-band energy fractions (App. E.1, Figure 9) ------------------
 * For every chunk, layer and tensor (K, V): the rFFT of each channel along the
 * tokens (transform length per fftlen, as cachetune_score_chunk), bin j
 * carrying w_j |X_j|^2 / nf summed over the H*D channels (w_j = 1 at DC and
 * Nyquist, else 2; the bins sum to the energy of the stored rows), grouped
 * into n_bands equal bands of the bin range [0, nb): bin j in band
 * floor(j * n_bands / nb).
 *  chunks, L, H, D, dtype, fftlen: as cachetune_score_chunk
 *  n_bands:  in [1, 1024] and at most the bin count nb of every chunk
 *  fraction: device double[n_chunks][L][2][n_bands] (2: K then V), band
 *            energy over the total (0 when the total is 0)
 *  total:    device double[n_chunks][L][2] total energies, or NULL
 *  ws:       device workspace of cachetune_band_energy_ws bytes, 256-aligned:
 *            the coefficients of every bin, L*2*2*nb*H*D*4 bytes per chunk
 *            (about 545 MB for 32 layers of 2048 tokens and 8 x 128 channels)
 * Deterministic (fixed-order fp64 sums).  Errors as cachetune_score_chunk;
 * n_bands out of range is CT_E_INVALID.  Asynchronous on `stream`. */
ct_status cachetune_band_energy_ws(const int32_t* n_per_chunk, int32_t n_chunks, int32_t L,
                                  int32_t H, int32_t D, ct_fftlen fftlen, size_t* bytes);
ct_status cachetune_band_energy(const ct_chunk* chunks, int32_t n_chunks, int32_t L, int32_t H,
                                int32_t D, ct_dtype dtype, ct_fftlen fftlen, int32_t n_bands,
                                double* fraction, double* total, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* ---- the rest of the selective-recompute layer (Sec. 4.1, App. B.2) --------
 * The selected tokens and the uncached suffix run through every layer in the
 * new context.  Besides assembly and attention, a layer of the models the
 * pages evaluate (Sec. 5.1, Llama-3-8B-shaped) normalises their hidden rows,
 * projects them to q / k / v (bias-free), projects the attention output back
 * with a residual, and applies the gated MLP (silu(gate) * up, down projection,
 * residual).  All tensors are bf16, row-major, device memory owned by the
 * caller; every output element is rounded once to bf16.
 *
 * cachetune_rmsnorm: out[r][c] = x[r][c] / sqrt(mean_c x[r][c]^2 + eps) * gain[c]
 *   (fp32 arithmetic).  x, out: [rows][dim]; gain: [dim]; dim a multiple of 8
 *   in [8, 65536]; 16-byte aligned.  out may equal x.
 * cachetune_silu_mul: out[r][j] = silu(gu[r][j]) * gu[r][ff + j] with
 *   silu(g) = g / (1 + exp(-g)) (fp32).  gate_up: [rows][2 ff]; out: [rows][ff];
 *   ff a multiple of 8; 16-byte aligned.
 * cachetune_linear: out[i][j] = sum_k x[i][k] w[j][k] (+ residual[i][j]) on the
 *   matrix cores (bf16 products, fp32 accumulation, the residual added before
 *   the one rounding).  x: [m][k]; w: [n][k] (the usual [out][in] weight
 *   layout); residual: [m][n] or NULL (may equal out); out: [m][n].  n, k
 *   multiples of 8, k below 4 194 304; 16-byte aligned.  No workspace.
 * cachetune_qkv_proj: the fused q / k / v projection of the rows: one product
 *   with w_qkv = [wq; wk; wv] ([nq + 2 nkv][d], the three weights stacked by
 *   rows), its output columns split into q_out [m][nq], k_out [m][nkv] and
 *   v_out [m][nkv] (each a plain row-major buffer, as the assembly and the
 *   attention take them).  Arithmetic as cachetune_linear, no residual.
 * Errors: CT_E_INVALID (shapes, NULL, alignment), CT_E_UNSUPPORTED (dtype other
 * than bf16, sizes past the stated limits), CT_E_HIP.  Asynchronous on `stream`. */
ct_status cachetune_rmsnorm(const void* x, const void* gain, int32_t rows, int32_t dim, float eps,
                            ct_dtype dtype, void* out, hipStream_t stream);
ct_status cachetune_silu_mul(const void* gate_up, int32_t rows, int32_t ff, ct_dtype dtype, void* out,
                             hipStream_t stream);
ct_status cachetune_linear(const void* x, const void* w, const void* residual, int32_t m, int32_t n,
                           int32_t k, ct_dtype dtype, void* out, hipStream_t stream);
ct_status cachetune_qkv_proj(const void* x, const void* w_qkv, int32_t m, int32_t d, int32_t nq,
                             int32_t nkv, ct_dtype dtype, void* q_out, void* k_out, void* v_out,
                             hipStream_t stream);

/* ---- selection (App. B.1) -------------------------------------------------
 * Per chunk of n scores: k = floor(r * n) with r = r_num / r_den in [0, 1].
 * Ranking order: higher score first, equal scores by lower local index (the
 * fp32 values are compared exactly; -0 equals +0; NaN ranks last).
 *  score:       device float[sum n] (as written by cachetune_score_chunk)
 *  n_per_chunk: host, n_chunks entries, each in [1, 8192]
 *  ranking:     device int32[sum n] local indices in rank order, or NULL
 *  sel:         device int32[sum k] the first k of each ranking, ascending
 *  comp:        device int32[sum (n-k)] the rest, ascending, or NULL
 *  k_per_chunk: host int32[n_chunks], written before the call returns.
 * cachetune_select_topr_counts gives the same k_per_chunk without device work
 * (to size sel and comp before the call). */
ct_status cachetune_select_topr_counts(const int32_t* n_per_chunk, int32_t n_chunks, int32_t r_num,
                                       int32_t r_den, int32_t* k_per_chunk);
ct_status cachetune_select_topr(ct_handle h, const float* score, const int32_t* n_per_chunk, int32_t n_chunks,
                                int32_t r_num, int32_t r_den, int32_t* ranking, int32_t* sel,
                                int32_t* comp, int32_t* k_per_chunk, hipStream_t stream);

/* ---- checking a device index array ------------------------------------------
 * The selection (sel, comp, ranking), assembly and attention (q_pos) calls
 * trust their device index arrays (survey convention: trusted in release
 * builds).  This call checks one such array without trusting it, in place of
 * a device-side trap (which would take the whole device down): idx[0..count)
 * (device) must lie in [0, bound) and, with ascending != 0, each entry must
 * be above its predecessor.  *bad (device, one int32) receives the number of
 * entries that break a rule.  The array is only read; none of its values is
 * used as an address.  Enqueues two small kernels on stream (the first sets
 * *bad to 0) and returns; read *bad after the stream.  count may be 0.
 * CT_E_INVALID: bad NULL, count or bound negative, idx NULL with count > 0. */
ct_status cachetune_check_indices(const int32_t* idx, int32_t count, int32_t bound, int32_t ascending,
                                  int32_t* bad, hipStream_t stream);

/* ---- assembly with deferred RoPE (App. B.2, B.3) ---------------------------
 * Builds one layer's working buffer k_out/v_out [T][H][D] (device):
 *   reused rows: V copied, K rotated at the row's global position;
 *   recomputed rows: from k_rec/v_rec, K rotated at the global position;
 *   n_sfx uncached rows (k_sfx/v_sfx [n_sfx][H][D] pre-RoPE, device) at
 *   positions sfx_offset .. sfx_offset + n_sfx - 1, K rotated likewise.
 * Rows of k_out/v_out not covered by any place or the suffix are left as they
 * are.  Every written row must lie in [0, T).  places: host array.
 * The rotation angle pos * theta^(-2j/D) and its sine and cosine are formed in
 * fp64; the rotated value is rounded once to the storage type.
 * D must be 64 or 128; device index arrays are trusted (not range-checked). */
ct_status cachetune_assemble_rope(ct_handle h, const ct_place* places, int32_t n_places, const void* k_sfx,
                                  const void* v_sfx, int32_t n_sfx, int32_t sfx_offset, int32_t H,
                                  int32_t D, ct_dtype dtype, double rope_theta, ct_rope style,
                                  void* k_out, void* v_out, int32_t T, hipStream_t stream);

/* ---- selected-query causal attention (Sec. 4.1, App. B.2) ------------------
 *  q_pre: device [n_q][Hq][D] pre-RoPE queries of the selected and uncached rows
 *  q_pos: device int32[n_q] their global positions, each in [0, T); any order
 *         (ascending order keeps the causal work of neighbouring rows alike)
 *  k, v:  device [T][H][D] assembled layer (keys already rotated)
 * Query head h uses KV head floor(h * H / Hq) (Hq % H == 0).  Each query is
 * rotated to its position and stored rounded once to the storage type, like a
 * rotated key (App. B.3: the angle, its sine and cosine and the rotation in
 * fp64), then attends to keys at positions <= its own:
 *   out = softmax(softmax_scale * q . k_t) . v_t,   softmax_scale > 0
 * Arithmetic: fp32 accumulation on the matrix cores.  bf16 storage: the stored
 * bf16 query against the bf16 keys (exact products); the scale is applied to
 * the fp32 logits in the exponent; probabilities and V as fp16 (V exact while
 * |v| < 65536; otherwise that 64-key block takes V as bf16 and the
 * probabilities as a bf16 pair).  fp32 storage: query, probabilities, K and V
 * all enter as bf16 pairs.
 *  out: device [n_q][Hq][D] in `dtype`
 *  lse: device float[n_q][Hq] natural-log sum of exp of the scaled logits, or NULL.
 *  ws/ws_bytes: device workspace of at least cachetune_recompute_attn_ws bytes
 *         (may be NULL when that size is 0), 256-byte aligned; for bf16 it
 *         holds the rotated bf16 queries, V as fp16 tiles, and the
 *         partial results of rows whose keys are split over several segments
 *         (fp16, or fp32 for a segment whose V exceeds the fp16 range).
 * D must be 64 or 128; n_q >= 0; T >= 1; a softmax_scale that is not positive
 * and finite is CT_E_INVALID. */
ct_status cachetune_recompute_attn(ct_handle h, const void* q_pre, const int32_t* q_pos, int32_t n_q,
                                   int32_t Hq, const void* k, const void* v, int32_t T,
                                   int32_t H, int32_t D, ct_dtype dtype, float softmax_scale,
                                   double rope_theta, ct_rope style, void* out, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace query for cachetune_recompute_attn with these shapes on the
 * handle's device, or the current device for a NULL handle (the size depends
 * on the device's compute-unit count). */
ct_status cachetune_recompute_attn_ws(ct_handle h, int32_t n_q, int32_t Hq, int32_t T, int32_t H, int32_t D,
                                      ct_dtype dtype, size_t* bytes);

/* ---- selected-query attention for callers that cannot allocate -------------
 * For code that may not call hipMalloc (work captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation): cachetune_recompute_attn
 * with the same arguments and results, whose workspace is a fixed array of
 * 256 MiB (268435456 bytes) inside the library instead of a caller's buffer.
 * Each device the library runs on holds its own copy of that array until the
 * process ends; the call allocates nothing.  Shapes whose workspace
 * (cachetune_recompute_attn_ws) exceeds 256 MiB are refused with
 * CT_E_WORKSPACE (the 8 x 2048-token Llama-3-8B-shaped request needs about
 * 235 MiB).  All calls on one device share the array, so calls that overlap
 * in time on one device (other streams, other threads) race: order them on
 * one stream or with events.  Errors otherwise as cachetune_recompute_attn. */
ct_status cachetune_recompute_attn_noalloc(ct_handle h, const void* q_pre, const int32_t* q_pos, int32_t n_q,
                                           int32_t Hq, const void* k, const void* v, int32_t T,
                                           int32_t H, int32_t D, ct_dtype dtype, float softmax_scale,
                                           double rope_theta, ct_rope style, void* out, float* lse,
                                           hipStream_t stream);

/* ---- host-tier sparse loading (App. B.1 stored ranking, App. B.2) ----------
 * Offline, when a chunk's cache is generated, its rows are stored in rank
 * order, so that for any r the reuse complement of a (chunk, layer) is the
 * contiguous tail [k, n) of that layer and loads with one copy.
 *
 * cachetune_rank_order: k_dst[l][j] = k_src[l][ranking[j]] (and likewise V)
 * for every layer l < L and row j < n.  k_src, v_src, k_dst, v_dst: device
 * [L][n][H][D], 16-byte aligned, destinations distinct from sources;
 * ranking: device int32[n] (a permutation of [0, n), as written by
 * cachetune_select_topr); trusted, not range-checked. */
ct_status cachetune_rank_order(const void* k_src, const void* v_src, const int32_t* ranking,
                               int32_t n, int32_t L, int32_t H, int32_t D, ct_dtype dtype,
                               void* k_dst, void* v_dst, hipStream_t stream);

/* One chunk of the host pool: K and V [L][n][H][D] in rank order (host memory;
 * pinned with hipHostMalloc for the copies to run asynchronously). */
typedef struct {
  const void* k;
  const void* v;
  int32_t n;
  int32_t L;
} ct_ranked_chunk;

/* Copies the reuse complement of layer `layer` of every chunk -- rank-ordered
 * rows [k_per_chunk[b], n_b) -- from the host pool into the device staging
 * buffers k_stage / v_stage, packed: chunk b's rows start at row
 * sum_{b' < b} (n_b' - k_b').  Two hipMemcpyAsync per chunk are enqueued on
 * `stream` (for the staged rows, row j of chunk b holds local row
 * ranking_b[k_b + j]: pass that tail of the ranking as ct_place.src_rows).
 * k_per_chunk: host int32[n_chunks]. */
ct_status cachetune_stage_complement(const ct_ranked_chunk* chunks, int32_t n_chunks, int32_t layer,
                                     int32_t H, int32_t D, ct_dtype dtype,
                                     const int32_t* k_per_chunk, void* k_stage, void* v_stage,
                                     hipStream_t stream);

/* ---- kernel timing (tracing aid) -----------------------------------------
 * While enabled, each kernel launch of the library is bracketed by a pair of
 * HIP events on the launch's stream, recorded under the kernel's name:
 *   "band", "band_redo", "gram", "topr", "assemble", "attention_setup", "attention",
 *   "attention_merge", "rank_order", "energy_l2", "highpass", "bin_energy",
 *   "rmsnorm", "silu_mul", "linear" (and "twiddle", "layer_norm", "layer_mean").
 * cachetune_timing_read waits for the events recorded under `kernel`, returns
 * their summed duration in milliseconds and the number of launches, and
 * forgets them.  Events of other names are kept.  Thread-safe; the events are
 * small host objects (no device memory is allocated). */
ct_status cachetune_timing_enable(int32_t on);
ct_status cachetune_timing_read(const char* kernel, double* total_ms, int32_t* launches);

/* ---- hardware-aware recomputation ratio -----------------------------------
 * App. C.1 (cost model) and App. C.2 (warm-started golden-section search):
 * host logic over a caller-supplied cost measurement; no device work.
 *
 * Warm start: r0 = t_i / (t_c + t_i), clamped to [r_min, r_max] -- the ratio at
 * which a layer's recomputation of r*N tokens (t_c per token) and its loading
 * of the other (1 - r)*N (t_i per token) take equal time.
 * Search: on [a, b] = [max(r_min, r0 - half_width), min(r_max, r0 + half_width)],
 * golden-section steps with phi = (sqrt(5) - 1)/2: probes x1 = b - phi(b - a)
 * and x2 = a + phi(b - a); the side with the lower cost is kept (ties keep
 * [a, x2]) and its inner probe is reused, so each step makes one new call.
 * When b - a < eps the midpoint of [a, b] is returned.
 *  t_c, t_i: per-token costs (any common unit, >= 0, not both 0).
 *  cost: host callback, cost(r, user) = the measured objective at ratio r
 *        (e.g. mean time to first token over a calibration set); it is called
 *        2 + (number of steps) times, in order, on the calling thread.
 *  r_out: host double, the calibrated ratio.  n_probes: host int32 (or NULL),
 *        the number of cost calls made.
 * Errors: CT_E_INVALID for a negative or non-finite t_c or t_i, both zero,
 * r_min > r_max, a range outside [0, 1], half_width <= 0, eps <= 0, a NULL
 * callback or output, or a cost that is not finite (the search stops there). */
typedef double (*ct_cost_fn)(double r, void* user);

/* The App. C.1 cost model fitted to measured request times (host logic):
 * per layer the pipeline overlaps recomputing r*N tokens (t_c each) with
 * loading the other (1 - r)*N (t_i each), plus a fixed per-layer overhead t_o
 * (kernel launches, event waits, buffer management):
 *   T(r) = L * (t_o + max(r*N*t_c, (1 - r)*N*t_i)).
 * The probes (r[i], t[i]), i < n, are split by ratio into a loading-bound lower
 * part and a recomputation-bound upper part of at least two probes each (one
 * probe would fit any slope); every split is a
 * linear least-squares problem in (t_o, t_c, t_i).  A split counts when
 * t_c, t_i > 0, t_o >= 0 and each probe lies on its side of the balance ratio
 * t_i / (t_c + t_i); the smallest squared residual wins (the lower split on a
 * tie).  t_o shifts every ratio's time alike, so the warm start of
 * cachetune_calibrate_ratio, t_i / (t_c + t_i), does not depend on it.
 *  r, t: host double[n], n in [4, 1024]; r in [0, 1]; t finite (any unit)
 *  L, N: layers and reusable tokens of the measured request
 *  t_c, t_i, t_o: host outputs, per token and layer (t_o per layer), in the
 *        unit of t.
 * CT_E_INVALID for bad arguments or probes that show no loading-bound and
 * recomputation-bound parts. */
ct_status cachetune_fit_cost_model(const double* r, const double* t, int32_t n, int32_t L, int32_t N,
                                   double* t_c, double* t_i, double* t_o);
ct_status cachetune_calibrate_ratio(double t_c, double t_i, double r_min, double r_max,
                                    double half_width, double eps, ct_cost_fn cost, void* user,
                                    double* r_out, int32_t* n_probes);

#ifdef __cplusplus
}
#endif

#endif /* CACHETUNE_H */

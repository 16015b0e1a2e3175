"""Python binding of ``libcachetune.so`` (MI355X / gfx950 CacheTune hot path).

The functions carry the C ABI names (see ``include/cachetune.h`` for the
operation, layouts and error behaviour of each).  This module only marshals
arguments: torch tensors supply device memory and the current HIP stream; all
computation runs in the library's HIP kernels.  If the library is missing the
import of a function raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcachetune.so")

CT_OK, CT_E_INVALID, CT_E_UNSUPPORTED, CT_E_WORKSPACE, CT_E_HIP = 0, -1, -2, -3, -4
CT_F32, CT_BF16 = 0, 1
CT_NORM_SUM, CT_NORM_MAX, CT_NORM_MINMAX, CT_NORM_NONE = 0, 1, 2, 3
CT_ROPE_HALF, CT_ROPE_INTERLEAVED = 0, 1
CT_FFT_EXACT_N, CT_FFT_ZEROPAD_POW2 = 0, 1
CT_SCORE_LOWPASS, CT_SCORE_L2, CT_SCORE_HIGHPASS = 0, 1, 2


class ct_chunk(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n", C.c_int32)]


class ct_place(C.Structure):
    _fields_ = [("k_src", C.c_void_p), ("v_src", C.c_void_p), ("src_rows", C.c_void_p),
                ("k_rec", C.c_void_p), ("v_rec", C.c_void_p), ("sel", C.c_void_p),
                ("comp", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32), ("offset", C.c_int32)]


class ct_ranked_chunk(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n", C.c_int32), ("L", C.c_int32)]


class CacheTuneError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


SYMBOLS = ["cachetune_status_string", "cachetune_last_error", "cachetune_version",
           "cachetune_score_chunk_ws", "cachetune_score_chunk", "cachetune_select_topr",
           "cachetune_assemble_rope", "cachetune_recompute_attn", "cachetune_recompute_attn_ws",
           "cachetune_timing_enable", "cachetune_timing_read", "cachetune_rank_order",
           "cachetune_stage_complement", "cachetune_calibrate_ratio", "cachetune_score_variant_ws",
           "cachetune_score_variant", "cachetune_band_energy_ws", "cachetune_band_energy",
           "cachetune_rmsnorm", "cachetune_silu_mul", "cachetune_linear", "cachetune_qkv_proj",
           "cachetune_recompute_attn_noalloc", "cachetune_create", "cachetune_destroy",
           "cachetune_prepare_scoring", "cachetune_select_topr_counts", "cachetune_fit_cost_model",
           "cachetune_check_indices"]

# cost(r, user) -> double, the callback type of cachetune_calibrate_ratio
COST_FN = C.CFUNCTYPE(C.c_double, C.c_double, C.c_void_p)

_lib = None


def lib():
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with non_prefix_kv_token_amd.build")
        L = C.CDLL(LIB_PATH)
        i32, vp, f64, f32, sz = C.c_int32, C.c_void_p, C.c_double, C.c_float, C.c_size_t
        L.cachetune_status_string.argtypes = [i32]
        L.cachetune_status_string.restype = C.c_char_p
        L.cachetune_last_error.restype = C.c_char_p
        L.cachetune_version.restype = i32
        L.cachetune_create.argtypes = [i32, C.POINTER(vp)]
        L.cachetune_destroy.argtypes = [vp]
        L.cachetune_destroy.restype = None
        L.cachetune_prepare_scoring.argtypes = [vp, vp, i32, i32, i32, i32, vp]
        L.cachetune_score_chunk_ws.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, C.POINTER(sz)]
        L.cachetune_score_chunk.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                                            vp, sz, vp]
        L.cachetune_select_topr_counts.argtypes = [vp, i32, i32, i32, vp]
        L.cachetune_check_indices.argtypes = [vp, i32, i32, i32, vp, vp]
        L.cachetune_select_topr.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.cachetune_assemble_rope.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, f64, i32,
                                              vp, vp, i32, vp]
        L.cachetune_recompute_attn.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, f32,
                                               f64, i32, vp, vp, vp, sz, vp]
        L.cachetune_recompute_attn_ws.argtypes = [vp, i32, i32, i32, i32, i32, i32, C.POINTER(sz)]
        L.cachetune_recompute_attn_noalloc.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, f32,
                                                       f64, i32, vp, vp, vp]
        L.cachetune_timing_enable.argtypes = [i32]
        L.cachetune_rank_order.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
        L.cachetune_stage_complement.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        L.cachetune_timing_read.argtypes = [C.c_char_p, C.POINTER(f64), C.POINTER(i32)]
        L.cachetune_calibrate_ratio.argtypes = [f64, f64, f64, f64, f64, f64, COST_FN, vp,
                                                C.POINTER(f64), C.POINTER(i32)]
        L.cachetune_score_variant_ws.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                                 C.POINTER(sz)]
        L.cachetune_score_variant.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                              vp, vp, vp, sz, vp]
        L.cachetune_band_energy_ws.argtypes = [vp, i32, i32, i32, i32, i32, C.POINTER(sz)]
        L.cachetune_band_energy.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        L.cachetune_fit_cost_model.argtypes = [vp, vp, i32, i32, i32, C.POINTER(f64), C.POINTER(f64),
                                                C.POINTER(f64)]
        L.cachetune_rmsnorm.argtypes = [vp, vp, i32, i32, f32, i32, vp, vp]
        L.cachetune_silu_mul.argtypes = [vp, i32, i32, i32, vp, vp]
        L.cachetune_linear.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
        L.cachetune_qkv_proj.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        for name in SYMBOLS[3:]:
            if name != "cachetune_destroy":
                getattr(L, name).restype = i32
        _lib = L
    return _lib


_handles = {}


def handle(device=None):
    """The binding's context handle (cachetune_create) for `device` (the
    current device by default), created on first use and kept for the
    process; calls of this module pass it.  Without a GPU (argument checks
    only) the handle is NULL."""
    import torch
    if not torch.cuda.is_available():
        return None
    dev = torch.cuda.current_device() if device is None else int(device)
    if dev not in _handles:
        h = C.c_void_p()
        _check(lib().cachetune_create(dev, C.byref(h)))
        _handles[dev] = h
    return _handles[dev]


def cachetune_prepare_scoring(n_per_chunk, alpha=(1, 16), fftlen=CT_FFT_EXACT_N, stream=None):
    """Build the handle's scoring tables for these chunk lengths (allocates;
    synchronises the stream), so that later score calls allocate and rebuild
    nothing."""
    arr = _i32_array(n_per_chunk)
    _check(lib().cachetune_prepare_scoring(handle(), arr, len(n_per_chunk), alpha[0], alpha[1], fftlen,
                                           _stream(stream)))


def _check(status: int):
    if status != CT_OK:
        raise CacheTuneError(status, lib().cachetune_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CT_BF16
    if t.dtype == torch.float32:
        return CT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _i32_array(vals):
    arr = (C.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


# ---- scoring -----------------------------------------------------------------

def cachetune_score_chunk_ws(n_per_chunk, L, H, D, alpha=(1, 16), fftlen=CT_FFT_EXACT_N,
                             variant=CT_SCORE_LOWPASS) -> int:
    arr = _i32_array(n_per_chunk)
    out = C.c_size_t(0)
    _check(lib().cachetune_score_variant_ws(handle(), arr, len(n_per_chunk), L, H, D, alpha[0], alpha[1],
                                            fftlen, variant, C.byref(out)))
    return out.value


def cachetune_score_chunk(chunks, L, H, D, alpha=(1, 16), fftlen=CT_FFT_EXACT_N, norm=CT_NORM_SUM,
                          score=None, layer_score=None, ws=None, want_layers=False, stream=None,
                          variant=CT_SCORE_LOWPASS):
    """chunks: list of (K, V) device tensors [L][n][H][D].  Returns (score,
    layer_score) fp32 device tensors (layer_score None unless requested).
    variant: CT_SCORE_LOWPASS (the method), CT_SCORE_L2 (magnitudes without
    the frequency analysis) or CT_SCORE_HIGHPASS (magnitudes of the bins at
    and above the cutoff); the last two go through cachetune_score_variant."""
    import torch
    dev = chunks[0][0].device
    ns = [int(k.shape[1]) for k, _ in chunks]
    total = sum(ns)
    if score is None:
        score = torch.empty(total, dtype=torch.float32, device=dev)
    if want_layers and layer_score is None:
        layer_score = torch.empty((L, total), dtype=torch.float32, device=dev)
    need = cachetune_score_chunk_ws(ns, L, H, D, alpha, fftlen, variant)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    arr = (ct_chunk * len(chunks))()
    for i, (k, v) in enumerate(chunks):
        arr[i].k, arr[i].v, arr[i].n = k.data_ptr(), v.data_ptr(), int(k.shape[1])
    if variant == CT_SCORE_LOWPASS:
        _check(lib().cachetune_score_chunk(handle(), arr, len(chunks), L, H, D, _dtype(chunks[0][0]), alpha[0],
                                           alpha[1], fftlen, norm, _ptr(score), _ptr(layer_score),
                                           _ptr(ws), ws.numel(), _stream(stream)))
    else:
        _check(lib().cachetune_score_variant(handle(), arr, len(chunks), L, H, D, _dtype(chunks[0][0]), alpha[0],
                                             alpha[1], fftlen, norm, variant, _ptr(score),
                                             _ptr(layer_score), _ptr(ws), ws.numel(), _stream(stream)))
    return score, layer_score


def cachetune_band_energy_ws(n_per_chunk, L, H, D, fftlen=CT_FFT_EXACT_N) -> int:
    arr = _i32_array(n_per_chunk)
    out = C.c_size_t(0)
    _check(lib().cachetune_band_energy_ws(arr, len(n_per_chunk), L, H, D, fftlen, C.byref(out)))
    return out.value


def cachetune_band_energy(chunks, L, H, D, n_bands, fftlen=CT_FFT_EXACT_N, ws=None, stream=None):
    """App. E.1 band energy fractions.  chunks: list of (K, V) device tensors
    [L][n][H][D].  Returns (fraction [n_chunks][L][2][n_bands], total
    [n_chunks][L][2]) float64 device tensors."""
    import torch
    dev = chunks[0][0].device
    ns = [int(k.shape[1]) for k, _ in chunks]
    need = cachetune_band_energy_ws(ns, L, H, D, fftlen)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    fraction = torch.empty((len(chunks), L, 2, n_bands), dtype=torch.float64, device=dev)
    total = torch.empty((len(chunks), L, 2), dtype=torch.float64, device=dev)
    arr = (ct_chunk * len(chunks))()
    for i, (k, v) in enumerate(chunks):
        arr[i].k, arr[i].v, arr[i].n = k.data_ptr(), v.data_ptr(), int(k.shape[1])
    _check(lib().cachetune_band_energy(arr, len(chunks), L, H, D, _dtype(chunks[0][0]), fftlen, n_bands,
                                       _ptr(fraction), _ptr(total), _ptr(ws), ws.numel(),
                                       _stream(stream)))
    return fraction, total


# ---- the rest of the selective-recompute layer --------------------------------------

def cachetune_rmsnorm(x, gain, eps=1e-5, out=None, stream=None):
    """x: [rows][dim] bf16 device tensor; gain [dim].  Returns out (bf16)."""
    import torch
    out = torch.empty_like(x) if out is None else out
    rows, dim = int(x.shape[0]), int(x.shape[-1])
    _check(lib().cachetune_rmsnorm(_ptr(x), _ptr(gain), rows, dim, float(eps), _dtype(x), _ptr(out),
                                   _stream(stream)))
    return out


def cachetune_silu_mul(gate_up, out=None, stream=None):
    """gate_up: [rows][2 ff] bf16.  Returns silu(gate) * up, [rows][ff]."""
    import torch
    rows, ff = int(gate_up.shape[0]), int(gate_up.shape[1]) // 2
    if out is None:
        out = torch.empty((rows, ff), dtype=gate_up.dtype, device=gate_up.device)
    _check(lib().cachetune_silu_mul(_ptr(gate_up), rows, ff, _dtype(gate_up), _ptr(out), _stream(stream)))
    return out


def cachetune_linear(x, w, residual=None, out=None, stream=None):
    """x: [m][k], w: [n][k] bf16 device tensors; residual [m][n] or None.
    Returns x w^T (+ residual) as [m][n] bf16."""
    import torch
    m, k = int(x.shape[0]), int(x.shape[1])
    n = int(w.shape[0])
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    _check(lib().cachetune_linear(_ptr(x), _ptr(w), _ptr(residual), m, n, k, _dtype(x), _ptr(out),
                                  _stream(stream)))
    return out


def cachetune_qkv_proj(x, w_qkv, nq, nkv, q=None, k=None, v=None, stream=None):
    """x: [m][d]; w_qkv: [nq + 2 nkv][d] (wq, wk, wv stacked).  Returns the
    q [m][nq], k [m][nkv], v [m][nkv] bf16 tensors."""
    import torch
    m, d = int(x.shape[0]), int(x.shape[1])
    mk = lambda n: torch.empty((m, n), dtype=x.dtype, device=x.device)  # noqa: E731
    q = mk(nq) if q is None else q
    k = mk(nkv) if k is None else k
    v = mk(nkv) if v is None else v
    _check(lib().cachetune_qkv_proj(_ptr(x), _ptr(w_qkv), m, d, nq, nkv, _dtype(x), _ptr(q), _ptr(k), _ptr(v),
                                    _stream(stream)))
    return q, k, v


# ---- selection ----------------------------------------------------------------

def cachetune_select_topr(score, n_per_chunk, r=(15, 100), ranking=None, sel=None, comp=None,
                          want_ranking=True, want_comp=True, stream=None):
    """Returns (k_per_chunk list, ranking, sel, comp) with device int32 tensors."""
    import torch
    dev = score.device
    ns = [int(n) for n in n_per_chunk]
    arr = _i32_array(ns)
    kq = (C.c_int32 * len(ns))()
    _check(lib().cachetune_select_topr_counts(arr, len(ns), r[0], r[1], kq))
    ks = list(kq)
    if ranking is None and want_ranking:
        ranking = torch.empty(sum(ns), dtype=torch.int32, device=dev)
    if sel is None:
        sel = torch.empty(max(1, sum(ks)), dtype=torch.int32, device=dev)
    if comp is None and want_comp:
        comp = torch.empty(max(1, sum(ns) - sum(ks)), dtype=torch.int32, device=dev)
    kout = (C.c_int32 * len(ns))()
    _check(lib().cachetune_select_topr(handle(), _ptr(score), arr, len(ns), r[0], r[1], _ptr(ranking),
                                       _ptr(sel), _ptr(comp), kout, _stream(stream)))
    return list(kout), ranking, sel, comp


# ---- checking device index arrays ---------------------------------------------

def cachetune_check_indices(idx, bound, ascending=True, stream=None) -> int:
    """Number of entries of the device int32 array idx outside [0, bound) or
    (ascending) not above their predecessor; waits for the stream."""
    import torch
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 device tensor")
    bad = torch.empty(1, dtype=torch.int32, device=idx.device)
    stream = torch.cuda.current_stream() if stream is None else stream
    _check(lib().cachetune_check_indices(_ptr(idx), idx.numel(), bound, int(bool(ascending)), _ptr(bad),
                                         _stream(stream)))
    stream.synchronize()
    return int(bad.item())


# ---- assembly -----------------------------------------------------------------

def make_place(k_src, v_src, n, k, offset, sel=None, comp=None, k_rec=None, v_rec=None,
               src_rows=None) -> ct_place:
    p = ct_place()
    p.k_src = None if k_src is None else k_src.data_ptr()
    p.v_src = None if v_src is None else v_src.data_ptr()
    p.src_rows = None if src_rows is None else src_rows.data_ptr()
    p.k_rec = None if k_rec is None else k_rec.data_ptr()
    p.v_rec = None if v_rec is None else v_rec.data_ptr()
    p.sel = None if sel is None else sel.data_ptr()
    p.comp = None if comp is None else comp.data_ptr()
    p.n, p.k, p.offset = int(n), int(k), int(offset)
    return p


def cachetune_assemble_rope(places, k_out, v_out, H, D, rope_theta, style=CT_ROPE_HALF,
                            k_sfx=None, v_sfx=None, n_sfx=0, sfx_offset=0, stream=None):
    arr = (ct_place * max(1, len(places)))(*places)
    T = int(k_out.shape[0])
    _check(lib().cachetune_assemble_rope(handle(), arr, len(places), _ptr(k_sfx), _ptr(v_sfx), n_sfx,
                                         sfx_offset, H, D, _dtype(k_out), rope_theta, style,
                                         _ptr(k_out), _ptr(v_out), T, _stream(stream)))


# ---- attention ----------------------------------------------------------------

def cachetune_recompute_attn_ws(n_q, Hq, T, H, D, dtype=CT_BF16) -> int:
    out = C.c_size_t(0)
    _check(lib().cachetune_recompute_attn_ws(handle(), n_q, Hq, T, H, D, dtype, C.byref(out)))
    return out.value


def cachetune_recompute_attn(q_pre, q_pos, k, v, softmax_scale, rope_theta, style=CT_ROPE_HALF,
                             out=None, lse=None, want_lse=False, ws=None, stream=None):
    """q_pre [n_q][Hq][D], q_pos int32 [n_q], k/v [T][H][D]; returns (out, lse).
    ws: optional uint8 device tensor, allocated here when missing or too small."""
    import torch
    n_q, Hq, D = (int(x) for x in q_pre.shape)
    T, H = int(k.shape[0]), int(k.shape[1])
    if out is None:
        out = torch.empty_like(q_pre)
    if want_lse and lse is None:
        lse = torch.empty((n_q, Hq), dtype=torch.float32, device=q_pre.device)
    dt = _dtype(q_pre)
    need = cachetune_recompute_attn_ws(n_q, Hq, T, H, D, dt)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=q_pre.device)
    _check(lib().cachetune_recompute_attn(handle(), _ptr(q_pre), _ptr(q_pos), n_q, Hq, _ptr(k), _ptr(v), T,
                                          H, D, dt, float(softmax_scale), float(rope_theta), style,
                                          _ptr(out), _ptr(lse), _ptr(ws) if need else None,
                                          ws.numel() if need else 0, _stream(stream)))
    return out, lse


def cachetune_recompute_attn_noalloc(q_pre, q_pos, k, v, softmax_scale, rope_theta, out, style=CT_ROPE_HALF,
                                     lse=None, stream=None):
    """cachetune_recompute_attn with the library's own per-device scratch as the
    workspace (the call allocates nothing).  `out` ([n_q][Hq][D]) and `lse`
    ([n_q][Hq] fp32 or None) are caller-owned device tensors."""
    n_q, Hq, D = (int(x) for x in q_pre.shape)
    T, H = int(k.shape[0]), int(k.shape[1])
    _check(lib().cachetune_recompute_attn_noalloc(handle(), _ptr(q_pre), _ptr(q_pos), n_q, Hq, _ptr(k), _ptr(v), T, H, D,
                                                  _dtype(q_pre), float(softmax_scale), float(rope_theta), style,
                                                  _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


# ---- kernel timing ---------------------------------------------------------------

def cachetune_timing_enable(on: bool = True):
    _check(lib().cachetune_timing_enable(1 if on else 0))


def cachetune_calibrate_ratio(t_c, t_i, cost, r_min=0.15, r_max=1.0, half_width=0.1, eps=0.01):
    """Warm-started golden-section search for the recomputation ratio (host
    logic in the library).  cost(r) -> float is called for each probe, in
    order; returns (r, number of probes).  An exception raised by `cost` stops
    the search and is re-raised here."""
    err = []

    def cb(r, _user):
        try:
            return float(cost(r))
        except BaseException as e:  # handed back after the library returns
            err.append(e)
            return float("nan")

    fn = COST_FN(cb)
    r_out = C.c_double(0.0)
    n = C.c_int32(0)
    st = lib().cachetune_calibrate_ratio(float(t_c), float(t_i), float(r_min), float(r_max),
                                         float(half_width), float(eps), fn, None, C.byref(r_out),
                                         C.byref(n))
    if err:
        raise err[0]
    _check(st)
    return r_out.value, n.value


def cachetune_fit_cost_model(r, times, L, N):
    """App. C.1 cost model from measured request times: returns (t_c, t_i,
    t_o) in the unit of `times` (per token and layer; t_o per layer)."""
    n = len(r)
    ra = (C.c_double * n)(*[float(x) for x in r])
    ta = (C.c_double * n)(*[float(x) for x in times])
    tc, ti, to = C.c_double(0.0), C.c_double(0.0), C.c_double(0.0)
    _check(lib().cachetune_fit_cost_model(ra, ta, n, int(L), int(N), C.byref(tc), C.byref(ti), C.byref(to)))
    return tc.value, ti.value, to.value


def cachetune_timing_read(kernel: str):
    """(total milliseconds, launches) recorded under `kernel` since the last read."""
    ms = C.c_double(0.0)
    n = C.c_int32(0)
    _check(lib().cachetune_timing_read(kernel.encode(), C.byref(ms), C.byref(n)))
    return ms.value, n.value


# ---- host tier ---------------------------------------------------------------------

def cachetune_rank_order(k_src, v_src, ranking, k_dst=None, v_dst=None, stream=None):
    """k_src/v_src [L][n][H][D] device, ranking int32[n] device; returns the
    rank-ordered copies (device)."""
    import torch
    L, n, H, D = (int(x) for x in k_src.shape)
    if k_dst is None:
        k_dst = torch.empty_like(k_src)
    if v_dst is None:
        v_dst = torch.empty_like(v_src)
    _check(lib().cachetune_rank_order(_ptr(k_src), _ptr(v_src), _ptr(ranking), n, L, H, D,
                                      _dtype(k_src), _ptr(k_dst), _ptr(v_dst), _stream(stream)))
    return k_dst, v_dst


def cachetune_stage_complement(chunks, layer, k_per_chunk, k_stage, v_stage, stream=None):
    """chunks: list of (K, V) rank-ordered host tensors [L][n][H][D] (pinned);
    copies the complement rows of `layer` into k_stage / v_stage (device)."""
    arr = (ct_ranked_chunk * len(chunks))()
    for i, (k, v) in enumerate(chunks):
        arr[i].k, arr[i].v = k.data_ptr(), v.data_ptr()
        arr[i].L, arr[i].n = int(k.shape[0]), int(k.shape[1])
    H, D = int(chunks[0][0].shape[2]), int(chunks[0][0].shape[3])
    ks = _i32_array(k_per_chunk)
    _check(lib().cachetune_stage_complement(arr, len(chunks), layer, H, D, _dtype(chunks[0][0]), ks,
                                            _ptr(k_stage), _ptr(v_stage), _stream(stream)))

"""Reference oracle for the CacheTune hot path -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper over ``oracle.c`` (plain fp64 C, direct DFT, sort-based
top-r, scalar RoPE, fp64 softmax attention).  Only the test-suite, the smoke
entry and the bench's CPU-baseline leg may import this package; the product
library never loads it and shares no code with it.

Storage convention shared with the product boundary: bf16 tensors are numpy
``uint16`` arrays of raw bit patterns, fp32 tensors are ``float32`` arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

F32, BF16 = 0, 1
FFT_EXACT_N, FFT_ZEROPAD_POW2 = 0, 1
NORM_SUM, NORM_MAX, NORM_MINMAX, NORM_NONE = 0, 1, 2, 3
ROPE_HALF, ROPE_INTERLEAVED = 0, 1

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared",
           SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        i32, f64, vp = C.c_int, C.c_double, C.c_void_p
        L.orc_nbins.argtypes = [i32]
        L.orc_kkeep.argtypes = [i32, i32, i32]
        L.orc_ksel.argtypes = [i32, i32, i32]
        L.orc_fft_len.argtypes = [i32, i32]
        L.orc_round_bf16.argtypes = [f64]
        L.orc_round_bf16.restype = C.c_uint16
        L.orc_rfft.argtypes = [vp, i32, vp, vp]
        L.orc_lowpass.argtypes = [vp, i32, i32, i32, i32, vp]
        L.orc_highpass.argtypes = [vp, i32, i32, i32, i32, vp]
        L.orc_round_bf16_array.argtypes = [vp, C.c_longlong, vp]
        L.orc_band_energy.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]
        L.orc_score_highpass.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
        L.orc_score_chunk.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
        L.orc_topr.argtypes = [vp, i32, i32, vp, vp, vp]
        L.orc_offsets.argtypes = [vp, vp, i32, i32, vp]
        L.orc_rope_freqs.argtypes = [i32, f64, vp]
        L.orc_rope.argtypes = [vp, i32, f64, f64, i32, vp]
        L.orc_assemble_chunk.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, i32, vp, vp]
        L.orc_assemble_rows.argtypes = [vp, vp, i32, i32, i32, i32, i32, f64, i32, vp, vp]
        L.orc_attention.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, f64, f64, i32, vp, i32, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"storage dtype must be float32 or uint16 (bf16 bits), got {a.dtype}")


def widen(a: np.ndarray) -> np.ndarray:
    """Exact value of stored data as float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---- sizes -------------------------------------------------------------

def nbins(n: int) -> int:
    return lib().orc_nbins(n)


def kkeep(nb: int, a_num: int, a_den: int) -> int:
    return lib().orc_kkeep(nb, a_num, a_den)


def ksel(n: int, r_num: int, r_den: int) -> int:
    return lib().orc_ksel(n, r_num, r_den)


def fft_len(n: int, mode: int = FFT_EXACT_N) -> int:
    return lib().orc_fft_len(n, mode)


def round_bf16(x) -> np.ndarray:
    """RNE rounding of float64 values to bf16 bit patterns (elementwise, slow)."""
    L = lib()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.array([L.orc_round_bf16(float(v)) for v in flat], dtype=np.uint16)
    return out.reshape(np.shape(x))


# ---- transforms ----------------------------------------------------------

def rfft(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[0]
    re = np.zeros(n // 2 + 1)
    im = np.zeros(n // 2 + 1)
    lib().orc_rfft(_p(x), n, _p(re), _p(im))
    return re + 1j * im


def lowpass(x: np.ndarray, a_num: int, a_den: int, mode: int = FFT_EXACT_N) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    lib().orc_lowpass(_p(x), x.shape[0], a_num, a_den, mode, _p(out))
    return out


def highpass(x: np.ndarray, a_num: int, a_den: int, mode: int = FFT_EXACT_N) -> np.ndarray:
    """High-frequency reconstruction: the bins at and above the low-pass cutoff."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    lib().orc_highpass(_p(x), x.shape[0], a_num, a_den, mode, _p(out))
    return out


# ---- scoring / selection ------------------------------------------------

def score_chunk(K: np.ndarray, V: np.ndarray, a_num: int, a_den: int,
                mode: int = FFT_EXACT_N, norm: int = NORM_SUM, layers: bool = False):
    """K, V: [L][N][H][D] storage arrays.  Returns score[N] (and [L][N])."""
    assert K.shape == V.shape and K.ndim == 4 and K.dtype == V.dtype
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    L_, N, H, D = K.shape
    score = np.zeros(N)
    ls = np.zeros((L_, N)) if layers else None
    rc = lib().orc_score_chunk(_p(K), _p(V), _dtype_code(K), L_, N, H, D, a_num, a_den,
                               mode, norm, _p(ls), _p(score))
    if rc != 0:
        raise ValueError("orc_score_chunk rejected its arguments")
    return (score, ls) if layers else score


def score_l2(K: np.ndarray, V: np.ndarray, norm: int = NORM_SUM, layers: bool = False):
    """§5.4 L2-norm selection score: joint K/V magnitudes of the stored rows,
    per-layer normalisation and layer mean, no frequency analysis."""
    assert K.shape == V.shape and K.ndim == 4 and K.dtype == V.dtype
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    L_, N, H, D = K.shape
    score = np.zeros(N)
    ls = np.zeros((L_, N)) if layers else None
    rc = lib().orc_score_l2(_p(K), _p(V), _dtype_code(K), L_, N, H, D, norm, _p(ls), _p(score))
    if rc != 0:
        raise ValueError("orc_score_l2 rejected its arguments")
    return (score, ls) if layers else score


def band_energy(X: np.ndarray, n_bands: int, mode: int = FFT_EXACT_N):
    """App. E.1 energy fractions of one tensor [L][N][H][D] over n_bands equal
    bands of its rFFT bins along the tokens (channels summed).  Returns
    (fraction [L][n_bands], total [L])."""
    assert X.ndim == 4
    X = np.ascontiguousarray(X)
    L_, N, H, D = X.shape
    fr = np.zeros((L_, n_bands))
    tot = np.zeros(L_)
    rc = lib().orc_band_energy(_p(X), _dtype_code(X), L_, N, H, D, mode, n_bands, _p(fr), _p(tot))
    if rc != 0:
        raise ValueError("orc_band_energy rejected its arguments")
    return fr, tot


def score_highpass(K: np.ndarray, V: np.ndarray, a_num: int, a_den: int,
                   mode: int = FFT_EXACT_N, norm: int = NORM_SUM, layers: bool = False):
    """Sec. 5.4 and App. E.2 (Table 3) high-frequency-guided selection score: the scoring of
    score_chunk applied to the high-frequency reconstruction (bins >= cutoff)."""
    assert K.shape == V.shape and K.ndim == 4 and K.dtype == V.dtype
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    L_, N, H, D = K.shape
    score = np.zeros(N)
    ls = np.zeros((L_, N)) if layers else None
    rc = lib().orc_score_highpass(_p(K), _p(V), _dtype_code(K), L_, N, H, D, a_num, a_den,
                                  mode, norm, _p(ls), _p(score))
    if rc != 0:
        raise ValueError("orc_score_highpass rejected its arguments")
    return (score, ls) if layers else score


def topr(score: np.ndarray, k: int):
    s = np.ascontiguousarray(score, dtype=np.float64)
    n = s.shape[0]
    ranking = np.zeros(n, np.int32)
    sel = np.zeros(max(k, 1), np.int32)
    comp = np.zeros(max(n - k, 1), np.int32)
    lib().orc_topr(_p(s), n, k, _p(ranking), _p(sel), _p(comp))
    return ranking, sel[:k].copy(), comp[:n - k].copy()


def offsets(n_per_chunk, order, prefix: int = 0) -> np.ndarray:
    n = np.ascontiguousarray(n_per_chunk, dtype=np.int32)
    o = np.ascontiguousarray(order, dtype=np.int32)
    out = np.zeros(n.shape[0], np.int32)
    lib().orc_offsets(_p(n), _p(o), n.shape[0], prefix, _p(out))
    return out


# ---- RoPE / assembly ----------------------------------------------------

def rope_freqs(D: int, theta: float) -> np.ndarray:
    f = np.zeros(D // 2)
    lib().orc_rope_freqs(D, theta, _p(f))
    return f


def rope(x: np.ndarray, pos: float, theta: float, style: int = ROPE_HALF) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.zeros_like(x)
    lib().orc_rope(_p(x), x.shape[0], float(pos), float(theta), style, _p(y))
    return y


def assemble_chunk(k_src, v_src, k_rec, v_rec, sel, offset, theta, style, k_out, v_out):
    """Place one chunk (rows [n][H][D]) into k_out/v_out ([T][H][D]) in place."""
    n, H, D = k_src.shape
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    k = sel.shape[0]
    kr = np.ascontiguousarray(k_rec) if k > 0 else np.zeros((1, H, D), k_src.dtype)
    vr = np.ascontiguousarray(v_rec) if k > 0 else np.zeros((1, H, D), k_src.dtype)
    lib().orc_assemble_chunk(_p(np.ascontiguousarray(k_src)), _p(np.ascontiguousarray(v_src)),
                             _p(kr), _p(vr), _p(sel if k > 0 else np.zeros(1, np.int32)), n, k,
                             int(offset), H, D, _dtype_code(k_src), float(theta), style,
                             _p(k_out), _p(v_out))


def assemble_rows(k_rows, v_rows, start, theta, style, k_out, v_out):
    n, H, D = k_rows.shape
    if n == 0:
        return
    lib().orc_assemble_rows(_p(np.ascontiguousarray(k_rows)), _p(np.ascontiguousarray(v_rows)),
                            n, int(start), H, D, _dtype_code(k_rows), float(theta), style,
                            _p(k_out), _p(v_out))


def attention(q_pre, qpos, k, v, scale, theta, style=ROPE_HALF, rows=None):
    """q_pre: [n_q][Hq][D]; k, v: [T][H][D] (assembled).  Returns (out, lse) in
    float64 for the requested rows (all rows by default)."""
    n_q, Hq, D = q_pre.shape
    T, H, _ = k.shape
    rows = np.arange(n_q, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    out = np.zeros((rows.shape[0], Hq, D))
    lse = np.zeros((rows.shape[0], Hq))
    qp = np.ascontiguousarray(qpos, dtype=np.int32)
    rc = lib().orc_attention(_p(np.ascontiguousarray(q_pre)), _p(qp), Hq, _p(np.ascontiguousarray(k)),
                             _p(np.ascontiguousarray(v)), T, H, D, _dtype_code(q_pre), float(scale),
                             float(theta), style, _p(rows), rows.shape[0], _p(out), _p(lse))
    if rc != 0:
        raise ValueError("orc_attention rejected its arguments")
    return out, lse


# ---- hardware-aware recomputation ratio (App. C.1, App. C.2) ----------------

def cost_model_time(r, t_c, t_i, t_o, L, N):
    """App. C.1 (reading): per layer the pipeline overlaps recomputing r*N
    tokens with loading the other (1 - r)*N, so the longer of the two sets the
    layer's time, plus the fixed per-layer overhead t_o; L layers."""
    r = np.asarray(r, dtype=np.float64)
    return L * (t_o + np.maximum(r * N * t_c, (1.0 - r) * N * t_i))


def fit_cost_model(r, times, L, N):
    """App. C.1: t_c, t_i and t_o from measured request times at several
    ratios.  Every split of the probes (sorted by r) into a lower part bounded
    by loading and an upper part bounded by recomputation, at least two probes
    each (a single probe fits any slope), is a linear least-squares problem in
    (t_o, t_c, t_i): lower probes satisfy
    T / L = t_o + (1 - r) N t_i, upper ones T / L = t_o + r N t_c.  A split
    counts when t_c, t_i > 0, t_o >= 0 and every probe lies on its side of the
    balance ratio t_i / (t_c + t_i); the one with the smallest squared
    residual of the model wins (the lower split on a tie).
    Returns (t_c, t_i, t_o), or None when no split counts."""
    r = np.asarray(r, dtype=np.float64)
    times = np.asarray(times, dtype=np.float64)
    order = np.argsort(r, kind="stable")
    r, times = r[order], times[order]
    n = len(r)
    best = None
    for k in range(2, n - 1):
        A = np.zeros((n, 3))
        A[:, 0] = 1.0
        A[k:, 1] = r[k:] * N
        A[:k, 2] = (1.0 - r[:k]) * N
        if np.linalg.matrix_rank(A) < 3:
            continue
        (t_o, t_c, t_i), *_ = np.linalg.lstsq(A, times / L, rcond=None)
        if not (t_c > 0 and t_i > 0 and t_o >= 0):
            continue
        rb = t_i / (t_c + t_i)
        if not (np.all(r[:k] <= rb) and np.all(r[k:] >= rb)):
            continue
        res = float(np.sum((times - cost_model_time(r, t_c, t_i, t_o, L, N)) ** 2))
        if best is None or res < best[0]:
            best = (res, float(t_c), float(t_i), float(t_o))
    return None if best is None else best[1:]


def warm_start_ratio(t_c: float, t_i: float, r_min: float, r_max: float) -> float:
    """App. C.1: per layer, recomputing r*N tokens costs r*N*t_c and loading the
    other (1 - r)*N costs (1 - r)*N*t_i; the two are equal at
    r = t_i / (t_c + t_i).  Clamped to the allowed range."""
    r = t_i / (t_c + t_i)
    return min(max(r, r_min), r_max)


def calibrate_ratio(t_c, t_i, cost, r_min=0.15, r_max=1.0, half_width=0.1, eps=0.01):
    """App. C.2, warm-started golden-section search, written out step by step.
    The interval around the warm start is [r0 - half_width, r0 + half_width]
    cut to [r_min, r_max].  Each step compares the costs at the two inner
    points x1 = b - phi (b - a) and x2 = a + phi (b - a), keeps the side with
    the lower cost (the lower side [a, x2] on a tie), and reuses the inner point
    that stays inside, so only one new cost is measured per step.  Once the
    width is below eps, the midpoint is the ratio.

    Returns (r, probes, widths): the probes in call order as (r, cost) pairs,
    and the interval width before each step and at the end."""
    phi = (5.0 ** 0.5 - 1.0) / 2.0
    r0 = warm_start_ratio(t_c, t_i, r_min, r_max)
    a, b = max(r_min, r0 - half_width), min(r_max, r0 + half_width)
    probes = []

    def f(r):
        v = float(cost(r))
        probes.append((r, v))
        return v

    x1, x2 = b - phi * (b - a), a + phi * (b - a)
    f1, f2 = f(x1), f(x2)
    widths = [b - a]
    while b - a >= eps:
        if f1 <= f2:
            b, x2, f2 = x2, x1, f1
            x1 = b - phi * (b - a)
            f1 = f(x1)
        else:
            a, x1, f1 = x1, x2, f2
            x2 = a + phi * (b - a)
            f2 = f(x2)
        widths.append(b - a)
    return 0.5 * (a + b), probes, widths


# ---- the rest of the selective-recompute layer (synthetic weights) ---------------
# The recomputed rows (Sec. 4.1, App. B.2: the selected tokens and the uncached
# suffix run through each layer in the new context) pass through a decoder layer
# of the models the pages evaluate (Sec. 5.1: Llama-3-8B and relatives): pre-norm
# RMSNorm, bias-free Q/K/V projections, RoPE at the global position and causal
# GQA attention over the assembled layer, output projection plus residual,
# RMSNorm, the gated MLP silu(gate) * up, down projection plus residual.  Plain
# fp64 definitions; numpy's matmul is the library primitive for the products.

def bf16_bits(x) -> np.ndarray:
    """Vectorised RNE rounding of float64 values to bf16 bit patterns."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().orc_round_bf16_array(_p(a), a.size, _p(out))
    return out


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * np.asarray(gain, np.float64)


def linear(x: np.ndarray, w: np.ndarray, residual: np.ndarray | None = None) -> np.ndarray:
    """x [m][k] times w [n][k] transposed (a bias-free projection), plus the
    residual [m][n] when given."""
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    return y if residual is None else y + np.asarray(residual, np.float64)


def silu_mul(gu: np.ndarray) -> np.ndarray:
    """gu [m][2f] holds gate (columns [0, f)) and up ([f, 2f)): silu(gate) * up
    with silu(g) = g / (1 + exp(-g))."""
    gu = np.asarray(gu, np.float64)
    f = gu.shape[-1] // 2
    g, u = gu[..., :f], gu[..., f:]
    return g / (1.0 + np.exp(-g)) * u


def recompute_layer(h, w, chunks, sel, offsets, sfx_start, qpos, H, Hq, D, theta, eps,
                    style=ROPE_HALF):
    """One layer for the n_q recomputed rows, in bf16 storage as the GPU path
    keeps it: every stored intermediate (normalised rows, q, k, v, attention
    output, h1, gate/up, MLP input, output) is rounded to bf16 where it is
    stored; arithmetic between stores is fp64.

    h: [n_q][d] float64 holding bf16 values, rows in qpos order (the selected
    rows of each chunk in placement order, then the suffix).  w: dict of float64
    arrays holding bf16 values: g1, g2 [d]; wq [Hq*D][d]; wk, wv [H*D][d];
    wo [d][Hq*D]; wgu [2f][d]; wd [d][f].  chunks: list of (K, V) cached
    [n][H][D] bf16 bit arrays of this layer; sel: per chunk the selected local
    indices (ascending); offsets: per chunk its global start; sfx_start: global
    position of the first suffix row.  Returns h2 [n_q][d] float64 (bf16 values)
    and the intermediates in a dict."""
    r = lambda a: widen(bf16_bits(a))  # noqa: E731  (stored as bf16)
    n_q = h.shape[0]
    x1 = r(rmsnorm(h, w["g1"], eps))
    q = r(linear(x1, w["wq"]))
    kr = r(linear(x1, w["wk"]))
    vr = r(linear(x1, w["wv"]))
    T = sfx_start + (n_q - sum(len(s) for s in sel))
    k_asm = np.zeros((T, H, D), np.uint16)
    v_asm = np.zeros((T, H, D), np.uint16)
    kb = bf16_bits(kr).reshape(n_q, H, D)
    vb = bf16_bits(vr).reshape(n_q, H, D)
    row = 0
    for (K, V), s, off in zip(chunks, sel, offsets):
        k = len(s)
        assemble_chunk(K, V, kb[row:row + k], vb[row:row + k], s, off, theta, style, k_asm, v_asm)
        row += k
    assemble_rows(kb[row:], vb[row:], sfx_start, theta, style, k_asm, v_asm)
    qb = bf16_bits(q).reshape(n_q, Hq, D)
    o, _ = attention(qb, qpos, k_asm, v_asm, 1.0 / np.sqrt(D), theta, style)
    o = r(o.reshape(n_q, Hq * D))
    h1 = r(linear(o, w["wo"], h))
    x2 = r(rmsnorm(h1, w["g2"], eps))
    gu = r(linear(x2, w["wgu"]))
    a = r(silu_mul(gu))
    h2 = r(linear(a, w["wd"], h1))
    return h2, dict(x1=x1, q=q, k=kr, v=vr, k_asm=k_asm, v_asm=v_asm, o=o, h1=h1, x2=x2, gu=gu, a=a)

"""GPU parity: every C-ABI call against the oracle on the same seeded inputs,
at sizes the oracle finishes in seconds (several tiles, ragged tails), plus
edge cases.  Tolerances: index sets bit-exact (outside a 1e-6 relative tie
band around the k-th score when the GPU ranks its own scores); fp32 scores
1e-4 relative; assembled V bit-exact and K within 1 ulp (>= 99.9% bit-exact);
attention outputs 2e-2 absolute for the computation, plus half an ulp of the
output's own storage rounding (a bf16 value in [16, 32) is only resolved to
0.0625)."""
import numpy as np
import pytest
import torch

from gpu_util import (LSE_TOL, assert_rotated_keys, check_index_sets, half_ulp_bf16, need_gpu, to_dev, to_host,
                      ulp_distance_bf16, ulp_distance_f32, widen)

pytestmark = pytest.mark.gpu

SEED = 20260600


def _chunks(syn, ns, L, H, D, dtype, seed=SEED):
    return [(syn.chunk(seed, syn.K, b, L, n, H, D, dtype), syn.chunk(seed, syn.V, b, L, n, H, D, dtype))
            for b, n in enumerate(ns)]


def _score_both(orc, syn, ns, L, H, D, dtype, alpha, mode=0, norm=0, edit=None):
    ct = need_gpu()
    host = _chunks(syn, ns, L, H, D, dtype)
    if edit is not None:
        edit(host)
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    s_gpu, ls_gpu = ct.cachetune_score_chunk(dev, L, H, D, alpha=alpha, fftlen=mode, norm=norm,
                                             want_layers=True)
    torch.cuda.synchronize()
    s_gpu, ls_gpu = to_host(s_gpu), to_host(ls_gpu)
    s_orc, ls_orc = [], []
    for k, v in host:
        s, ls = orc.score_chunk(k, v, alpha[0], alpha[1], mode, norm, layers=True)
        s_orc.append(s)
        ls_orc.append(ls)
    return s_gpu, ls_gpu, np.concatenate(s_orc), np.concatenate(ls_orc, axis=1)


def _rel_close(got, want, rtol=1e-4, floor=0.0):
    scale = np.maximum(np.abs(want), floor)
    err = np.abs(got.astype(np.float64) - want)
    bad = err > rtol * scale
    assert not bad.any(), f"max rel err {np.max(err / np.maximum(scale, 1e-300))}"


@pytest.mark.parametrize("ns,L,H,D,alpha", [
    ([300, 512, 1000, 64], 2, 2, 64, (1, 16)),     # ragged tails, several 32-token steps
    ([2048], 2, 8, 128, (1, 16)),                   # bench shapes, two layers
    ([96, 257], 2, 1, 64, (1, 2)),                  # the paper's default alpha
    ([130, 77], 1, 1, 64, (1, 1)),                  # alpha = 1: every bin (odd N, Nyquist)
    ([600, 4096], 1, 1, 64, (1, 32)),               # 1/32 cutoff, shortest/longest lengths
    ([2, 8192, 3], 1, 1, 64, (1, 16)),              # the smallest and largest chunk lengths
    ([64, 33], 1, 64, 128, (1, 16)),                # H*D = 8192, the most channels a call takes
    ([1024, 700], 1, 64, 128, (1, 8)),              # radix-4 and folded band passes at 8192 channels (64 and 43 bins)
    ([1152, 640, 384], 1, 2, 64, (1, 4)),           # radix-4 at lengths 9, 5 and 3 x 128: 144, 80 and 48 bins
])
def test_score_parity_bf16(orc, syn, ns, L, H, D, alpha):
    s_gpu, ls_gpu, s_orc, ls_orc = _score_both(orc, syn, ns, L, H, D, "bf16", alpha)
    _rel_close(s_gpu, s_orc)
    _rel_close(ls_gpu, ls_orc)


def _bf16_scaled(bits, factor):
    """bf16 bits times a power of two (exact)."""
    x = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_score_parity_bf16_wide_values(orc, syn):
    """bf16 data beyond the fp16 range: a band tile whose folded sums
    x[n] +- x[nf-n] reach 65520 in magnitude is redone unfolded with the three
    bf16 twiddle planes, the others stay on the fp16 pairs.  Whole problems
    are scaled by powers of two, which leaves each problem's conditioning as
    it was: chunk 1 layer 1 K reaches 75264 and chunk 0 layer 0 V 113664
    (redone); chunk 0 layer 1 K reaches 27776, so its sums stay below 55553
    (fp16, near the top of its range)."""
    def edit(host):
        host[1][0][1] = _bf16_scaled(host[1][0][1], 2.0 ** 11)
        host[0][1][0] = _bf16_scaled(host[0][1][0], 2.0 ** 12)
        host[0][0][1] = _bf16_scaled(host[0][0][1], 2.0 ** 10)
        wide = lambda a: float(np.abs((a.astype(np.uint32) << 16).view(np.float32)).max())
        assert wide(host[1][0][1]) >= 65536 and wide(host[0][1][0]) >= 65536
        assert 16384 <= wide(host[0][0][1]) and 2 * wide(host[0][0][1]) < 65520
    s_gpu, ls_gpu, s_orc, ls_orc = _score_both(orc, syn, [300, 2048], 2, 2, 64, "bf16", (1, 16), edit=edit)
    _rel_close(s_gpu, s_orc)
    _rel_close(ls_gpu, ls_orc)


def test_score_parity_bf16_radix4_overflow(orc, syn):
    """A 2048-token chunk (transform length divisible by 128: the radix-4 band
    pass) whose layer 0 is scaled by 2^9 (exact; its largest value becomes
    17024) and then carries 20480 in every channel at the four quarter-aligned
    tokens n, n + 512, n + 1024, n + 1536, with signs (+, +, +, +) in V and
    (+, -, +, -) in K: the four-term sums y0 (V) and y2 (K) reach 81920, past
    fp16's range, while every value and every pair sum stays inside it, so
    the radix-4 tiles of layer 0 are redone with the three bf16 twiddle
    planes; layer 1 stays on the fp16 pairs.  (Unscaled, the planted values
    would stand 10^4 standard deviations above the rest, and the scores of
    that layer would then be conditioned far worse than fp32 arithmetic
    resolves to 1e-4, on every band path alike.)"""
    big = np.uint16(0x46A0)  # bf16 20480
    def edit(host):
        for kv, signs in ((1, (1, 1, 1, 1)), (0, (1, -1, 1, -1))):
            a = host[0][kv]
            a[0] = _bf16_scaled(a[0], 2.0 ** 9)
            for q, sg in enumerate(signs):
                a[0, 7 + 512 * q] = big if sg > 0 else big | np.uint16(0x8000)
            x = (a.astype(np.uint32) << 16).view(np.float32)
            assert np.abs(x).max() == 20480.0 and 2 * np.abs(x).max() < 65504
    s_gpu, ls_gpu, s_orc, ls_orc = _score_both(orc, syn, [2048], 2, 2, 64, "bf16", (1, 16), edit=edit)
    _rel_close(s_gpu, s_orc)
    _rel_close(ls_gpu, ls_orc)


def test_score_parity_fp32_single_chunk(orc, syn):
    """The 1 x 512-token fp32 workload: L=1, 8 KV heads x 64."""
    s_gpu, ls_gpu, s_orc, _ = _score_both(orc, syn, [512], 1, 8, 64, "f32", (1, 16))
    _rel_close(s_gpu, s_orc)


@pytest.mark.parametrize("mode", [1])
@pytest.mark.parametrize("alpha", [(1, 16), (1, 8), (1, 2)])
def test_score_parity_zeropad(orc, syn, mode, alpha):
    """Transform lengths padded to 512 and 1024; at alpha 1/8 the 700-token
    chunk keeps 64 bins and takes the radix-4 band pass (length 1024), whose
    last quarter lies past the chunk's end (zeros); at alpha 1/2 both chunks
    take it (128 and 256 bins), the 300-token one with its last quarter
    (tokens 384 .. 511) entirely past the end.  Padded lengths are powers of
    two, so every block with more than 32 bins takes the radix-4 pass."""
    s_gpu, _, s_orc, _ = _score_both(orc, syn, [300, 700], 2, 1, 64, "bf16", alpha, mode=mode)
    _rel_close(s_gpu, s_orc)


@pytest.mark.parametrize("norm", [1, 2, 3])
def test_score_parity_norm_modes(orc, syn, norm):
    s_gpu, ls_gpu, s_orc, ls_orc = _score_both(orc, syn, [200, 333], 3, 1, 64, "bf16", (1, 8), norm=norm)
    floor = 1e-3 if norm == 2 else 0.0
    _rel_close(ls_gpu, ls_orc, floor=floor)
    _rel_close(s_gpu, s_orc, floor=floor)


def test_score_many_chunks_multiple_launches(orc, syn):
    ns = [64 + 3 * i for i in range(40)]
    s_gpu, _, s_orc, _ = _score_both(orc, syn, ns, 1, 1, 64, "bf16", (1, 16))
    _rel_close(s_gpu, s_orc)


def test_score_deterministic(syn):
    ct = need_gpu()
    host = _chunks(syn, [700, 1500], 2, 2, 64, "bf16")
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    a, _ = ct.cachetune_score_chunk(dev, 2, 2, 64)
    b, _ = ct.cachetune_score_chunk(dev, 2, 2, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---- selection ---------------------------------------------------------------

def _topr_exact(orc, scores_list, r):
    """Both top-r paths against the oracle: with the ranking stored (ranks by
    counting, then the lists) and without it (one sort per chunk)."""
    ct = need_gpu()
    ns = [len(s) for s in scores_list]
    flat = np.concatenate(scores_list).astype(np.float32)
    for want_ranking in (True, False):
        ks, ranking, sel, comp = ct.cachetune_select_topr(to_dev(flat), ns, r=r, want_ranking=want_ranking)
        torch.cuda.synchronize()
        sel, comp = to_host(sel), to_host(comp)
        ranking = to_host(ranking) if want_ranking else None
        o = so = co = 0
        for n, k, s in zip(ns, ks, scores_list):
            assert k == orc.ksel(n, *r)
            want_r, want_s, want_c = orc.topr(np.asarray(s, np.float32).astype(np.float64), k)
            if want_ranking:
                np.testing.assert_array_equal(ranking[o:o + n], want_r)
            np.testing.assert_array_equal(sel[so:so + k], want_s)
            np.testing.assert_array_equal(comp[co:co + n - k], want_c)
            o, so, co = o + n, so + k, co + n - k


def test_topr_exact_on_oracle_scores(orc, syn):
    scores = []
    for n in (512, 2048, 1000, 3):
        k, v = _chunks(syn, [n], 1, 1, 64, "bf16", seed=n)[0]
        scores.append(orc.score_chunk(k, v, 1, 16))
    for r in ((15, 100), (5, 100), (30, 100), (0, 1), (1, 1)):
        _topr_exact(orc, scores, r)


def test_topr_ties_and_signed_zero(orc):
    rng = np.random.default_rng(3)
    a = np.round(rng.random(700) * 5) / 5          # many exact ties
    b = np.zeros(64)
    b[::3] = -0.0                                   # -0 equals +0
    b[5] = 1.0
    c = np.array([0.25])                            # single-token chunk
    d = np.full(8192, 0.5)                          # maximum length, all equal
    d[8191] = 0.75
    _topr_exact(orc, [a, b, c, d], (15, 100))
    _topr_exact(orc, [a, b, c, d], (1, 2))


def test_topr_many_chunks(orc):
    rng = np.random.default_rng(4)
    scores = [rng.random(int(n)) for n in rng.integers(1, 300, 75)]
    _topr_exact(orc, scores, (15, 100))


@pytest.mark.parametrize("ns,L,H,D,dtype", [([300, 2048, 7], 2, 8, 128, "bf16"), ([512, 65], 3, 2, 64, "f32")])
def test_score_variant_l2(orc, syn, ns, L, H, D, dtype):
    """§5.4 L2-norm selection: joint K/V magnitudes without the frequency
    analysis, per-layer scores and the layer mean, against the oracle; then the
    index sets it selects."""
    ct = need_gpu()
    host = _chunks(syn, ns, L, H, D, dtype)
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    for norm in (ct.CT_NORM_SUM, ct.CT_NORM_MINMAX):
        s_gpu, ls_gpu = ct.cachetune_score_chunk(dev, L, H, D, norm=norm, want_layers=True,
                                                 variant=ct.CT_SCORE_L2)
        torch.cuda.synchronize()
        s_gpu, ls_gpu = to_host(s_gpu), to_host(ls_gpu)
        s_orc, ls_orc = [], []
        for k, v in host:
            s, ls = orc.score_l2(k, v, norm, layers=True)
            s_orc.append(s)
            ls_orc.append(ls)
        s_orc, ls_orc = np.concatenate(s_orc), np.concatenate(ls_orc, axis=1)
        _rel_close(s_gpu, s_orc, floor=1e-6 * np.abs(s_orc).max())
        _rel_close(ls_gpu, ls_orc, floor=1e-6 * np.abs(ls_orc).max())
    ks, _, sel, _ = ct.cachetune_select_topr(to_dev(s_gpu), ns, r=(15, 100))
    torch.cuda.synchronize()
    sel = to_host(sel)
    o = so = 0
    for n, k in zip(ns, ks):
        _, want, _ = orc.topr(s_orc[o:o + n], k)
        check_index_sets(sel[so:so + k], want, s_orc[o:o + n], k)
        o, so = o + n, so + k


@pytest.mark.parametrize("ns,L,H,D,dtype,alpha,fftlen", [
    ([300, 2048, 7], 1, 2, 64, "bf16", (1, 16), 0),
    ([2048], 1, 8, 128, "bf16", (1, 16), 0),       # the per-chunk shape of the 8 x 2048 workload
    ([513, 65], 2, 1, 64, "f32", (1, 2), 1),       # zero padding; a band of 512 rows (4 slices)
])
def test_score_variant_highpass(orc, syn, ns, L, H, D, dtype, alpha, fftlen):
    """Sec. 5.4 / App. E.2 high-frequency-guided selection: magnitudes of the
    bins at and above the cutoff, per-layer scores and the layer mean against
    the oracle's explicit high-band reconstruction; then the index sets."""
    ct = need_gpu()
    host = _chunks(syn, ns, L, H, D, dtype)
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    for norm in (ct.CT_NORM_SUM, ct.CT_NORM_NONE):
        s_gpu, ls_gpu = ct.cachetune_score_chunk(dev, L, H, D, alpha=alpha, fftlen=fftlen, norm=norm,
                                                 want_layers=True, variant=ct.CT_SCORE_HIGHPASS)
        torch.cuda.synchronize()
        s_gpu, ls_gpu = to_host(s_gpu), to_host(ls_gpu)
        s_orc, ls_orc = [], []
        for k, v in host:
            s, ls = orc.score_highpass(k, v, *alpha, mode=fftlen, norm=norm, layers=True)
            s_orc.append(s)
            ls_orc.append(ls)
        s_orc, ls_orc = np.concatenate(s_orc), np.concatenate(ls_orc, axis=1)
        _rel_close(s_gpu, s_orc, floor=1e-6 * np.abs(s_orc).max())
        _rel_close(ls_gpu, ls_orc, floor=1e-6 * np.abs(ls_orc).max())
    ks, _, sel, _ = ct.cachetune_select_topr(to_dev(s_gpu), ns, r=(15, 100))
    torch.cuda.synchronize()
    sel = to_host(sel)
    o = so = 0
    for n, k in zip(ns, ks):
        _, want, _ = orc.topr(s_orc[o:o + n], k)
        check_index_sets(sel[so:so + k], want, s_orc[o:o + n], k)
        o, so = o + n, so + k


@pytest.mark.parametrize("ns,L,H,D,dtype,fftlen,n_bands", [
    ([300, 64, 9], 2, 2, 64, "bf16", 0, 5),
    ([2048], 1, 8, 128, "bf16", 0, 10),            # the per-chunk shape of the 8 x 2048 workload
    ([513, 100], 1, 1, 64, "f32", 1, 10),         # zero padding to 1024 and 128
])
def test_band_energy(orc, syn, ns, L, H, D, dtype, fftlen, n_bands):
    """App. E.1 energy fractions of equal bands of rFFT bins, for K and V of
    every chunk and layer, and the totals, against the oracle."""
    ct = need_gpu()
    host = _chunks(syn, ns, L, H, D, dtype)
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    fr, tot = ct.cachetune_band_energy(dev, L, H, D, n_bands, fftlen=fftlen)
    torch.cuda.synchronize()
    fr, tot = to_host(fr), to_host(tot)
    for b, (k, v) in enumerate(host):
        for t, X in enumerate((k, v)):
            want_fr, want_tot = orc.band_energy(X, n_bands, fftlen)
            np.testing.assert_allclose(fr[b, :, t], want_fr, rtol=1e-4, atol=1e-7)
            np.testing.assert_allclose(tot[b, :, t], want_tot, rtol=1e-5)


def test_random_selection(orc, syn):
    """§5.4 random selection: top-r over seeded uniform scores (drawn by the
    input generator and passed in) is a uniformly random set of k tokens per
    chunk; GPU and oracle select the same set."""
    ns = [2048, 512, 1000]
    scores = [syn.uniform_ints(SEED, 77 + b, n, 0, 1 << 24).astype(np.float32) for b, n in enumerate(ns)]
    _topr_exact(orc, scores, (15, 100))


@pytest.mark.parametrize("ns,L,H,D,alpha", [([512, 2048, 999], 2, 2, 64, (1, 16)),
                                            ([2048], 3, 8, 128, (1, 16))])
def test_index_sets_end_to_end(orc, syn, ns, L, H, D, alpha):
    """GPU scores ranked on the GPU vs oracle scores ranked by the oracle."""
    ct = need_gpu()
    s_gpu, _, s_orc, _ = _score_both(orc, syn, ns, L, H, D, "bf16", alpha)
    ks, _, sel, _ = ct.cachetune_select_topr(to_dev(s_gpu), ns, r=(15, 100))
    torch.cuda.synchronize()
    sel = to_host(sel)
    o = so = 0
    for n, k in zip(ns, ks):
        _, want, _ = orc.topr(s_orc[o:o + n], k)
        check_index_sets(sel[so:so + k], want, s_orc[o:o + n], k)
        o, so = o + n, so + k


# ---- assembly ------------------------------------------------------------------

def _assembly_case(orc, syn, ns, H, D, dtype, theta, style, prefix, n_sfx, packed):
    ct = need_gpu()
    rng = np.random.default_rng(sum(ns) + D)
    order = rng.permutation(len(ns)).astype(np.int32)
    offs = orc.offsets(ns, order, prefix)
    T = prefix + sum(ns) + n_sfx
    edt = np.uint16 if dtype == "bf16" else np.float32
    k_ref = np.zeros((T, H, D), edt)
    v_ref = np.zeros((T, H, D), edt)
    places, keep = [], []
    for b, n in enumerate(ns):
        ks = syn.rows(SEED, syn.K, b, 5, n, H, D, np.arange(n), dtype)
        vs = syn.rows(SEED, syn.V, b, 5, n, H, D, np.arange(n), dtype)
        k = orc.ksel(n, 15, 100)
        sel = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
        comp = np.setdiff1d(np.arange(n, dtype=np.int32), sel).astype(np.int32)
        kr = syn.rows(SEED, syn.K, b, 5, n, H, D, sel, dtype, extra_sigma=0.25)
        vr = syn.rows(SEED, syn.V, b, 5, n, H, D, sel, dtype, extra_sigma=0.25)
        orc.assemble_chunk(ks, vs, kr, vr, sel, offs[b], theta, style, k_ref, v_ref)
        if packed:  # staging buffer: reused rows in an arbitrary (here: reversed) order
            src_rows = comp[::-1].copy()
            d = dict(k_src=to_dev(ks[src_rows]), v_src=to_dev(vs[src_rows]), src_rows=to_dev(src_rows))
        else:
            d = dict(k_src=to_dev(ks), v_src=to_dev(vs), comp=to_dev(comp))
        d.update(sel=to_dev(sel), k_rec=to_dev(kr) if k else None, v_rec=to_dev(vr) if k else None)
        keep.append(d)
        places.append(ct.make_place(n=n, k=k, offset=int(offs[b]), **d))
    ksf = syn.rows(SEED, syn.K, syn.SUFFIX_CHUNK, 5, n_sfx, H, D, np.arange(n_sfx), dtype)
    vsf = syn.rows(SEED, syn.V, syn.SUFFIX_CHUNK, 5, n_sfx, H, D, np.arange(n_sfx), dtype)
    orc.assemble_rows(ksf, vsf, prefix + sum(ns), theta, style, k_ref, v_ref)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k_out = torch.zeros((T, H, D), dtype=dt, device="cuda")
    v_out = torch.zeros((T, H, D), dtype=dt, device="cuda")
    ct.cachetune_assemble_rope(places, k_out, v_out, H, D, theta, style,
                               k_sfx=to_dev(ksf) if n_sfx else None,
                               v_sfx=to_dev(vsf) if n_sfx else None,
                               n_sfx=n_sfx, sfx_offset=prefix + sum(ns))
    torch.cuda.synchronize()
    kg, vg = to_host(k_out), to_host(v_out)
    np.testing.assert_array_equal(vg, v_ref)
    assert_rotated_keys(kg, k_ref, ulp_distance_bf16 if dtype == "bf16" else ulp_distance_f32)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("style", [0, 1])
def test_assemble_parity_bf16(orc, syn, D, style):
    _assembly_case(orc, syn, [300, 129, 512], 2, D, "bf16", 500000.0, style, prefix=17, n_sfx=33,
                   packed=False)


def test_assemble_parity_fp32_packed(orc, syn):
    _assembly_case(orc, syn, [200, 71], 8, 64, "f32", 10000.0, 0, prefix=0, n_sfx=16, packed=True)


def test_assemble_large_positions(orc, syn):
    """Positions around 1.5e5 (128K-context offsets): fp64 angles keep K exact."""
    _assembly_case(orc, syn, [256, 300], 1, 128, "bf16", 1000000.0, 0, prefix=150000, n_sfx=5,
                   packed=True)


def test_assemble_many_places(orc, syn):
    _assembly_case(orc, syn, [20 + i for i in range(37)], 1, 64, "bf16", 500000.0, 0, prefix=3,
                   n_sfx=0, packed=False)


# ---- attention -------------------------------------------------------------------

def _attn_case(orc, syn, T, H, Hq, D, n_q, dtype, theta, style, scale=None, v_mul=None):
    ct = need_gpu()
    rng = np.random.default_rng(T + n_q + D)
    k = syn.rows(SEED, syn.K, 0, 1, T, H, D, np.arange(T), dtype)
    v = syn.rows(SEED, syn.V, 0, 1, T, H, D, np.arange(T), dtype)
    if v_mul is not None:  # scale some rows of V by a power of two (exact in bf16)
        rows_, mul = v_mul
        v = v.copy()
        v[rows_] = (v[rows_].astype(np.uint32) + (int(np.log2(mul)) << 7)).astype(np.uint16)
    if n_q:
        qpos = np.sort(rng.choice(np.arange(1, T - 1), max(0, n_q - 2), replace=False))
        qpos = np.concatenate([[0], qpos, [T - 1]])[:n_q].astype(np.int32)
        qpos.sort()
    else:
        qpos = np.zeros(0, np.int32)
    q = syn.rows(SEED, syn.Q, 0, 1, T, Hq, D, qpos, dtype)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out, lse = ct.cachetune_recompute_attn(to_dev(q) if n_q else torch.zeros((0, Hq, D), device="cuda"),
                                           to_dev(qpos) if n_q else torch.zeros(0, dtype=torch.int32, device="cuda"),
                                           to_dev(k), to_dev(v), scale, theta, style, want_lse=True)
    torch.cuda.synchronize()
    if n_q == 0:
        return
    og, lg = widen(to_host(out)), to_host(lse).astype(np.float64)
    ref, lref = orc.attention(q, qpos, k, v, scale, theta, style)
    err = np.abs(og - ref)
    tol = 2e-2 + (half_ulp_bf16(ref) if dtype == "bf16" else 0.0)
    if v_mul is not None:
        # Huge V rows can cancel: the output's rounding then scales with
        # sum_t p_t |v_t| (the oracle run on |V|), not with the output itself.
        absv = (v & 0x7FFF) if dtype == "bf16" else np.abs(v)
        ref_abs, _ = orc.attention(q, qpos, k, absv, scale, theta, style)
        tol = tol + 2.0 ** -14 * ref_abs
    assert (err <= tol).all(), (err.max(), (err - tol).max())
    assert (np.abs(lg - lref) <= LSE_TOL).all(), np.abs(lg - lref).max()


@pytest.mark.parametrize("D", [128, 64])
def test_attention_parity_bf16(orc, syn, D):
    _attn_case(orc, syn, 1100, 2, 8, D, 150, "bf16", 500000.0, 0)


def test_attention_parity_fp32_mha(orc, syn):
    """Group size 1 (8 query heads over 8 KV heads), fp32 storage, theta 1e4."""
    _attn_case(orc, syn, 528, 8, 8, 64, 92, "f32", 10000.0, 0)


@pytest.mark.parametrize("n_q", [0, 1, 33])
def test_attention_edge_sizes(orc, syn, n_q):
    _attn_case(orc, syn, 300, 1, 4, 128, n_q, "bf16", 500000.0, 1)


def test_attention_wide_values(orc, syn):
    """V rows beyond the fp16 range (|v| >= 65536) in a few 64-key blocks: those
    segments take the bf16 path, the rest stays on fp16."""
    _attn_case(orc, syn, 1500, 2, 8, 128, 90, "bf16", 500000.0, 0, v_mul=([5, 700, 1400], 2.0 ** 16))


def test_attention_long_split(orc, syn):
    """Rows whose keys span several split-KV segments (T = 9000), ragged tile."""
    _attn_case(orc, syn, 9000, 1, 4, 128, 77, "bf16", 500000.0, 0)


@pytest.mark.parametrize("D", [128, 64])
def test_attention_split_partial_head_group(orc, syn, D):
    """Keys split over several segments with 6 query heads (groups of 3 over 2
    KV heads): the merge takes heads in fours, so its second group holds 2
    heads and half its lanes idle; D = 64 gives 4 dims per merge lane; both
    RoPE styles."""
    _attn_case(orc, syn, 9000, 2, 6, D, 70, "bf16", 500000.0, 0 if D == 128 else 1)


def test_attention_split_wide_values(orc, syn):
    """Split segments with V beyond the fp16 range in some of them: those
    segments' partials are stored as fp32, the others as fp16, and one row's
    merge can read both kinds."""
    _attn_case(orc, syn, 9000, 1, 4, 128, 60, "bf16", 500000.0, 0, v_mul=([40, 3000, 8500], 2.0 ** 16))


def test_attention_group8_long(orc, syn):
    _attn_case(orc, syn, 3000, 1, 8, 128, 70, "bf16", 500000.0, 0, scale=0.1)


def test_attention_many_items_natural_order(orc, syn, monkeypatch):
    """More (tile group, segment) items than the set-up launch sorts (54 tile
    groups x 40 segments of 1024 keys = 2160): the work list keeps its natural
    order, empty items included, and every row still gets all its segments
    merged.  Sampled rows across the context, all query heads."""
    monkeypatch.setenv("CACHETUNE_ATTN_SEG", "1024")
    ct = need_gpu()
    T, H, Hq, D, n_q = 40000, 1, 4, 128, 3400
    rng = np.random.default_rng(T + n_q)
    k = syn.rows(SEED, syn.K, 0, 1, T, H, D, np.arange(T), "bf16")
    v = syn.rows(SEED, syn.V, 0, 1, T, H, D, np.arange(T), "bf16")
    qpos = np.sort(rng.choice(np.arange(1, T - 1), n_q - 2, replace=False))
    qpos = np.concatenate([[0], qpos, [T - 1]]).astype(np.int32)
    q = syn.rows(SEED, syn.Q, 0, 1, T, Hq, D, qpos, "bf16")
    scale = 1.0 / np.sqrt(D)
    out, lse = ct.cachetune_recompute_attn(to_dev(q), to_dev(qpos), to_dev(k), to_dev(v), scale, 500000.0, 0,
                                           want_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, n_q - 2, n_q - 1], rng.choice(n_q, 12, replace=False)]))
    ref, lref = orc.attention(q, qpos, k, v, scale, 500000.0, 0, rows=rows)
    og, lg = widen(to_host(out))[rows], to_host(lse).astype(np.float64)[rows]
    assert (np.abs(og - ref) <= 2e-2 + half_ulp_bf16(ref)).all(), np.abs(og - ref).max()
    assert (np.abs(lg - lref) <= LSE_TOL).all(), np.abs(lg - lref).max()


# ---- host-tier sparse loading -------------------------------------------------------

@pytest.mark.parametrize("r", [(15, 100), (0, 1), (1, 1)])
def test_host_tier_matches_device_path(orc, syn, r):
    """Rank-ordered pinned host pool -> staged complement -> assembly from the
    packed staging (src_rows = ranking tail) equals the assembly from the
    device-resident chunks bit for bit, and the oracle's."""
    ct = need_gpu()
    ns, L, H, D, theta, layer = [300, 512, 129], 3, 2, 128, 500000.0, 1
    host = _chunks(syn, ns, L, H, D, "bf16")
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    score, _ = ct.cachetune_score_chunk(dev, L, H, D, alpha=(1, 16))
    ks, ranking, sel, comp = ct.cachetune_select_topr(score, ns, r=r)
    pool = []
    for b, (k, v) in enumerate(dev):
        off = sum(ns[:b])
        kr, vr = ct.cachetune_rank_order(k, v, ranking[off:off + ns[b]])
        pk = torch.empty(kr.shape, dtype=kr.dtype, pin_memory=True)
        pv = torch.empty(vr.shape, dtype=vr.dtype, pin_memory=True)
        pk.copy_(kr)
        pv.copy_(vr)
        pool.append((pk, pv))
    torch.cuda.synchronize()
    rows = sum(n - k for n, k in zip(ns, ks))
    k_stage = torch.zeros((max(rows, 1), H, D), dtype=torch.bfloat16, device="cuda")
    v_stage = torch.zeros_like(k_stage)
    ct.cachetune_stage_complement(pool, layer, ks, k_stage, v_stage)
    sel_h, comp_h = to_host(sel), to_host(comp)
    T = sum(ns) + 7
    offs = [sum(ns[:b]) for b in range(len(ns))]
    ref = [torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    k_ref = np.zeros((T, H, D), np.uint16)
    v_ref = np.zeros((T, H, D), np.uint16)
    pl_dev, pl_host, keep = [], [], []
    so = co = at = 0
    for b, n in enumerate(ns):
        k = ks[b]
        s_b = sel_h[so:so + k]
        krec = syn.rows(SEED, syn.K, b, layer, n, H, D, s_b, "bf16", extra_sigma=0.25)
        vrec = syn.rows(SEED, syn.V, b, layer, n, H, D, s_b, "bf16", extra_sigma=0.25)
        orc.assemble_chunk(host[b][0][layer], host[b][1][layer], krec, vrec, s_b, offs[b], theta, 0,
                           k_ref, v_ref)
        d = dict(sel=sel[so:] if k else None, k_rec=to_dev(krec) if k else None,
                 v_rec=to_dev(vrec) if k else None)
        keep.append(d)
        pl_dev.append(ct.make_place(dev[b][0][layer], dev[b][1][layer], n, k, offs[b],
                                    comp=comp[co:] if k < n else None, **d))
        o = sum(ns[:b])
        pl_host.append(ct.make_place(k_stage[at:] if k < n else None, v_stage[at:] if k < n else None,
                                     n, k, offs[b], src_rows=ranking[o + k:] if k < n else None, **d))
        so, co, at = so + k, co + n - k, at + n - k
    ct.cachetune_assemble_rope(pl_dev, ref[0], ref[1], H, D, theta)
    ct.cachetune_assemble_rope(pl_host, ref[2], ref[3], H, D, theta)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], ref[2]) and torch.equal(ref[1], ref[3])
    kg, vg = to_host(ref[2])[:sum(ns)], to_host(ref[3])[:sum(ns)]
    np.testing.assert_array_equal(vg, v_ref[:sum(ns)])
    assert_rotated_keys(kg, k_ref[:sum(ns)])


def test_rank_order_is_a_gather(syn):
    ct = need_gpu()
    L, n, H, D = 2, 333, 2, 64
    k = syn.chunk(SEED, syn.K, 3, L, n, H, D, "bf16")
    v = syn.chunk(SEED, syn.V, 3, L, n, H, D, "bf16")
    perm = np.random.default_rng(5).permutation(n).astype(np.int32)
    kd, vd = ct.cachetune_rank_order(to_dev(k), to_dev(v), to_dev(perm))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(kd), k[:, perm])
    np.testing.assert_array_equal(to_host(vd), v[:, perm])


def test_assembly_and_attention_deterministic(syn):
    """Two runs of the assembly and of the attention (persistent grid, work
    items taken from atomic counters in whatever order the blocks arrive) give
    bit-identical outputs: every item's arithmetic is independent of the block
    that runs it and the split-KV merge has a fixed order."""
    ct = need_gpu()
    T, H, Hq, D, theta = 9000, 8, 32, 128, 500000.0
    k = to_dev(syn.rows(SEED, syn.K, 0, 1, T, H, D, np.arange(T), "bf16"))
    v = to_dev(syn.rows(SEED, syn.V, 0, 1, T, H, D, np.arange(T), "bf16"))
    rng = np.random.default_rng(5)
    qpos = np.sort(rng.choice(T, 700, replace=False)).astype(np.int32)
    q = to_dev(syn.rows(SEED, syn.Q, 0, 1, T, Hq, D, qpos, "bf16"))
    n = T // 2
    sel = np.sort(rng.choice(n, 100, replace=False)).astype(np.int32)
    comp = np.setdiff1d(np.arange(n, dtype=np.int32), sel).astype(np.int32)
    keep = dict(sel=to_dev(sel), comp=to_dev(comp), k_rec=k[:100].contiguous(), v_rec=v[:100].contiguous())
    all2 = to_dev(np.arange(T - n, dtype=np.int32))
    places = [ct.make_place(k[:n], v[:n], n, 100, 0, **keep), ct.make_place(k[n:], v[n:], T - n, 0, n, comp=all2)]
    outs = []
    for _ in range(2):
        ka = torch.empty_like(k)
        va = torch.empty_like(v)
        ct.cachetune_assemble_rope(places, ka, va, H, D, theta)
        o, lse = ct.cachetune_recompute_attn(q, to_dev(qpos), ka, va, 1.0 / np.sqrt(D), theta, want_lse=True)
        torch.cuda.synchronize()
        outs.append((ka.clone(), va.clone(), o.clone(), lse.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)

"""Pins for the oracle's chunk scoring, top-r selection and index mapping
(App. B.1 of the CacheTune page).  Expected values come from hand derivations
(tests/golden), invariances of the definition, and brute force."""
import itertools
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(99)


def _rows(name):
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            yield line


def test_config_sizes(orc):
    for line in _rows("config_sizes.txt"):
        kind, n, num, den, want = line.split()
        n, num, den, want = int(n), int(num), int(den), int(want)
        if kind == "kkeep":
            assert orc.kkeep(orc.nbins(n), num, den) == want, line
        else:
            assert orc.ksel(n, num, den) == want, line


def test_hand_cases(orc):
    for line in _rows("score_hand_cases.txt"):
        head, ks, vs, exp = [p.strip() for p in line.split("|")]
        _, L, N, an, ad = head.split()
        L, N, an, ad = int(L), int(N), int(an), int(ad)
        K = np.array([float(v) for v in ks.split()], np.float32).reshape(L, N, 1, 1)
        V = np.array([float(v) for v in vs.split()], np.float32).reshape(L, N, 1, 1)
        nums, den = exp.split("/")
        want = np.array([float(v) for v in nums.split()]) / float(den)
        got = orc.score_chunk(K, V, an, ad)
        np.testing.assert_allclose(got, want, rtol=1e-13)


def _kv(syn, L=3, N=96, H=2, D=8, dtype="bf16", seed=5):
    K = syn.chunk(seed, syn.K, 0, L, N, H, D, dtype)
    V = syn.chunk(seed, syn.V, 0, L, N, H, D, dtype)
    return K, V


def test_sum_normalisation_total_is_one(orc, syn):
    K, V = _kv(syn)
    s, ls = orc.score_chunk(K, V, 1, 16, layers=True)
    assert abs(s.sum() - 1.0) < 1e-12
    np.testing.assert_allclose(ls.sum(axis=1), 1.0, atol=1e-12)
    assert (s > 0).all()


def test_invariances(orc, syn):
    K, V = _kv(syn, dtype="f32")
    base = orc.score_chunk(K, V, 1, 8)
    # global scale of K and V (exact in storage)
    np.testing.assert_allclose(orc.score_chunk(K * 4, V * 4, 1, 8), base, rtol=1e-12)
    # layers are averaged: their order does not matter
    p = [2, 0, 1]
    np.testing.assert_allclose(orc.score_chunk(K[p].copy(), V[p].copy(), 1, 8), base, rtol=1e-12)
    # K and V enter with equal weights
    np.testing.assert_allclose(orc.score_chunk(V, K, 1, 8), base, rtol=1e-12)
    # channels enter through an L2 norm: their order does not matter
    L, N, H, D = K.shape
    perm = RNG.permutation(H * D)
    Kp = K.reshape(L, N, H * D)[:, :, perm].reshape(L, N, H, D).copy()
    Vp = V.reshape(L, N, H * D)[:, :, perm].reshape(L, N, H, D).copy()
    np.testing.assert_allclose(orc.score_chunk(Kp, Vp, 1, 8), base, rtol=1e-12)
    # a circular shift of the chunk shifts the scores (exact-length transform)
    for s in (1, 17):
        got = orc.score_chunk(np.roll(K, s, axis=1).copy(), np.roll(V, s, axis=1).copy(), 1, 8)
        np.testing.assert_allclose(got, np.roll(base, s), rtol=1e-11)


def test_alpha_one_is_l2_ranking(orc, syn):
    """App. E.4: keeping all bins reduces the score to the L2 norms of K and V."""
    K, V = _kv(syn, L=2, N=50)
    got = orc.score_chunk(K, V, 1, 1)
    k, v = orc.widen(K), orc.widen(V)
    L, N = K.shape[:2]
    s = 0.5 * np.sqrt((k.reshape(L, N, -1) ** 2).sum(-1)) + 0.5 * np.sqrt((v.reshape(L, N, -1) ** 2).sum(-1))
    want = (s / s.sum(axis=1, keepdims=True)).mean(axis=0)
    np.testing.assert_allclose(got, want, rtol=1e-11)


def test_low_pass_score_matches_numpy_pipeline(orc, syn):
    """The whole score rebuilt from numpy's rfft/irfft (a library routine)."""
    K, V = _kv(syn, L=2, N=70, H=2, D=4)
    L, N = K.shape[:2]
    kk = orc.kkeep(N // 2 + 1, 1, 4)

    def mags(X):
        x = orc.widen(X).reshape(L, N, -1)
        F = np.fft.rfft(x, axis=1)
        F[:, kk:, :] = 0
        r = np.fft.irfft(F, n=N, axis=1)
        return np.sqrt((r ** 2).sum(-1))

    s = 0.5 * mags(K) + 0.5 * mags(V)
    want = (s / s.sum(axis=1, keepdims=True)).mean(axis=0)
    np.testing.assert_allclose(orc.score_chunk(K, V, 1, 4), want, rtol=1e-10)


def test_norm_modes(orc, syn):
    K, V = _kv(syn, L=2, N=64)
    _, lmax = orc.score_chunk(K, V, 1, 8, norm=orc.NORM_MAX, layers=True)
    np.testing.assert_allclose(lmax.max(axis=1), 1.0, atol=1e-15)
    _, lmm = orc.score_chunk(K, V, 1, 8, norm=orc.NORM_MINMAX, layers=True)
    np.testing.assert_allclose(lmm.min(axis=1), 0.0, atol=1e-15)
    np.testing.assert_allclose(lmm.max(axis=1), 1.0, atol=1e-15)
    _, lnone = orc.score_chunk(K, V, 1, 8, norm=orc.NORM_NONE, layers=True)
    _, lsum = orc.score_chunk(K, V, 1, 8, norm=orc.NORM_SUM, layers=True)
    np.testing.assert_allclose(lsum, lnone / lnone.sum(axis=1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(lmax, lnone / lnone.max(axis=1, keepdims=True), rtol=1e-13)


def test_zero_layer_sum_gives_uniform(orc):
    K = np.zeros((1, 8, 1, 2), np.float32)
    np.testing.assert_allclose(orc.score_chunk(K, K, 1, 2), 1.0 / 8, rtol=0)


def test_spike_tokens_rank_first(orc, syn):
    """Sanity on the synthetic model: with alpha = 1 the 5x spike tokens are the
    largest magnitudes of every channel, so they head the ranking."""
    K, V = _kv(syn, L=1, N=256, H=4, D=16)
    s = orc.score_chunk(K, V, 1, 1)
    top4 = set(np.argsort(-s)[:4].tolist())
    assert top4 == set(syn.spikes(5, 0, 256).tolist())


# ---- top-r -------------------------------------------------------------

def _check_selection(s, k, ranking, sel, comp):
    n = s.shape[0]
    order = sorted(range(n), key=lambda i: (-s[i], i))
    assert ranking.tolist() == order
    assert sel.tolist() == sorted(order[:k])
    assert comp.tolist() == sorted(order[k:])


@pytest.mark.parametrize("n", [1, 2, 7, 64, 513])
def test_topr_matches_sorted_reference(orc, n):
    s = RNG.random(n)
    s[::5] = 0.5  # plenty of exact ties
    for k in sorted({0, 1, n // 3, n - 1, n} - {-1}):
        if 0 <= k <= n:
            _check_selection(s, k, *orc.topr(s, k))


@pytest.mark.parametrize("n", [4, 9, 12])
def test_topr_brute_force(orc, n):
    """Among all k-subsets exactly one dominates its complement under the rule
    (higher score, or equal score and lower index); the oracle returns it."""
    s = np.round(RNG.random(n) * 4) / 4  # coarse values -> ties
    for k in range(n + 1):
        def beats(i, j):
            return s[i] > s[j] or (s[i] == s[j] and i < j)
        good = [c for c in itertools.combinations(range(n), k)
                if all(beats(i, j) for i in c for j in set(range(n)) - set(c))]
        assert len(good) == 1
        _, sel, comp = orc.topr(s, k)
        assert tuple(sel.tolist()) == good[0]
        assert sorted(sel.tolist() + comp.tolist()) == list(range(n))


def test_topr_nested(orc):
    """App. B.1: changing r changes the set size along one stored ranking."""
    s = RNG.random(300)
    prev = set()
    for k in range(0, 301, 7):
        cur = set(orc.topr(s, k)[1].tolist())
        assert prev <= cur and len(cur) == k
        prev = cur


# ---- index mapping ------------------------------------------------------

def test_offsets(orc):
    n = [5, 3, 7]
    # App. B.1: chunk b starting at o_b maps local i to o_b + i (0-based here)
    np.testing.assert_array_equal(orc.offsets(n, [0, 1, 2]), [0, 5, 8])
    np.testing.assert_array_equal(orc.offsets(n, [2, 0, 1]), [7, 12, 0])
    np.testing.assert_array_equal(orc.offsets(n, [2, 0, 1], prefix=1024), [1031, 1036, 1024])


def test_reordering_changes_only_mapping(orc, syn):
    """Scores and indices depend on chunk content only (App. B.1, E.2)."""
    a = _kv(syn, seed=1)
    b = _kv(syn, seed=2)
    sa = orc.score_chunk(*a, 1, 16)
    sb = orc.score_chunk(*b, 1, 16)
    # the same chunks scored in another order give identical per-chunk results
    np.testing.assert_array_equal(orc.score_chunk(*b, 1, 16), sb)
    np.testing.assert_array_equal(orc.score_chunk(*a, 1, 16), sa)


# ---- §5.4 L2-norm selection score ------------------------------------------------------

def test_l2_score_hand_case(orc):
    # one layer, two tokens, H = D = 1: a = |k|, b = |v|, s = a/2 + b/2, sum-normalised
    K = np.array([[[[3.0]], [[0.0]]]], np.float32)
    V = np.array([[[[-4.0]], [[1.0]]]], np.float32)
    s = orc.score_l2(K, V)
    assert np.allclose(s, [3.5 / 4.0, 0.5 / 4.0], rtol=0, atol=1e-15)


def test_l2_score_equals_alpha_one_score(orc):
    # App. E.4: keeping every bin reconstructs the stored rows, so the
    # frequency-guided score at alpha = 1 is the L2 score (two independent code
    # paths: direct DFT and inverse vs plain norms)
    rng = np.random.default_rng(11)
    for N in (7, 16, 33):
        K = rng.standard_normal((3, N, 2, 4)).astype(np.float32)
        V = rng.standard_normal((3, N, 2, 4)).astype(np.float32)
        for norm in (orc.NORM_SUM, orc.NORM_MAX, orc.NORM_MINMAX, orc.NORM_NONE):
            a = orc.score_l2(K, V, norm)
            b = orc.score_chunk(K, V, 1, 1, norm=norm)
            assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


def test_l2_score_scale_and_layer_permutation(orc):
    rng = np.random.default_rng(12)
    K = rng.standard_normal((4, 20, 2, 4)).astype(np.float32)
    V = rng.standard_normal((4, 20, 2, 4)).astype(np.float32)
    s = orc.score_l2(K, V)
    assert np.isclose(s.sum(), 1.0, rtol=1e-12)
    assert np.allclose(orc.score_l2(4.0 * K, 4.0 * V), s, rtol=1e-12)   # exact power-of-two scale
    assert np.allclose(orc.score_l2(K[::-1].copy(), V[::-1].copy()), s, rtol=1e-12)


# ---- Sec. 5.4 / App. E.2 high-frequency-guided selection score -----------------------

def test_highpass_score_matches_numpy_pipeline(orc, syn):
    """The high-frequency score rebuilt from numpy's rfft/irfft."""
    K, V = _kv(syn, L=2, N=70, H=2, D=4)
    L, N = K.shape[:2]
    kk = orc.kkeep(N // 2 + 1, 1, 4)

    def mags(X):
        x = orc.widen(X).reshape(L, N, -1)
        F = np.fft.rfft(x, axis=1)
        F[:, :kk, :] = 0
        r = np.fft.irfft(F, n=N, axis=1)
        return np.sqrt((r ** 2).sum(-1))

    s = 0.5 * mags(K) + 0.5 * mags(V)
    for norm, want in ((orc.NORM_SUM, (s / s.sum(axis=1, keepdims=True)).mean(axis=0)),
                       (orc.NORM_NONE, s.mean(axis=0))):
        np.testing.assert_allclose(orc.score_highpass(K, V, 1, 4, norm=norm), want, rtol=1e-10)


def test_highpass_score_zeropad_matches_numpy(orc, syn):
    K, V = _kv(syn, L=1, N=50, H=1, D=4, dtype="f32")
    L, N = K.shape[:2]
    nf = 64
    kk = orc.kkeep(nf // 2 + 1, 1, 8)

    def mags(X):
        x = np.concatenate([orc.widen(X).reshape(L, N, -1), np.zeros((L, nf - N, 4))], axis=1)
        F = np.fft.rfft(x, axis=1)
        F[:, :kk, :] = 0
        r = np.fft.irfft(F, n=nf, axis=1)[:, :N]
        return np.sqrt((r ** 2).sum(-1))

    s = 0.5 * mags(K) + 0.5 * mags(V)
    got = orc.score_highpass(K, V, 1, 8, mode=orc.FFT_ZEROPAD_POW2, norm=orc.NORM_MAX)
    np.testing.assert_allclose(got, (s / s.max(axis=1, keepdims=True)).mean(axis=0), rtol=1e-10)


def test_highpass_score_of_high_band_content_is_l2(orc):
    # rows built from bins at or above the cutoff pass unchanged, so the
    # high-frequency score equals the L2 score; the low-frequency score of the
    # same rows sees only the float32 rounding of the stored rows
    L, N, H, D = 2, 64, 2, 3
    t = np.arange(N)
    rng = np.random.default_rng(21)
    K = np.zeros((L, N, H, D))
    V = np.zeros((L, N, H, D))
    for X in (K, V):
        for l in range(L):
            for h in range(H):
                for d in range(D):
                    f = rng.integers(4, N // 2 + 1)  # cutoff for alpha 1/8, N = 64: bin 4
                    X[l, :, h, d] = rng.uniform(0.5, 2.0) * np.cos(2 * np.pi * f * t / N + rng.uniform(0, 6))
    K, V = K.astype(np.float32), V.astype(np.float32)
    assert orc.kkeep(N // 2 + 1, 1, 8) == 4
    # float32 storage rounds the rows: compare against the rows as stored
    np.testing.assert_allclose(orc.score_highpass(K, V, 1, 8), orc.score_l2(K, V), rtol=1e-6)
    assert orc.score_chunk(K, V, 1, 8, norm=orc.NORM_NONE).max() < 1e-6


def test_highpass_score_hand_case(orc):
    # N = 2, one channel, exact length: bins 0 (mean) and 1 (Nyquist, half the
    # difference); alpha 1/2 keeps bin 0 low, so the high view is
    # x - mean = (+-d/2): magnitudes |k0-k1|/2 at both tokens
    K = np.array([[[[3.0]], [[1.0]]]], np.float32)
    V = np.array([[[[-2.0]], [[2.0]]]], np.float32)
    s = orc.score_highpass(K, V, 1, 2, norm=orc.NORM_NONE)
    assert orc.kkeep(2, 1, 2) == 1
    np.testing.assert_allclose(s, [0.5 * 1.0 + 0.5 * 2.0] * 2, atol=1e-14)

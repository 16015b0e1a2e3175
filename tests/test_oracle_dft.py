"""Pins for the oracle's transform and low-pass reconstruction (App. B.1 of the
CacheTune page: rFFT along tokens, keep the lowest alpha fraction of the
floor(N/2)+1 bins, inverse transform with output length N).

Each pin comes from outside the oracle: closed forms of the DFT, Parseval's
identity, a textbook radix-2 FFT written here, numpy's FFT routines, and
structural invariants of an ideal low-pass projector."""
import numpy as np
import pytest

RNG = np.random.default_rng(1234)


def radix2_fft(x):
    """Textbook recursive Cooley-Tukey FFT (power-of-two lengths)."""
    x = np.asarray(x, dtype=complex)
    n = x.shape[0]
    if n == 1:
        return x
    even = radix2_fft(x[0::2])
    odd = radix2_fft(x[1::2])
    tw = np.exp(-2j * np.pi * np.arange(n // 2) / n)
    return np.concatenate([even + tw * odd, even - tw * odd])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 17, 64])
def test_impulse_has_flat_spectrum(orc, n):
    x = np.zeros(n)
    x[0] = 1.0
    X = orc.rfft(x)
    assert X.shape == (n // 2 + 1,)
    np.testing.assert_allclose(X, np.ones(n // 2 + 1), atol=1e-15)


@pytest.mark.parametrize("n", [2, 7, 16, 33])
def test_constant_only_dc(orc, n):
    X = orc.rfft(np.full(n, 2.5))
    assert abs(X[0] - 2.5 * n) < 1e-12
    np.testing.assert_allclose(X[1:], 0.0, atol=1e-12)


@pytest.mark.parametrize("n,f", [(16, 3), (17, 5), (64, 1), (30, 7)])
def test_on_bin_cosine(orc, n, f):
    A, phi = 1.7, 0.4
    t = np.arange(n)
    X = orc.rfft(A * np.cos(2 * np.pi * f * t / n + phi))
    expect = np.zeros(n // 2 + 1, complex)
    expect[f] = A * n / 2 * np.exp(1j * phi)
    np.testing.assert_allclose(X, expect, atol=1e-11)


def test_nyquist_bin_real(orc):
    n = 12
    x = np.cos(np.pi * np.arange(n))  # (-1)^n: all energy in bin N/2
    X = orc.rfft(x)
    assert abs(X[n // 2] - n) < 1e-12 and abs(X[n // 2].imag) == 0.0
    np.testing.assert_allclose(X[: n // 2], 0.0, atol=1e-12)


@pytest.mark.parametrize("n", [5, 16, 31, 100, 257])
def test_parseval(orc, n):
    x = RNG.standard_normal(n)
    X = orc.rfft(x)
    w = np.full(n // 2 + 1, 2.0)
    w[0] = 1.0
    if n % 2 == 0:
        w[-1] = 1.0
    assert abs(np.sum(x * x) - np.sum(w * np.abs(X) ** 2) / n) < 1e-10 * np.sum(x * x)


@pytest.mark.parametrize("n", [8, 64, 512])
def test_matches_textbook_radix2(orc, n):
    x = RNG.standard_normal(n)
    np.testing.assert_allclose(orc.rfft(x), radix2_fft(x)[: n // 2 + 1], atol=1e-11 * n)


@pytest.mark.parametrize("n", [6, 9, 100, 333])
def test_matches_numpy_rfft(orc, n):
    x = RNG.standard_normal(n)
    np.testing.assert_allclose(orc.rfft(x), np.fft.rfft(x), atol=1e-11 * n)


# ---- low-pass -----------------------------------------------------------

def np_lowpass(x, kk, nf=None):
    """Library-routine construction: numpy rfft, zero bins >= kk, irfft(n)."""
    n = x.shape[0]
    nf = n if nf is None else nf
    xp = np.zeros(nf)
    xp[:n] = x
    X = np.fft.rfft(xp)
    X[kk:] = 0
    return np.fft.irfft(X, n=nf)[:n]


@pytest.mark.parametrize("n", [2, 3, 4, 7, 16, 61, 128, 300])
def test_alpha_one_is_identity(orc, n):
    x = RNG.standard_normal(n)
    np.testing.assert_allclose(orc.lowpass(x, 1, 1), x, atol=1e-12)


@pytest.mark.parametrize("n,a_num,a_den", [(64, 1, 16), (65, 1, 16), (100, 1, 2), (2048, 1, 16),
                                           (513, 1, 32), (16, 3, 7), (9, 1, 100)])
def test_matches_numpy_projector(orc, n, a_num, a_den):
    x = RNG.standard_normal(n)
    kk = max(1, (a_num * (n // 2 + 1)) // a_den)
    np.testing.assert_allclose(orc.lowpass(x, a_num, a_den), np_lowpass(x, kk), atol=1e-11)


@pytest.mark.parametrize("n,a_num,a_den", [(100, 1, 16), (600, 1, 32), (33, 1, 2)])
def test_zeropad_mode_matches_numpy(orc, n, a_num, a_den):
    x = RNG.standard_normal(n)
    nf = 1 << (n - 1).bit_length()
    kk = max(1, (a_num * (nf // 2 + 1)) // a_den)
    got = orc.lowpass(x, a_num, a_den, orc.FFT_ZEROPAD_POW2)
    np.testing.assert_allclose(got, np_lowpass(x, kk, nf), atol=1e-11)


def test_cosine_passband_and_stopband(orc):
    n, a_num, a_den = 2048, 1, 16  # keeps bins 0..63
    t = np.arange(n)
    below = 1.3 * np.cos(2 * np.pi * 63 * t / n + 0.2)
    above = 0.8 * np.cos(2 * np.pi * 64 * t / n + 1.1)
    np.testing.assert_allclose(orc.lowpass(below, a_num, a_den), below, atol=1e-11)
    np.testing.assert_allclose(orc.lowpass(above, a_num, a_den), 0.0, atol=1e-11)


def test_dc_only_gives_mean(orc):
    x = RNG.standard_normal(40)
    # alpha so small that only the DC bin survives
    np.testing.assert_allclose(orc.lowpass(x, 1, 1000), np.full(40, x.mean()), atol=1e-13)


@pytest.mark.parametrize("n", [10, 64, 77])
def test_projector_properties(orc, n):
    a = RNG.standard_normal(n)
    b = RNG.standard_normal(n)
    lp = lambda v: orc.lowpass(v, 1, 4)
    la = lp(a)
    np.testing.assert_allclose(lp(la), la, atol=1e-12)                       # idempotent
    np.testing.assert_allclose(lp(2.0 * a - 3.0 * b), 2.0 * la - 3.0 * lp(b), atol=1e-11)  # linear
    for s in (1, 5, n - 1):                                                   # shift equivariant
        np.testing.assert_allclose(lp(np.roll(a, s)), np.roll(la, s), atol=1e-11)
    rev = lambda v: np.roll(v[::-1], 1)                                       # x[-n mod N]
    np.testing.assert_allclose(lp(rev(a)), rev(la), atol=1e-11)               # time reversal
    # orthogonal projector: residual orthogonal to the kept part
    assert abs(np.dot(a - la, la)) < 1e-9 * np.dot(a, a)


@pytest.mark.parametrize("n", [4, 5, 8, 11, 16])
def test_brute_force_projector_matrix(orc, n):
    """Explicit N x N projector built from complex exponentials of the kept
    frequencies (+-j for j < kk, counting the Nyquist frequency once)."""
    for kk_target in range(1, n // 2 + 2):
        # choose alpha = kk/(nbins) exactly
        nb = n // 2 + 1
        kk = max(1, (kk_target * nb) // nb)
        freqs = {0}
        for j in range(1, kk):
            freqs.add(j % n)
            freqs.add((-j) % n)
        F = np.exp(2j * np.pi * np.outer(np.arange(n), sorted(freqs)) / n)
        P = (F @ F.conj().T).real / n
        x = RNG.standard_normal(n)
        np.testing.assert_allclose(orc.lowpass(x, kk_target, nb), P @ x, atol=1e-12)


# ---- high-frequency view (Sec. 5.4, App. E.2 Table 3) ---------------------------------

def np_highpass(x, kk, nf=None):
    n = x.shape[0]
    nf = n if nf is None else nf
    F = np.fft.rfft(np.concatenate([x, np.zeros(nf - n)]))
    F[:kk] = 0
    return np.fft.irfft(F, n=nf)[:n]


@pytest.mark.parametrize("n,a_num,a_den", [(64, 1, 16), (65, 1, 16), (100, 1, 2), (513, 1, 32),
                                           (16, 3, 7), (9, 1, 100)])
def test_highpass_matches_numpy(orc, n, a_num, a_den):
    x = RNG.standard_normal(n)
    kk = max(1, (a_num * (n // 2 + 1)) // a_den)
    np.testing.assert_allclose(orc.highpass(x, a_num, a_den), np_highpass(x, kk), atol=1e-11)


@pytest.mark.parametrize("n,a_num,a_den", [(100, 1, 16), (600, 1, 32), (33, 1, 2)])
def test_highpass_zeropad_matches_numpy(orc, n, a_num, a_den):
    x = RNG.standard_normal(n)
    nf = 1 << (n - 1).bit_length()
    kk = max(1, (a_num * (nf // 2 + 1)) // a_den)
    got = orc.highpass(x, a_num, a_den, orc.FFT_ZEROPAD_POW2)
    np.testing.assert_allclose(got, np_highpass(x, kk, nf), atol=1e-11)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("n", [5, 32, 77, 300])
def test_low_plus_high_is_signal(orc, n, mode):
    # the two views split the spectrum, so they add up to the signal at every
    # stored position (also with zero padding: the padded tail is cut after)
    x = RNG.standard_normal(n)
    for a in ((1, 16), (1, 2), (3, 7)):
        np.testing.assert_allclose(orc.lowpass(x, *a, mode) + orc.highpass(x, *a, mode), x, atol=1e-11)


def test_highpass_cosine_pass_and_stop(orc):
    n, a_num, a_den = 2048, 1, 16  # cutoff at bin 64
    t = np.arange(n)
    below = 1.3 * np.cos(2 * np.pi * 63 * t / n + 0.2)
    above = 0.8 * np.cos(2 * np.pi * 64 * t / n + 1.1)
    nyq = np.where(t % 2 == 0, 2.5, -2.5)  # the Nyquist bin, real by construction
    np.testing.assert_allclose(orc.highpass(below, a_num, a_den), 0.0, atol=1e-11)
    np.testing.assert_allclose(orc.highpass(above, a_num, a_den), above, atol=1e-11)
    np.testing.assert_allclose(orc.highpass(nyq, a_num, a_den), nyq, atol=1e-11)


def test_highpass_parseval_and_empty_band(orc):
    n = 90
    x = RNG.standard_normal(n)
    kk = (1 * (n // 2 + 1)) // 4
    F = np.fft.rfft(x)
    w = np.full(n // 2 + 1, 2.0)
    w[0] = 1.0
    w[-1] = 1.0  # n even: Nyquist counted once
    want = (w[kk:] * np.abs(F[kk:]) ** 2).sum() / n
    assert np.isclose((orc.highpass(x, 1, 4) ** 2).sum(), want, rtol=1e-11)
    # alpha = 1 keeps every bin in the low view: nothing is left above it
    np.testing.assert_allclose(orc.highpass(x, 1, 1), 0.0, atol=1e-12)
    # the DC bin is always in the low view: the high view has zero mean
    assert abs(orc.highpass(x, 1, 1000).sum()) < 1e-10


# ---- App. E.1 band energy fractions ----------------------------------------------------

def _np_band(x, n_bands, nf):
    # x [L][N][C] float64 -> fractions [L][n_bands], totals [L] from numpy's rfft
    L, N, C = x.shape
    xp = np.concatenate([x, np.zeros((L, nf - N, C))], axis=1)
    F = np.fft.rfft(xp, axis=1)
    nb = nf // 2 + 1
    w = np.full(nb, 2.0)
    w[0] = 1.0
    if nf % 2 == 0:
        w[-1] = 1.0
    e = (w[None, :, None] * np.abs(F) ** 2 / nf).sum(-1)  # [L][nb]
    band = (np.arange(nb) * n_bands) // nb
    fr = np.stack([np.bincount(band, weights=e[l], minlength=n_bands) for l in range(L)])
    tot = e.sum(-1)
    return fr / tot[:, None], tot


@pytest.mark.parametrize("N,mode,n_bands", [(64, 0, 10), (77, 0, 5), (100, 1, 8), (33, 1, 17), (9, 0, 5)])
def test_band_energy_matches_numpy(orc, N, mode, n_bands):
    X = RNG.standard_normal((2, N, 2, 3)).astype(np.float32)
    fr, tot = orc.band_energy(X, n_bands, mode)
    nf = N if mode == 0 else 1 << (N - 1).bit_length()
    want_fr, want_tot = _np_band(X.astype(np.float64).reshape(2, N, 6), n_bands, nf)
    np.testing.assert_allclose(fr, want_fr, atol=1e-12)
    np.testing.assert_allclose(tot, want_tot, rtol=1e-11)


@pytest.mark.parametrize("mode", [0, 1])
def test_band_energy_parseval_and_sum(orc, mode):
    # Parseval: the bins carry the energy of the stored sequence (zero padding adds none)
    X = RNG.standard_normal((3, 50, 1, 4)).astype(np.float32)
    fr, tot = orc.band_energy(X, 7, mode)
    np.testing.assert_allclose(tot, (X.astype(np.float64) ** 2).sum(axis=(1, 2, 3)), rtol=1e-12)
    np.testing.assert_allclose(fr.sum(axis=1), 1.0, atol=1e-13)
    assert (fr >= 0).all()


def test_band_energy_single_bins(orc):
    N, nb, n_bands = 40, 21, 4   # bands of bins: [0,6) [6,11) [11,16) [16,21)
    t = np.arange(N)
    for f, band in ((0, 0), (5, 0), (6, 1), (10, 1), (11, 2), (15, 2), (16, 3), (20, 3)):
        x = np.cos(2 * np.pi * f * t / N + (0.0 if f in (0, 20) else 0.7))
        X = np.tile(x[None, :, None, None], (1, 1, 1, 2)).astype(np.float64).astype(np.float32)
        fr, _ = orc.band_energy(X, n_bands)
        assert fr[0, band] > 1.0 - 1e-6, (f, fr)
    # constant rows: all energy at DC; n_bands = nb puts each bin in a band of its own
    fr, tot = orc.band_energy(np.full((1, N, 1, 1), 3.0, np.float32), nb)
    assert fr[0, 0] == pytest.approx(1.0, abs=1e-14) and tot[0] == pytest.approx(9.0 * N, rel=1e-14)
    with pytest.raises(ValueError):
        orc.band_energy(np.zeros((1, N, 1, 1), np.float32), nb + 1)

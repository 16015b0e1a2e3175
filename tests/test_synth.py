"""Checks of the seeded input generator: determinism (also across thread
counts), row evaluation consistent with whole-chunk evaluation, and the value
model's statistics."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_deterministic_and_thread_independent(syn):
    code = ("import sys; sys.path.insert(0, %r); import synth, hashlib;"
            "x = synth.chunk(77, 1, 3, 2, 300, 4, 16, 'bf16');"
            "print(hashlib.sha256(x.tobytes()).hexdigest())") % ROOT
    outs = set()
    for th in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=th)
        outs.add(subprocess.check_output([sys.executable, "-c", code], env=env).strip())
    assert len(outs) == 1


def test_rows_match_chunk(syn):
    x = syn.chunk(5, syn.V, 2, 3, 128, 2, 8, "f32")
    idx = np.array([127, 0, 64, 3], np.int32)
    np.testing.assert_array_equal(syn.rows(5, syn.V, 2, 1, 128, 2, 8, idx, "f32"), x[1, idx])
    # a different tensor / chunk / layer / seed gives different values
    assert not np.array_equal(syn.chunk(5, syn.K, 2, 3, 128, 2, 8, "f32"), x)
    assert not np.array_equal(syn.chunk(6, syn.V, 2, 3, 128, 2, 8, "f32"), x)


def test_value_model_statistics(syn):
    N, H, D = 2048, 4, 32
    x = syn.chunk(11, syn.K, 0, 1, N, H, D, "f32")[0].reshape(N, H * D).astype(np.float64)
    spk = syn.spikes(11, 0, N)
    assert len(set(spk.tolist())) == 4
    mask = np.ones(N, bool)
    mask[spk] = False
    # spectrum of the non-spike part: sinusoids live in bins 1..8
    y = x.copy()
    y[spk] /= 5.0
    F = np.abs(np.fft.rfft(y, axis=0)) ** 2 / N
    low = F[1:9].sum(axis=0)
    high = F[9:].mean(axis=0)
    assert np.median(high) < 2.0 and np.median(low) > 100.0
    # noise part: remove bins 1..8, the rest is white with unit variance
    G = np.fft.rfft(y, axis=0)
    G[1:9] = 0
    G[0] = 0
    z = np.fft.irfft(G, n=N, axis=0)
    assert abs(z.var() - 1.0) < 0.05
    # spike tokens have ~5x the rms of other tokens
    assert np.sqrt((x[spk] ** 2).mean()) > 3.5 * np.sqrt((x[mask] ** 2).mean())


def test_recomputed_rows_are_perturbed_copies(syn):
    idx = np.arange(0, 512, 3, dtype=np.int32)
    base = syn.rows(8, syn.K, 1, 0, 512, 8, 64, idx, "f32")
    rec = syn.rows(8, syn.K, 1, 0, 512, 8, 64, idx, "f32", extra_sigma=0.25)
    d = (rec - base).astype(np.float64)
    assert abs(d.std() - 0.25) < 0.01 and abs(d.mean()) < 0.01


def test_lengths_and_orders(syn):
    n = syn.uniform_ints(20260524, 0, 64, 512, 4096)
    assert n.min() >= 512 and n.max() <= 4096 and len(set(n.tolist())) > 50
    p = syn.permutation(20260523, 0, 16)
    assert sorted(p.tolist()) == list(range(16)) and p.tolist() != list(range(16))


def test_normal_stream(syn):
    a = syn.normal(5, 2, (300, 40), "f32", mean=1.0, sigma=0.5)
    b = syn.normal(5, 2, (300, 40), "f32", mean=1.0, sigma=0.5)
    np.testing.assert_array_equal(a, b)  # counter-based: same seed and stream, same values
    assert not np.array_equal(a, syn.normal(5, 3, (300, 40), "f32", mean=1.0, sigma=0.5))
    assert abs(a.mean() - 1.0) < 0.01 and abs(a.std() - 0.5) < 0.01
    h = syn.normal(5, 2, (300, 40), "bf16", mean=1.0, sigma=0.5)
    assert h.dtype == np.uint16
    w = (h.astype(np.uint32) << 16).view(np.float32)
    assert np.abs(w - a).max() <= 2.0 ** -8 * np.abs(a).max()

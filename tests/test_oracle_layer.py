"""Pins for the oracle's selective-recompute layer pieces (synthetic weights):
RMSNorm, the bias-free projection, the gated MLP activation and their
composition into one decoder layer over the assembled cache."""
import math

import numpy as np
import pytest


def test_rmsnorm_hand_case_and_invariants(orc):
    y = orc.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    np.testing.assert_allclose(y, [3.0 / math.sqrt(12.5), 4.0 / math.sqrt(12.5)], rtol=1e-15)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64))
    g = rng.uniform(0.5, 2.0, 64)
    y = orc.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-14)  # unit rms
    np.testing.assert_allclose(orc.rmsnorm(7.5 * x, g, 0.0), orc.rmsnorm(x, g, 0.0), rtol=1e-13)
    np.testing.assert_allclose(orc.rmsnorm(x, g, 0.0), y * g, rtol=1e-14)  # gain after normalising
    # eps: a zero row stays zero, a tiny row is damped
    assert np.all(orc.rmsnorm(np.zeros((1, 8)), np.ones(8), 1e-5) == 0.0)
    t = orc.rmsnorm(np.full((1, 4), 1e-3), np.ones(4), 1e-5)
    np.testing.assert_allclose(t, 1e-3 / math.sqrt(1e-6 + 1e-5), rtol=1e-14)


def test_linear_brute_force(orc):
    rng = np.random.default_rng(4)
    x, w, res = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal((3, 4))
    want = np.array([[sum(x[i, k] * w[j, k] for k in range(5)) for j in range(4)] for i in range(3)])
    np.testing.assert_allclose(orc.linear(x, w), want, rtol=1e-13)
    np.testing.assert_allclose(orc.linear(x, w, res), want + res, rtol=1e-13)


def test_silu_mul_closed_forms(orc):
    g = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    gu = np.concatenate([g, np.full(5, 2.0)])[None, :]
    out = orc.silu_mul(gu)[0]
    want = 2.0 * np.array([0.0, 1.0 / (1.0 + math.exp(-1.0)), -1.0 / (1.0 + math.e), 40.0, 0.0])
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-15)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(50)
    s = orc.silu_mul(np.concatenate([x, np.ones(50)]))
    sn = orc.silu_mul(np.concatenate([-x, np.ones(50)]))
    np.testing.assert_allclose(s - sn, x, atol=1e-14)  # silu(x) - silu(-x) = x


def _layer_case(orc, syn, zero_wo=False, zero_wd=False, seed=8):
    rng = np.random.default_rng(seed)
    H, Hq, D, d, f = 2, 4, 64, 128, 96
    ns = [40, 24]
    chunks = [(syn.chunk(seed, syn.K, b, 1, n, H, D, "bf16")[0], syn.chunk(seed, syn.V, b, 1, n, H, D, "bf16")[0])
              for b, n in enumerate(ns)]
    sel = [np.array([1, 7, 8, 30]), np.array([0, 23])]
    offsets = [0, 40]
    sfx_start, n_sfx = 64, 3
    qpos = np.concatenate([offsets[b] + s for b, s in enumerate(sel)] + [np.arange(sfx_start, sfx_start + n_sfx)])
    n_q = len(qpos)
    r = lambda a: orc.widen(orc.bf16_bits(a))  # noqa: E731
    w = dict(g1=r(rng.uniform(0.5, 1.5, d)), g2=r(rng.uniform(0.5, 1.5, d)),
             wq=r(rng.standard_normal((Hq * D, d)) / math.sqrt(d)),
             wk=r(rng.standard_normal((H * D, d)) / math.sqrt(d)),
             wv=r(rng.standard_normal((H * D, d)) / math.sqrt(d)),
             wo=np.zeros((d, Hq * D)) if zero_wo else r(rng.standard_normal((d, Hq * D)) / math.sqrt(Hq * D)),
             wgu=r(rng.standard_normal((2 * f, d)) / math.sqrt(d)),
             wd=np.zeros((d, f)) if zero_wd else r(rng.standard_normal((d, f)) / math.sqrt(f)))
    h = r(rng.standard_normal((n_q, d)))
    out, mid = orc.recompute_layer(h, w, chunks, sel, offsets, sfx_start, qpos, H, Hq, D, 500000.0, 1e-5)
    return h, w, chunks, sel, offsets, sfx_start, qpos, out, mid


def test_layer_residual_paths(orc, syn):
    # with both output projections zero the layer is the identity on h
    h, *_, out, mid = _layer_case(orc, syn, zero_wo=True, zero_wd=True)
    np.testing.assert_array_equal(out, h)
    np.testing.assert_array_equal(mid["h1"], h)
    # with only the MLP's down projection zero, the output is h1 = h + attention part
    h, *_, out, mid = _layer_case(orc, syn, zero_wd=True)
    np.testing.assert_array_equal(out, mid["h1"])
    assert np.abs(mid["h1"] - h).max() > 1e-3


def test_layer_routes_recomputed_rows(orc, syn):
    h, w, chunks, sel, offsets, sfx_start, qpos, out, mid = _layer_case(orc, syn)
    H, D = 2, 64
    k_asm = orc.widen(mid["k_asm"])
    v_asm = orc.widen(mid["v_asm"])
    kr = mid["k"].reshape(-1, H, D)
    vr = mid["v"].reshape(-1, H, D)
    # V is not rotated: each recomputed (selected or suffix) row lands at its
    # global position, every other row is the cached one
    for i, p in enumerate(qpos):
        np.testing.assert_array_equal(v_asm[p], vr[i])
    reused = np.setdiff1d(np.arange(sfx_start), qpos)
    for p in reused:
        b = 0 if p < 40 else 1
        np.testing.assert_array_equal(v_asm[p], orc.widen(chunks[b][1][p - offsets[b]]))
    # K is rotated at the global position: norms per head are kept (to bf16 rounding)
    for i, p in enumerate(qpos):
        np.testing.assert_allclose(np.linalg.norm(k_asm[p], axis=-1), np.linalg.norm(kr[i], axis=-1), rtol=1e-2)

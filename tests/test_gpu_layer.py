"""GPU parity of the rest of the selective-recompute layer (synthetic weights)
against the oracle: RMSNorm, the gated activation, the projections, and one
composed decoder layer over the assembled cache.  Calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

from gpu_util import need_gpu, to_dev, to_host, widen

pytestmark = pytest.mark.gpu


def _bf16(orc, a):
    return orc.bf16_bits(a)


def _within_rounding(got_bits, exact, slack):
    """A result rounded once to bf16 lies within half an ulp (2^-8 relative) of
    the exact value, plus the fp32 arithmetic's own error `slack`."""
    got = widen(got_bits)
    err = np.abs(got - exact)
    bound = 2.0 ** -8 * np.abs(exact) + slack
    assert (err <= bound).all(), f"max excess {np.max(err - bound)}"


@pytest.mark.parametrize("rows,dim", [(37, 4096), (5, 136), (1, 8), (0, 64)])
def test_rmsnorm(orc, rows, dim):
    ct = need_gpu()
    rng = np.random.default_rng(rows + dim)
    x = _bf16(orc, 2.0 * rng.standard_normal((max(rows, 1), dim)))[:rows]
    g = _bf16(orc, rng.uniform(0.5, 1.5, dim))
    out = ct.cachetune_rmsnorm(to_dev(x) if rows else torch.zeros((0, dim), dtype=torch.bfloat16, device="cuda"),
                               to_dev(g), eps=1e-5)
    torch.cuda.synchronize()
    if rows == 0:
        return
    exact = orc.rmsnorm(widen(x), widen(g), 1e-5)
    _within_rounding(to_host(out), exact, 1e-5 * np.abs(exact) + 1e-30)


@pytest.mark.parametrize("rows,ff", [(19, 14336), (3, 8)])
def test_silu_mul(orc, rows, ff):
    ct = need_gpu()
    rng = np.random.default_rng(rows + ff)
    gu = _bf16(orc, 3.0 * rng.standard_normal((rows, 2 * ff)))
    gu[0, :4] = _bf16(orc, np.array([0.0, 60.0, -60.0, -100.0]))  # silu's flat and linear ends
    out = ct.cachetune_silu_mul(to_dev(gu))
    torch.cuda.synchronize()
    exact = orc.silu_mul(widen(gu))
    _within_rounding(to_host(out), exact, 1e-6 * np.abs(exact) + 1e-30)


@pytest.mark.parametrize("m,n,k,res", [(77, 256, 512, True), (3, 8, 8, False), (130, 1024, 4096, False),
                                       (2584, 1024, 4096, True), (200, 264, 40, True),
                                       # the 8 x 2048 workload's gate/up and down projections
                                       (2584, 28672, 4096, False), (2584, 4096, 14336, True)])
def test_linear(orc, syn, m, n, k, res):
    """Bias-free projection with fp32 accumulation: each output within half a
    bf16 ulp of the exact sum plus 2^-16 of sum_k |x_k w_k| (fp32 accumulation
    error, with room over its random-walk size and under its worst case
    k 2^-24).  Large shapes are checked on sampled rows."""
    ct = need_gpu()
    rng = np.random.default_rng(m + n + k)
    x = syn.normal(m + n, 1, (m, k), "bf16")
    w = syn.normal(m + n, 2, (n, k), "bf16", sigma=1.0 / math.sqrt(k))
    r = _bf16(orc, rng.standard_normal((m, n))) if res else None
    out = ct.cachetune_linear(to_dev(x), to_dev(w), to_dev(r) if res else None)
    torch.cuda.synchronize()
    got = to_host(out)
    rows = np.arange(m) if m * n * k <= 2e8 else np.sort(rng.choice(m, 48, replace=False))
    xs, ws_ = widen(x[rows]), widen(w)
    exact = orc.linear(xs, ws_, widen(r[rows]) if res else None)
    slack = 2.0 ** -16 * (np.abs(xs) @ np.abs(ws_).T)
    _within_rounding(got[rows], exact, slack)


@pytest.mark.parametrize("m,d,nq,nkv", [(2584, 4096, 4096, 1024), (45, 256, 256, 128), (3, 64, 16, 8)])
def test_qkv_proj(orc, syn, m, d, nq, nkv):
    """Fused q / k / v projection: one product with the stacked weights, its
    columns split over three buffers; each against the oracle's projection."""
    ct = need_gpu()
    x = syn.normal(m + d, 3, (m, d), "bf16")
    w = syn.normal(m + d, 4, (nq + 2 * nkv, d), "bf16", sigma=1.0 / math.sqrt(d))
    q, k, v = ct.cachetune_qkv_proj(to_dev(x), to_dev(w), nq, nkv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(m)
    rows = np.arange(m) if m <= 64 else np.sort(rng.choice(m, 48, replace=False))
    xs = widen(x[rows])
    for got, lo, hi in ((q, 0, nq), (k, nq, nq + nkv), (v, nq + nkv, nq + 2 * nkv)):
        ws_ = widen(w[lo:hi])
        exact = orc.linear(xs, ws_)
        _within_rounding(to_host(got)[rows], exact, 2.0 ** -16 * (np.abs(xs) @ np.abs(ws_).T))


def test_linear_in_place_residual(orc):
    ct = need_gpu()
    rng = np.random.default_rng(2)
    x = _bf16(orc, rng.standard_normal((64, 128)))
    w = _bf16(orc, rng.standard_normal((256, 128)) / math.sqrt(128))
    h = _bf16(orc, rng.standard_normal((64, 256)))
    hd = to_dev(h)
    ct.cachetune_linear(to_dev(x), to_dev(w), residual=hd, out=hd)
    torch.cuda.synchronize()
    exact = orc.linear(widen(x), widen(w), widen(h))
    _within_rounding(to_host(hd), exact, 2.0 ** -16 * (np.abs(widen(x)) @ np.abs(widen(w)).T))


def test_composed_layer(orc, syn):
    """One decoder layer for the recomputed rows, GPU calls chained as a layer
    runs them, against the oracle's layer in the same bf16 storage.  Both sides
    round every stored intermediate; a rounding that lands on the other side of
    a tie, and the attention's own tolerance, make the two differ slightly, so
    the final rows are compared at 3 % of their rms plus 2^-7 relative."""
    ct = need_gpu()
    rng = np.random.default_rng(8)
    H, Hq, D, d, f, theta, eps = 2, 4, 64, 256, 512, 500000.0, 1e-5
    ns = [300, 129]
    offsets = [0, 300]
    sfx_start, n_sfx = 429, 16
    chunks, sel = [], []
    for b, n in enumerate(ns):
        chunks.append((syn.chunk(8, syn.K, b, 1, n, H, D, "bf16")[0], syn.chunk(8, syn.V, b, 1, n, H, D, "bf16")[0]))
        sel.append(np.sort(rng.choice(n, orc.ksel(n, 15, 100), replace=False)).astype(np.int32))
    qpos = np.concatenate([offsets[b] + s for b, s in enumerate(sel)] + [np.arange(sfx_start, sfx_start + n_sfx)])
    qpos = qpos.astype(np.int32)
    n_q = len(qpos)
    r = lambda a: widen(_bf16(orc, a))  # noqa: E731
    w = dict(g1=r(rng.uniform(0.5, 1.5, d)), g2=r(rng.uniform(0.5, 1.5, d)),
             wq=r(rng.standard_normal((Hq * D, d)) / math.sqrt(d)),
             wk=r(rng.standard_normal((H * D, d)) / math.sqrt(d)),
             wv=r(rng.standard_normal((H * D, d)) / math.sqrt(d)),
             wo=r(rng.standard_normal((d, Hq * D)) / math.sqrt(Hq * D)),
             wgu=r(rng.standard_normal((2 * f, d)) / math.sqrt(d)),
             wd=r(rng.standard_normal((d, f)) / math.sqrt(f)))
    h = r(rng.standard_normal((n_q, d)))
    want, mid = orc.recompute_layer(h, w, chunks, sel, offsets, sfx_start, qpos, H, Hq, D, theta, eps)

    dv = {kname: to_dev(_bf16(orc, v)) for kname, v in w.items()}
    hd = to_dev(_bf16(orc, h))
    x1 = ct.cachetune_rmsnorm(hd, dv["g1"], eps)
    q = ct.cachetune_linear(x1, dv["wq"])
    kr = ct.cachetune_linear(x1, dv["wk"])
    vr = ct.cachetune_linear(x1, dv["wv"])
    T = sfx_start + n_sfx
    k_asm = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    v_asm = torch.zeros((T, H, D), dtype=torch.bfloat16, device="cuda")
    places, keep, row = [], [], 0
    for b, n in enumerate(ns):
        k = len(sel[b])
        comp = np.setdiff1d(np.arange(n, dtype=np.int32), sel[b]).astype(np.int32)
        dd = dict(k_src=to_dev(chunks[b][0]), v_src=to_dev(chunks[b][1]), comp=to_dev(comp), sel=to_dev(sel[b]),
                  k_rec=kr[row:row + k].view(k, H, D), v_rec=vr[row:row + k].view(k, H, D))
        keep.append(dd)
        places.append(ct.make_place(n=n, k=k, offset=offsets[b], **dd))
        row += k
    ct.cachetune_assemble_rope(places, k_asm, v_asm, H, D, theta, k_sfx=kr[row:].view(n_sfx, H, D),
                               v_sfx=vr[row:].view(n_sfx, H, D), n_sfx=n_sfx, sfx_offset=sfx_start)
    o, _ = ct.cachetune_recompute_attn(q.view(n_q, Hq, D), to_dev(qpos), k_asm, v_asm, 1.0 / math.sqrt(D), theta)
    h1 = ct.cachetune_linear(o.view(n_q, Hq * D), dv["wo"], residual=hd)
    x2 = ct.cachetune_rmsnorm(h1, dv["g2"], eps)
    gu = ct.cachetune_linear(x2, dv["wgu"])
    a = ct.cachetune_silu_mul(gu)
    h2 = ct.cachetune_linear(a, dv["wd"], residual=h1)
    torch.cuda.synchronize()
    got = widen(to_host(h2))
    # the first stages match to rounding
    _within_rounding(to_host(x1), orc.rmsnorm(h, w["g1"], eps), 1e-5 * np.abs(h).max())
    rms = np.sqrt((want ** 2).mean())
    err = np.abs(got - want)
    assert (err <= 0.03 * rms + 2.0 ** -7 * np.abs(want)).all(), f"max err {err.max()} (rms {rms})"

"""The host-tier pipeline as it runs (CacheTune page, Sec. 4.2 and App. B.2,
"Sparse KV Reuse Pipeline"), at the full size of the host-tier workload:
32 chunks x 2048 tokens of Llama-3-8B-shaped bf16 K/V (32 layers, 32 Q / 8 KV
heads x 128) in a rank-ordered pinned host pool, a 128-token suffix.

``HostTierPipeline.request`` stages each layer's complement on a copy stream
into one of two staging buffers, ordered by events against the assembly and
attention on the compute stream.  Its per-layer outputs (assembled K and V,
attention output) must equal, bit for bit, the same calls made in order on
one stream with the chunks resident on the device (the complement read by
index), for two requests in a row (the second reuses the staging buffers
across requests).  Sampled layers are also checked against the oracle: the
assembled layer (V bit-exact, K within 1 ulp) and sampled attention rows.

The full-layer variant adds, per layer, RMSNorm and the fused q/k/v projection
before the wait for the transfer and the output projection and gated MLP after
the attention; the recomputed rows and queries come from the layer's own
projection.  Its final hidden rows and every layer's attention output must
equal the serial composed layer's bit for bit."""
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_rotated_keys, check_index_sets, half_ulp_bf16, need_gpu, to_dev, to_host, widen

pytestmark = pytest.mark.gpu

SEED, NB, N, L, H, HQ, D = 20260525, 32, 2048, 32, 8, 32, 128
THETA, N_SFX = 500000.0, 128
T_C = NB * N
T = T_C + N_SFX
OFFS = [b * N for b in range(NB)]


@pytest.fixture(scope="module")
def pool_state(syn):
    """Host chunks, device chunks, scores, stored ranking, the pinned pool."""
    ct = need_gpu()
    from non_prefix_kv_token_amd.hosttier import build_host_pool
    print(f"[hosttier] generating {NB} x {N} x {L} layers", flush=True)
    host = [(syn.chunk(SEED, syn.K, b, L, N, H, D, "bf16"), syn.chunk(SEED, syn.V, b, L, N, H, D, "bf16"))
            for b in range(NB)]
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    score, _ = ct.cachetune_score_chunk(dev, L, H, D, alpha=(1, 16))
    ns = [N] * NB
    ranking = torch.empty(T_C, dtype=torch.int32, device="cuda")
    ct.cachetune_select_topr(score, ns, r=(15, 100), ranking=ranking)
    pool = build_host_pool(dev, ranking, ns)
    print("[hosttier] pool ready", flush=True)
    return ct, host, dev, score, ranking, pool


def _select(ct, score, r):
    ns = [N] * NB
    ks, ranking, sel, comp = ct.cachetune_select_topr(score, ns, r=r)
    torch.cuda.synchronize()
    sl = to_host(sel)
    so = np.cumsum([0] + ks)
    return ks, sel, comp, [sl[so[b]:so[b + 1]] for b in range(NB)]


def _qpos(sel_list):
    return np.sort(np.concatenate([OFFS[b] + sel_list[b] for b in range(NB)] +
                                  [np.arange(T_C, T)])).astype(np.int32)


def _serial_places(ct, dev, l, ks, sel, comp, rec):
    places, so, co = [], 0, 0
    for b in range(NB):
        k = ks[b]
        kr, vr = rec(l, b) if k else (None, None)
        places.append(ct.make_place(dev[b][0][l], dev[b][1][l], N, k, OFFS[b], sel=sel[so:] if k else None,
                                    comp=comp[co:] if k < N else None, k_rec=kr, v_rec=vr))
        so, co = so + k, co + N - k
    return places


def test_host_tier_pipeline_full_size(orc, syn, pool_state):
    ct, host, dev, score, ranking, pool = pool_state
    from non_prefix_kv_token_amd.hosttier import HostTierPipeline
    r = (15, 100)
    ks, sel, comp, sel_list = _select(ct, score, r)
    assert ks == [307] * NB
    s_h = to_host(score)
    for b in (0, NB - 1):  # the selection itself against the oracle (sampled chunks)
        s_orc = orc.score_chunk(host[b][0], host[b][1], 1, 16)
        assert np.all(np.abs(s_h[b * N:(b + 1) * N] - s_orc) <= 1e-4 * s_orc)
        check_index_sets(sel_list[b], orc.topr(s_orc, ks[b])[1], s_orc, ks[b])
    qpos = _qpos(sel_list)
    n_q = len(qpos)
    # recomputed rows (cached rows + seeded noise), suffix rows and queries of every layer
    rec_h = [[(syn.rows(SEED, syn.K, b, l, N, H, D, sel_list[b], "bf16", extra_sigma=0.25),
               syn.rows(SEED, syn.V, b, l, N, H, D, sel_list[b], "bf16", extra_sigma=0.25))
              for b in range(NB)] for l in range(L)]
    rec_d = [[(to_dev(kr), to_dev(vr)) for kr, vr in layer] for layer in rec_h]
    idx = np.arange(N_SFX)
    sfx_h = [(syn.rows(SEED, syn.K, syn.SUFFIX_CHUNK, l, N_SFX, H, D, idx, "bf16"),
              syn.rows(SEED, syn.V, syn.SUFFIX_CHUNK, l, N_SFX, H, D, idx, "bf16")) for l in range(L)]
    sfx_d = [(to_dev(a), to_dev(b_)) for a, b_ in sfx_h]
    owner = np.where(qpos < T_C, qpos // N, -1)
    local = np.where(qpos < T_C, qpos % N, qpos - T_C)
    check_layers = (0, 17, L - 1)
    q_h = {}
    q_d = []
    for l in range(L):
        q = np.empty((n_q, HQ, D), np.uint16)
        for b in np.unique(owner):
            m = owner == b
            q[m] = syn.rows(SEED, syn.Q, syn.SUFFIX_CHUNK if b < 0 else int(b), l, N_SFX if b < 0 else N, HQ, D,
                            local[m], "bf16")
        if l in check_layers:
            q_h[l] = q
        q_d.append(to_dev(q))
    qpos_d = to_dev(qpos)
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(max(256, ct.cachetune_recompute_attn_ws(n_q, HQ, T, H, D)), dtype=torch.uint8, device="cuda")
    k_asm = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    v_asm = torch.empty_like(k_asm)
    out = torch.empty((n_q, HQ, D), dtype=torch.bfloat16, device="cuda")
    rec = lambda l, b: rec_d[l][b]  # noqa: E731

    # serial reference: device-resident chunks, one stream
    ref = []
    for l in range(L):
        ct.cachetune_assemble_rope(_serial_places(ct, dev, l, ks, sel, comp, rec), k_asm, v_asm, H, D, THETA,
                                   k_sfx=sfx_d[l][0], v_sfx=sfx_d[l][1], n_sfx=N_SFX, sfx_offset=T_C)
        ct.cachetune_recompute_attn(q_d[l], qpos_d, k_asm, v_asm, scale, THETA, out=out, ws=ws)
        ref.append((k_asm.clone(), v_asm.clone(), out.clone()))
    torch.cuda.synchronize()
    print("[hosttier] serial reference done", flush=True)

    pipe = HostTierPipeline(pool, ranking, [N] * NB, ks, OFFS, sel, rec, lambda l: sfx_d[l], N_SFX, THETA)
    assert pipe.h2d_bytes() == 2 * NB * (N - 307) * H * D * 2 * L
    for rep in range(2):
        got = []

        def attend(l, ka, va):
            ct.cachetune_recompute_attn(q_d[l], qpos_d, ka, va, scale, THETA, out=out, ws=ws)
            got.append((ka.clone(), va.clone(), out.clone()))

        pipe.request(k_asm, v_asm, attend)
        torch.cuda.synchronize()
        assert len(got) == L
        for l in range(L):
            for a, b_ in zip(got[l], ref[l]):
                assert torch.equal(a, b_), (rep, l)
        print(f"[hosttier] request {rep}: all {L} layers equal the serial path", flush=True)

    # oracle: sampled layers' assembly and attention rows
    rng = np.random.default_rng(55)
    for l in check_layers:
        k_ref = np.zeros((T, H, D), np.uint16)
        v_ref = np.zeros((T, H, D), np.uint16)
        for b in range(NB):
            orc.assemble_chunk(host[b][0][l], host[b][1][l], rec_h[l][b][0], rec_h[l][b][1], sel_list[b], OFFS[b],
                               THETA, 0, k_ref, v_ref)
        orc.assemble_rows(sfx_h[l][0], sfx_h[l][1], T_C, THETA, 0, k_ref, v_ref)
        kg, vg, og = (to_host(x) for x in ref[l])
        np.testing.assert_array_equal(vg, v_ref)
        assert_rotated_keys(kg, k_ref)
        rows = np.unique(np.concatenate([[0, n_q - 1], rng.choice(n_q, 10, replace=False)])).astype(np.int32)
        o_ref, _ = orc.attention(q_h[l], qpos, k_ref, v_ref, scale, THETA, rows=rows)
        err = np.abs(widen(og)[rows] - o_ref)
        assert (err <= 2e-2 + half_ulp_bf16(o_ref)).all(), (l, err.max())
        print(f"[hosttier] layer {l}: oracle assembly and {len(rows)} attention rows ok", flush=True)


def test_host_tier_full_layer_pipeline(syn, pool_state):
    """The full-layer variant against the serial composed layer, bit for bit."""
    ct, host, dev, score, ranking, pool = pool_state
    from non_prefix_kv_token_amd.hosttier import HostTierPipeline
    ks, sel, comp, sel_list = _select(ct, score, (10, 100))
    qpos = _qpos(sel_list)
    n_q = len(qpos)
    d_model, d_ff, wseed = HQ * D, 14336, 20260601
    wgen = lambda stream, shape, sigma, mean=0.0: to_dev(syn.normal(wseed, stream, shape, "bf16", mean, sigma))  # noqa: E731
    g1, g2 = wgen(1, (d_model,), 0.1, 1.0), wgen(2, (d_model,), 0.1, 1.0)
    wqkv = wgen(3, ((HQ + 2 * H) * D, d_model), d_model ** -0.5)
    wo = wgen(6, (d_model, HQ * D), (HQ * D) ** -0.5)
    wgu = wgen(7, (2 * d_ff, d_model), d_model ** -0.5)
    wd = wgen(8, (d_model, d_ff), d_ff ** -0.5)
    h0 = to_dev(syn.normal(wseed, 9, (n_q, d_model), "bf16"))
    bf = torch.bfloat16
    mk = lambda n: torch.empty((n_q, n), dtype=bf, device="cuda")  # noqa: E731
    hb, h1b, xb = mk(d_model), mk(d_model), mk(d_model)
    qb, krb, vrb = mk(HQ * D), mk(H * D), mk(H * D)
    gub, ab = mk(2 * d_ff), mk(d_ff)
    row0 = [int(np.searchsorted(qpos, OFFS[b])) for b in range(NB)]
    rec = lambda l, b: (krb[row0[b]:row0[b] + ks[b]].view(ks[b], H, D),  # noqa: E731
                        vrb[row0[b]:row0[b] + ks[b]].view(ks[b], H, D))
    s0 = n_q - N_SFX
    sfx = lambda l: (krb[s0:].view(N_SFX, H, D), vrb[s0:].view(N_SFX, H, D))  # noqa: E731
    qpos_d = to_dev(qpos)
    scale = 1.0 / math.sqrt(D)
    ws = torch.empty(max(256, ct.cachetune_recompute_attn_ws(n_q, HQ, T, H, D)), dtype=torch.uint8, device="cuda")
    k_asm = torch.empty((T, H, D), dtype=bf, device="cuda")
    v_asm = torch.empty_like(k_asm)
    out = torch.empty((n_q, HQ, D), dtype=bf, device="cuda")

    def before_wait(l):
        ct.cachetune_rmsnorm(hb, g1, 1e-5, out=xb)
        ct.cachetune_qkv_proj(xb, wqkv, HQ * D, H * D, q=qb, k=krb, v=vrb)

    def after_attend(l):
        ct.cachetune_linear(out.view(n_q, HQ * D), wo, residual=hb, out=h1b)
        ct.cachetune_rmsnorm(h1b, g2, 1e-5, out=xb)
        ct.cachetune_linear(xb, wgu, out=gub)
        ct.cachetune_silu_mul(gub, out=ab)
        ct.cachetune_linear(ab, wd, residual=h1b, out=hb)

    # serial composed layer, device-resident chunks
    hb.copy_(h0)
    ref_out = []
    for l in range(L):
        before_wait(l)
        ct.cachetune_assemble_rope(_serial_places(ct, dev, l, ks, sel, comp, rec), k_asm, v_asm, H, D, THETA,
                                   k_sfx=sfx(l)[0], v_sfx=sfx(l)[1], n_sfx=N_SFX, sfx_offset=T_C)
        ct.cachetune_recompute_attn(qb.view(n_q, HQ, D), qpos_d, k_asm, v_asm, scale, THETA, out=out, ws=ws)
        ref_out.append(out.clone())
        after_attend(l)
    h_ref = hb.clone()
    torch.cuda.synchronize()
    assert torch.isfinite(h_ref.float()).all()

    pipe = HostTierPipeline(pool, ranking, [N] * NB, ks, OFFS, sel, rec, sfx, N_SFX, THETA)
    for rep in range(2):
        got = []

        def attend(l, ka, va):
            ct.cachetune_recompute_attn(qb.view(n_q, HQ, D), qpos_d, ka, va, scale, THETA, out=out, ws=ws)
            got.append(out.clone())

        hb.copy_(h0)
        pipe.request(k_asm, v_asm, attend, before_wait=before_wait, after_attend=after_attend)
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(got[l], ref_out[l]), (rep, l)
        assert torch.equal(hb, h_ref), rep
        print(f"[hosttier] full-layer request {rep}: equal to the serial composed layer", flush=True)

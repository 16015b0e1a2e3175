"""GPU parity at the measured workloads' full sizes, in the launch configuration
bench.py times, on outputs the oracle computes one by one:

* 1 x 512 tokens, fp32, L=1 (the small workload): everything, end to end;
* 8 x 2048 tokens, Llama-3-8B-shaped (32 layers, 32 Q / 8 KV heads x 128),
  bf16: scores of sampled chunks over all 32 layers, their top-r sets, one
  whole assembled layer, sampled attention rows (all query heads);
* 16 x 2048 tokens in a seeded random order: the r sweep {5,10,15,20,30}% from
  one stored ranking, assembly at the shuffled offsets, sampled attention;
* 64 chunks of seeded lengths in [512, 4096], Qwen3-4B-shaped (36 layers),
  cutoff 1/32: scores of every chunk (two launches of 32 chunks), sampled
  chunks against the oracle, assembly and sampled attention at T ~ 147K
  (RoPE angles at positions up to ~1.5e5).

Tolerances as in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

from gpu_util import (LSE_TOL, assert_rotated_keys, check_index_sets, half_ulp_bf16, need_gpu, to_dev, to_host,
                      widen)

pytestmark = pytest.mark.gpu


def _score_chunks(ct, syn, seed, ns, L, H, D, dtype, alpha):
    host = [(syn.chunk(seed, syn.K, b, L, n, H, D, dtype), syn.chunk(seed, syn.V, b, L, n, H, D, dtype))
            for b, n in enumerate(ns)]
    dev = [(to_dev(k), to_dev(v)) for k, v in host]
    score, _ = ct.cachetune_score_chunk(dev, L, H, D, alpha=alpha)
    torch.cuda.synchronize()
    return host, dev, to_host(score)


def _check_scores(orc, host, s_gpu, ns, idx, alpha):
    """Oracle scores of the sampled chunks; returns them keyed by chunk."""
    out = {}
    for b in idx:
        o = sum(ns[:b])
        k, v = host[b]
        s = orc.score_chunk(k, v, *alpha)
        got = s_gpu[o:o + ns[b]].astype(np.float64)
        assert np.all(np.abs(got - s) <= 1e-4 * s), (b, np.max(np.abs(got - s) / s))
        out[b] = s
    return out


def _request(ct, syn, seed, ns, offs, layer, H, D, dtype, sel_list, comp_d, sel_d, theta, n_sfx,
             T, dev_layer):
    """Places of one layer (device chunks, complement + recomputed rows) plus
    the suffix; returns (k_out, v_out, oracle inputs)."""
    places, keep, rec = [], [], []
    so = co = 0
    for b, n in enumerate(ns):
        s_b = sel_list[b]
        k = len(s_b)
        kr = syn.rows(seed, syn.K, b, layer, n, H, D, s_b, dtype, extra_sigma=0.25)
        vr = syn.rows(seed, syn.V, b, layer, n, H, D, s_b, dtype, extra_sigma=0.25)
        rec.append((kr, vr))
        d = dict(sel=sel_d[so:] if k else None, k_rec=to_dev(kr) if k else None,
                 v_rec=to_dev(vr) if k else None, comp=comp_d[co:] if k < n else None)
        keep.append(d)
        places.append(ct.make_place(dev_layer[b][0], dev_layer[b][1], n, k, int(offs[b]), **d))
        so, co = so + k, co + n - k
    idx = np.arange(n_sfx)
    ksf = syn.rows(seed, syn.K, syn.SUFFIX_CHUNK, layer, n_sfx, H, D, idx, dtype)
    vsf = syn.rows(seed, syn.V, syn.SUFFIX_CHUNK, layer, n_sfx, H, D, idx, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k_out = torch.zeros((T, H, D), dtype=tdt, device="cuda")
    v_out = torch.zeros_like(k_out)
    ct.cachetune_assemble_rope(places, k_out, v_out, H, D, theta, k_sfx=to_dev(ksf), v_sfx=to_dev(vsf),
                               n_sfx=n_sfx, sfx_offset=T - n_sfx)
    torch.cuda.synchronize()
    return k_out, v_out, rec, (ksf, vsf), keep


def _oracle_layer(orc, host_layer, rec, sfx, sel_list, offs, T, H, D, dtype, theta, n_sfx):
    edt = np.uint16 if dtype == "bf16" else np.float32
    k_ref = np.zeros((T, H, D), edt)
    v_ref = np.zeros((T, H, D), edt)
    for b, (k, v) in enumerate(host_layer):
        orc.assemble_chunk(k, v, rec[b][0], rec[b][1], sel_list[b], int(offs[b]), theta, 0, k_ref, v_ref)
    orc.assemble_rows(sfx[0], sfx[1], T - n_sfx, theta, 0, k_ref, v_ref)
    return k_ref, v_ref


def _queries(syn, seed, ns, offs, layer, Hq, D, dtype, qpos, T_c, n_sfx):
    owner = np.full(qpos.shape, -1)
    local = qpos - T_c
    for b, n in enumerate(ns):
        m = (qpos >= offs[b]) & (qpos < offs[b] + n)
        owner[m] = b
        local[m] = qpos[m] - offs[b]
    q = np.empty((len(qpos), Hq, D), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in set(owner.tolist()):
        m = owner == b
        chunk = syn.SUFFIX_CHUNK if b < 0 else b
        n = n_sfx if b < 0 else ns[b]
        q[m] = syn.rows(seed, syn.Q, chunk, layer, n, Hq, D, local[m], dtype)
    return q


def _check_attention(ct, orc, q, qpos, k_out, v_out, k_ref, v_ref, theta, rows, dtype):
    D = q.shape[2]
    scale = 1.0 / np.sqrt(D)
    out, lse = ct.cachetune_recompute_attn(to_dev(q), to_dev(qpos), k_out, v_out, scale, theta,
                                           want_lse=True)
    torch.cuda.synchronize()
    og, lg = widen(to_host(out)), to_host(lse).astype(np.float64)
    ref, lref = orc.attention(q, qpos, k_ref, v_ref, scale, theta, rows=rows)
    err = np.abs(og[rows] - ref)
    tol = 2e-2 + (half_ulp_bf16(ref) if dtype == "bf16" else 0.0)
    assert (err <= tol).all(), (err.max(), (err - tol).max())
    assert (np.abs(lg[rows] - lref) <= LSE_TOL).all(), np.abs(lg[rows] - lref).max()


def _rows_sample(n_q, rng, count):
    return np.unique(np.concatenate([[0, n_q - 1], rng.choice(n_q, count - 2, replace=False)])).astype(np.int32)


def test_workload_1x512_fp32_end_to_end(orc, syn):
    ct = need_gpu()
    seed, ns, L, H, Hq, D, theta, n_sfx = 20260521, [512], 1, 8, 8, 64, 10000.0, 16
    host, dev, s_gpu = _score_chunks(ct, syn, seed, ns, L, H, D, "f32", (1, 16))
    s_orc = _check_scores(orc, host, s_gpu, ns, [0], (1, 16))[0]
    ks, ranking, sel, comp = ct.cachetune_select_topr(to_dev(s_gpu), ns, r=(15, 100))
    torch.cuda.synchronize()
    assert ks == [76]
    check_index_sets(to_host(sel)[:76], orc.topr(s_orc, 76)[1], s_orc, 76)
    sel_list = [to_host(sel)[:76]]
    T = 512 + n_sfx
    k_out, v_out, rec, sfx, _ = _request(ct, syn, seed, ns, [0], 0, H, D, "f32", sel_list, comp, sel,
                                         theta, n_sfx, T, [(dev[0][0][0], dev[0][1][0])])
    k_ref, v_ref = _oracle_layer(orc, [(host[0][0][0], host[0][1][0])], rec, sfx, sel_list, [0], T, H,
                                 D, "f32", theta, n_sfx)
    np.testing.assert_array_equal(to_host(v_out), v_ref)
    kd = np.abs(widen(to_host(k_out)) - widen(k_ref))
    assert kd.max() <= 1e-6 * np.abs(widen(k_ref)).max()
    qpos = np.sort(np.concatenate([sel_list[0], np.arange(512, T)])).astype(np.int32)
    q = _queries(syn, seed, ns, [0], 0, Hq, D, "f32", qpos, 512, n_sfx)
    _check_attention(ct, orc, q, qpos, k_out, v_out, k_ref, v_ref, theta, np.arange(len(qpos)), "f32")


@pytest.mark.parametrize("shuffle", [False, True])
def test_workload_llama3_8b(orc, syn, shuffle):
    """8 x 2048 in stored order: the scores and index sets of every chunk, one
    assembled layer, every attention row and query head of that layer.
    16 x 2048 in a seeded random order: the r sweep on sampled chunks, then
    one layer's assembly and attention at r = 15 % (every row and head) and at
    r = 30 % (sampled rows)."""
    ct = need_gpu()
    nb = 16 if shuffle else 8
    seed = 20260523 if shuffle else 20260522
    ns, L, H, Hq, D, theta, n_sfx = [2048] * nb, 32, 8, 32, 128, 500000.0, 128
    rng = np.random.default_rng(nb)
    host, dev, s_gpu = _score_chunks(ct, syn, seed, ns, L, H, D, "bf16", (1, 16))
    sample = [0, 5, 10, nb - 3] if shuffle else list(range(nb))
    s_orc = _check_scores(orc, host, s_gpu, ns, sample, (1, 16))
    print(f"[workload] scores of {len(sample)} chunks match the oracle", flush=True)
    # selection: every r of the sweep cuts the same stored ranking (App. B.1)
    r_list = [(5, 100), (10, 100), (15, 100), (20, 100), (30, 100)] if shuffle else [(15, 100)]
    prev = None
    sels = {}
    for r in r_list:
        ks, ranking, sel, comp = ct.cachetune_select_topr(to_dev(s_gpu), ns, r=r)
        torch.cuda.synchronize()
        rk, sl = to_host(ranking), to_host(sel)
        if prev is not None:
            assert np.array_equal(rk, prev)
        prev = rk
        for b in sample:
            k = ks[b]
            check_index_sets(sl[sum(ks[:b]):sum(ks[:b]) + k], orc.topr(s_orc[b], k)[1], s_orc[b], k)
        for b in range(nb):  # the set is the sorted head of the stored ranking
            o = b * 2048
            assert np.array_equal(np.sort(rk[o:o + ks[b]]), sl[sum(ks[:b]):sum(ks[:b]) + ks[b]])
        sels[r] = (ks, sel, comp, sl)
    # chunk order and offsets
    import synth
    order = synth.permutation(seed, 0, nb) if shuffle else np.arange(nb)
    offs = np.zeros(nb, np.int64)
    pos = 0
    for p in range(nb):
        offs[order[p]] = pos
        pos += ns[order[p]]
    T_c, T = pos, pos + n_sfx
    layer = 5
    checks = [((15, 100), None), ((30, 100), 24)] if shuffle else [((15, 100), None)]
    for r, n_rows in checks:
        ks, sel, comp, sl = sels[r]
        sel_list = [sl[sum(ks[:b]):sum(ks[:b]) + ks[b]] for b in range(nb)]
        k_out, v_out, rec, sfx, _ = _request(ct, syn, seed, ns, offs, layer, H, D, "bf16", sel_list, comp,
                                             sel, theta, n_sfx, T, [(k[layer], v[layer]) for k, v in dev])
        k_ref, v_ref = _oracle_layer(orc, [(k[layer], v[layer]) for k, v in host], rec, sfx, sel_list, offs,
                                     T, H, D, "bf16", theta, n_sfx)
        kg, vg = to_host(k_out), to_host(v_out)
        np.testing.assert_array_equal(vg, v_ref)
        assert_rotated_keys(kg, k_ref)
        qpos = np.sort(np.concatenate([offs[b] + sel_list[b] for b in range(nb)] +
                                      [np.arange(T_c, T)])).astype(np.int32)
        q = _queries(syn, seed, ns, offs, layer, Hq, D, "bf16", qpos, T_c, n_sfx)
        rows = np.arange(len(qpos), dtype=np.int32) if n_rows is None else _rows_sample(len(qpos), rng, n_rows)
        _check_attention(ct, orc, q, qpos, k_out, v_out, k_ref, v_ref, theta, rows, "bf16")
        print(f"[workload] r={r[0]}/{r[1]}: assembled layer and {len(rows)} of {len(qpos)} attention rows "
              "(all heads) match the oracle", flush=True)


def test_workload_qwen3_4b_ragged(orc, syn):
    ct = need_gpu()
    import synth
    seed, nb, H, Hq, D, theta, n_sfx = 20260524, 64, 8, 32, 128, 1000000.0, 128
    ns = [int(x) for x in synth.uniform_ints(seed, 1, nb, 512, 4096)]
    L = 36
    rng = np.random.default_rng(7)
    host, dev, s_gpu = _score_chunks(ct, syn, seed, ns, L, H, D, "bf16", (1, 32))
    # the shortest chunk (cutoff 8 bins), the longest, and two odd lengths
    odd = [b for b in range(nb) if ns[b] % 2 == 1][:2]
    sample = sorted({int(np.argmin(ns)), int(np.argmax(ns)), *odd})
    s_orc = _check_scores(orc, host, s_gpu, ns, sample, (1, 32))
    ks, ranking, sel, comp = ct.cachetune_select_topr(to_dev(s_gpu), ns, r=(15, 100))
    torch.cuda.synchronize()
    sl = to_host(sel)
    for b in sample:
        k = ks[b]
        check_index_sets(sl[sum(ks[:b]):sum(ks[:b]) + k], orc.topr(s_orc[b], k)[1], s_orc[b], k)
    offs = np.cumsum([0] + ns[:-1])
    T_c = sum(ns)
    T = T_c + n_sfx
    sel_list = [sl[sum(ks[:b]):sum(ks[:b]) + ks[b]] for b in range(nb)]
    qpos = np.sort(np.concatenate([offs[b] + sel_list[b] for b in range(nb)] +
                                  [np.arange(T_c, T)])).astype(np.int32)
    # a middle layer and the last one: the whole assembled layer, and sampled
    # attention rows (the first, the last and seeded ones) over all heads
    for layer, n_rows in ((2, 192), (L - 1, 64)):
        k_out, v_out, rec, sfx, _ = _request(ct, syn, seed, ns, offs, layer, H, D, "bf16", sel_list, comp,
                                             sel, theta, n_sfx, T, [(k[layer], v[layer]) for k, v in dev])
        k_ref, v_ref = _oracle_layer(orc, [(k[layer], v[layer]) for k, v in host], rec, sfx, sel_list,
                                     offs, T, H, D, "bf16", theta, n_sfx)
        kg, vg = to_host(k_out), to_host(v_out)
        np.testing.assert_array_equal(vg, v_ref)
        assert_rotated_keys(kg, k_ref)
        q = _queries(syn, seed, ns, offs, layer, Hq, D, "bf16", qpos, T_c, n_sfx)
        _check_attention(ct, orc, q, qpos, k_out, v_out, k_ref, v_ref, theta,
                         _rows_sample(len(qpos), rng, n_rows), "bf16")
        del k_out, v_out

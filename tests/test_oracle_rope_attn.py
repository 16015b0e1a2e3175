"""Pins for the oracle's RoPE, assembly (App. B.2/B.3 of the CacheTune page)
and selected-query causal attention (Sec. 4.1).  Expected values come from
closed forms, group properties of rotations, explicit numpy softmax on tiny
inputs, and torch's own float->bfloat16 conversion."""
import numpy as np
import pytest
import torch

RNG = np.random.default_rng(7)


# ---- bf16 rounding ---------------------------------------------------------

def test_round_bf16_known_values(orc):
    assert orc.round_bf16(np.array([1.0]))[0] == 0x3F80
    assert orc.round_bf16(np.array([1.0 + 2 ** -8]))[0] == 0x3F80      # tie -> even
    assert orc.round_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82  # tie -> even (up)
    assert orc.round_bf16(np.array([-2.0]))[0] == 0xC000
    assert orc.round_bf16(np.array([0.0]))[0] == 0x0000
    assert orc.round_bf16(np.array([1e39]))[0] == 0x7F80


def test_round_bf16_matches_torch_on_fp32_values(orc):
    x = np.concatenate([RNG.standard_normal(3000) * 10.0 ** RNG.integers(-30, 30, 3000),
                        np.array([1e-40, -3e-39, 5.9e-39])]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.round_bf16(x.astype(np.float64)), want)


# ---- RoPE ------------------------------------------------------------------

def test_rope_closed_form(orc):
    # D = 2: a single pair with frequency theta^0 = 1
    y = orc.rope(np.array([1.0, 0.0]), 0.7, 10000.0)
    np.testing.assert_allclose(y, [np.cos(0.7), np.sin(0.7)], atol=1e-15)
    # D = 4, theta = 10000: frequencies 1 and 10000^(-1/2) = 0.01
    x = np.array([1.0, 2.0, 3.0, 4.0])
    p = 5.0
    y = orc.rope(x, p, 10000.0)
    a0, a1 = p * 1.0, p * 0.01
    want = [1 * np.cos(a0) - 3 * np.sin(a0), 2 * np.cos(a1) - 4 * np.sin(a1),
            1 * np.sin(a0) + 3 * np.cos(a0), 2 * np.sin(a1) + 4 * np.cos(a1)]
    np.testing.assert_allclose(y, want, atol=1e-14)
    np.testing.assert_allclose(orc.rope_freqs(4, 10000.0), [1.0, 0.01], rtol=1e-15)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_group_properties(orc, style):
    D, th = 64, 500000.0
    q = RNG.standard_normal(D)
    k = RNG.standard_normal(D)
    R = lambda v, p: orc.rope(v, p, th, style)
    np.testing.assert_allclose(R(q, 0.0), q, atol=0)                           # R(0) = I
    for p in (1.0, 777.0, 150000.0):
        y = R(q, p)
        assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12                # isometry
        np.testing.assert_allclose(R(y, -p), q, atol=1e-9)                        # R(-p)R(p) = I
    np.testing.assert_allclose(R(R(q, 300.0), 4100.0), R(q, 4400.0), atol=1e-9)  # R(a)R(b) = R(a+b)
    # relative position: <R(p)q, R(p')k> depends on p - p' only
    for p, pp, s in ((10, 3, 1000), (5000, 4990, 123456)):
        a = np.dot(R(q, p), R(k, pp))
        b = np.dot(R(q, p + s), R(k, pp + s))
        assert abs(a - b) < 1e-9


def test_rope_styles_are_a_permutation(orc):
    D = 16
    x = RNG.standard_normal(D)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # interleaved -> half
    yi = orc.rope(x, 31.0, 10000.0, orc.ROPE_INTERLEAVED)
    yh = orc.rope(x[perm], 31.0, 10000.0, orc.ROPE_HALF)
    np.testing.assert_allclose(yi[perm], yh, atol=1e-14)


# ---- assembly ----------------------------------------------------------------

def test_assembly_routing(orc, syn):
    H, D, th = 2, 16, 10000.0
    n = [40, 25]
    offs = orc.offsets(n, [1, 0], prefix=3)   # chunk 1 first, then chunk 0
    T = 3 + sum(n)
    k_out = np.zeros((T, H, D), np.uint16)
    v_out = np.zeros((T, H, D), np.uint16)
    sels = {}
    for b in range(2):
        ks = syn.rows(9, syn.K, b, 0, n[b], H, D, np.arange(n[b]), "bf16")
        vs = syn.rows(9, syn.V, b, 0, n[b], H, D, np.arange(n[b]), "bf16")
        sel = np.sort(RNG.choice(n[b], 6, replace=False)).astype(np.int32)
        kr = syn.rows(9, syn.K, b, 0, n[b], H, D, sel, "bf16", extra_sigma=0.25)
        vr = syn.rows(9, syn.V, b, 0, n[b], H, D, sel, "bf16", extra_sigma=0.25)
        assert not np.array_equal(kr, ks[sel])           # recomputed rows differ
        orc.assemble_chunk(ks, vs, kr, vr, sel, offs[b], th, 0, k_out, v_out)
        sels[b] = (ks, vs, kr, vr, sel)
    for b in range(2):
        ks, vs, kr, vr, sel = sels[b]
        pos_in_sel = {int(i): t for t, i in enumerate(sel)}
        for i in range(n[b]):
            g = offs[b] + i
            if i in pos_in_sel:
                srck, srcv = kr[pos_in_sel[i]], vr[pos_in_sel[i]]
            else:
                srck, srcv = ks[i], vs[i]
            np.testing.assert_array_equal(v_out[g], srcv)          # V: bit copy
            for h in range(H):
                want = orc.round_bf16(orc.rope(orc.widen(srck[h]), g, th))
                np.testing.assert_array_equal(k_out[g, h], want)   # K: RoPE at g
    assert not k_out[:3].any()                                      # prefix untouched


def test_assembly_fp32_offset_zero_is_plain_rope(orc, syn):
    H, D, n = 1, 8, 10
    ks = syn.rows(3, syn.K, 0, 0, n, H, D, np.arange(n), "f32")
    vs = syn.rows(3, syn.V, 0, 0, n, H, D, np.arange(n), "f32")
    k_out = np.zeros((n, H, D), np.float32)
    v_out = np.zeros((n, H, D), np.float32)
    orc.assemble_chunk(ks, vs, None, None, np.zeros(0, np.int32), 0, 10000.0, 0, k_out, v_out)
    for i in range(n):
        want = orc.rope(ks[i, 0].astype(np.float64), i, 10000.0).astype(np.float32)
        np.testing.assert_array_equal(k_out[i, 0], want)
    np.testing.assert_array_equal(v_out, vs)


# ---- attention -----------------------------------------------------------------

def _stored_query(orc, q_pre_row, pos, theta):
    """The rotated query as stored: RoPE, then one rounding to the storage type
    (bf16 through the pinned round_bf16, fp32 by numpy's conversion)."""
    y = orc.rope(orc.widen(q_pre_row), pos, theta)
    if q_pre_row.dtype == np.uint16:
        return orc.widen(orc.round_bf16(y))
    return y.astype(np.float32).astype(np.float64)


def _np_attention(q_pre, qpos, k, v, scale, theta, orc):
    n_q, Hq, D = q_pre.shape
    T, H, _ = k.shape
    out = np.zeros((n_q, Hq, D))
    for r in range(n_q):
        for h in range(Hq):
            q = _stored_query(orc, q_pre[r, h], qpos[r], theta)
            kh = orc.widen(k[: qpos[r] + 1, h * H // Hq])
            vh = orc.widen(v[: qpos[r] + 1, h * H // Hq])
            z = scale * kh @ q
            p = np.exp(z - z.max())
            out[r, h] = (p / p.sum()) @ vh
    return out


def _attn_inputs(syn, T=40, H=2, Hq=4, D=16, nq=9):
    # a generator of its own: the inputs do not depend on which tests ran first
    rng = np.random.default_rng(11)
    k = syn.rows(4, syn.K, 0, 0, T, H, D, np.arange(T), "bf16")
    v = syn.rows(4, syn.V, 0, 0, T, H, D, np.arange(T), "bf16")
    qpos = np.sort(rng.choice(T, nq, replace=False)).astype(np.int32)
    q = syn.rows(4, syn.Q, 0, 0, T, Hq, D, qpos, "bf16")
    return q, qpos, k, v


def test_attention_brute_force(orc, syn):
    q, qpos, k, v = _attn_inputs(syn)
    out, lse = orc.attention(q, qpos, k, v, 0.25, 10000.0)
    np.testing.assert_allclose(out, _np_attention(q, qpos, k, v, 0.25, 10000.0, orc), atol=1e-12)


def test_attention_brute_force_fp32(orc, syn):
    T, H, Hq, D, nq = 30, 1, 2, 8, 6
    k = syn.rows(5, syn.K, 0, 0, T, H, D, np.arange(T), "f32")
    v = syn.rows(5, syn.V, 0, 0, T, H, D, np.arange(T), "f32")
    qpos = np.sort(RNG.choice(T, nq, replace=False)).astype(np.int32)
    q = syn.rows(5, syn.Q, 0, 0, T, Hq, D, qpos, "f32")
    out, _ = orc.attention(q, qpos, k, v, 0.4, 10000.0)
    np.testing.assert_allclose(out, _np_attention(q, qpos, k, v, 0.4, 10000.0, orc), atol=1e-12)


def test_attention_takes_the_stored_query(orc, syn):
    """The bf16 query is rounded after the rotation: the unrounded rotation
    gives a different output (by far more than the oracle's own rounding)."""
    q, qpos, k, v = _attn_inputs(syn)
    out, _ = orc.attention(q, qpos, k, v, 0.25, 10000.0)
    T, H, _ = k.shape
    diff = 0.0
    for r in range(len(qpos)):
        for h in range(q.shape[1]):
            qq = orc.rope(orc.widen(q[r, h]), qpos[r], 10000.0)  # not rounded
            z = 0.25 * orc.widen(k[: qpos[r] + 1, h * H // q.shape[1]]) @ qq
            p = np.exp(z - z.max())
            unrounded = (p / p.sum()) @ orc.widen(v[: qpos[r] + 1, h * H // q.shape[1]])
            diff = max(diff, np.abs(out[r, h] - unrounded).max())
    assert diff > 1e-9


def test_attention_special_cases(orc, syn):
    q, qpos, k, v = _attn_inputs(syn)
    T, H, D = k.shape
    # a query at position 0 sees one key: output = that value
    q0pos = np.array([0], np.int32)
    out, lse = orc.attention(q[:1], q0pos, k, v, 0.25, 10000.0)
    for h in range(q.shape[1]):
        np.testing.assert_allclose(out[0, h], orc.widen(v[0, h * H // q.shape[1]]), atol=1e-15)
    # identical keys: output = mean of the visible values
    kc = np.repeat(k[:1], T, axis=0)
    out, _ = orc.attention(q, qpos, kc, v, 0.25, 10000.0)
    for r, p in enumerate(qpos):
        for h in range(q.shape[1]):
            np.testing.assert_allclose(out[r, h], orc.widen(v[: p + 1, h * H // q.shape[1]]).mean(0),
                                       atol=1e-12)
    # causality: changing keys/values after a query's position leaves it unchanged
    out, lse = orc.attention(q, qpos, k, v, 0.25, 10000.0)
    k2, v2 = k.copy(), v.copy()
    p0 = int(qpos[3])
    k2[p0 + 1:] = 0x4000
    v2[p0 + 1:] = 0xC000
    out2, lse2 = orc.attention(q, qpos, k2, v2, 0.25, 10000.0)
    np.testing.assert_array_equal(out2[:4], out[:4])
    np.testing.assert_array_equal(lse2[:4], lse[:4])


def test_attention_gqa_equals_repeated_mha(orc, syn):
    q, qpos, k, v = _attn_inputs(syn, H=2, Hq=4)
    out, lse = orc.attention(q, qpos, k, v, 0.3, 10000.0)
    kr = np.ascontiguousarray(np.repeat(k, 2, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, 2, axis=1))
    out2, lse2 = orc.attention(q, qpos, kr, vr, 0.3, 10000.0)
    np.testing.assert_allclose(out, out2, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, atol=1e-15)


def test_attention_lse_normalises(orc, syn):
    q, qpos, k, v = _attn_inputs(syn, H=1, Hq=1, nq=3)
    _, lse = orc.attention(q, qpos, k, v, 0.25, 10000.0)
    for r, p in enumerate(qpos):
        qq = _stored_query(orc, q[r, 0], p, 10000.0)
        z = 0.25 * orc.widen(k[: p + 1, 0]) @ qq
        assert abs(np.exp(z - lse[r, 0]).sum() - 1.0) < 1e-12


def test_attention_row_subset(orc, syn):
    q, qpos, k, v = _attn_inputs(syn)
    full, lf = orc.attention(q, qpos, k, v, 0.25, 10000.0)
    rows = np.array([7, 2], np.int32)
    part, lp = orc.attention(q, qpos, k, v, 0.25, 10000.0, rows=rows)
    np.testing.assert_array_equal(part, full[rows])
    np.testing.assert_array_equal(lp, lf[rows])

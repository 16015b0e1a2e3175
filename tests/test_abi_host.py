"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/cachetune.h declares, and rejects invalid arguments
before touching the device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cachetune.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cachetune_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import non_prefix_kv_token_amd as ct
    if not os.path.exists(ct.LIB_PATH):
        pytest.skip("library not built")
    return ct.lib()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("cachetune_score_chunk", "cachetune_select_topr", "cachetune_assemble_rope",
              "cachetune_recompute_attn"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_symbol_list_matches_header():
    import non_prefix_kv_token_amd as ct
    assert sorted(ct.SYMBOLS) == _declared()


def test_status_strings(lib):
    import non_prefix_kv_token_amd as ct
    for s in (ct.CT_OK, ct.CT_E_INVALID, ct.CT_E_UNSUPPORTED, ct.CT_E_WORKSPACE, ct.CT_E_HIP):
        assert lib.cachetune_status_string(s)
    assert lib.cachetune_version() >= 1


def test_score_ws_validation(lib):
    import non_prefix_kv_token_amd as ct
    n = (C.c_int32 * 2)(2048, 2048)
    out = C.c_size_t(0)
    assert lib.cachetune_score_chunk_ws(None, n, 2, 32, 8, 128, 1, 16, 0, C.byref(out)) == ct.CT_OK
    assert out.value > 0
    bad = (C.c_int32 * 1)(1)  # chunk shorter than 2 tokens
    assert lib.cachetune_score_chunk_ws(None, bad, 1, 32, 8, 128, 1, 16, 0, C.byref(out)) == ct.CT_E_INVALID
    assert b"chunk length" in lib.cachetune_last_error()
    assert lib.cachetune_score_chunk_ws(None, n, 2, 32, 8, 128, 3, 2, 0, C.byref(out)) == ct.CT_E_INVALID
    assert lib.cachetune_score_chunk_ws(None, n, 2, 32, 3, 7, 1, 16, 0, C.byref(out)) == ct.CT_E_UNSUPPORTED


def test_calls_reject_bad_arguments_without_device_work(lib):
    import non_prefix_kv_token_amd as ct
    kout = (C.c_int32 * 1)()
    n = (C.c_int32 * 1)(100)
    # r outside [0, 1]
    assert lib.cachetune_select_topr(None, C.c_void_p(16), n, 1, 3, 2, None, C.c_void_p(16), None, kout,
                                     None) == ct.CT_E_INVALID
    # head_dim not supported
    assert lib.cachetune_assemble_rope(None, None, 0, None, None, 0, 0, 8, 96, ct.CT_BF16, 10000.0, 0,
                                       C.c_void_p(16), C.c_void_p(16), 10, None) == ct.CT_E_UNSUPPORTED
    # misaligned output
    assert lib.cachetune_assemble_rope(None, None, 0, None, None, 0, 0, 8, 128, ct.CT_BF16, 10000.0, 0,
                                       C.c_void_p(18), C.c_void_p(16), 10, None) == ct.CT_E_INVALID
    # Hq not a multiple of H
    assert lib.cachetune_recompute_attn(None, None, None, 0, 6, None, None, 10, 4, 128, ct.CT_BF16, 0.1,
                                        10000.0, 0, None, None, None, 0, None) == ct.CT_E_INVALID
    # index-array check: NULL array with entries, negative count or bound, NULL result
    assert lib.cachetune_check_indices(None, 4, 10, 1, C.c_void_p(16), None) == ct.CT_E_INVALID
    assert lib.cachetune_check_indices(C.c_void_p(16), -1, 10, 1, C.c_void_p(16), None) == ct.CT_E_INVALID
    assert lib.cachetune_check_indices(C.c_void_p(16), 4, -1, 1, C.c_void_p(16), None) == ct.CT_E_INVALID
    assert lib.cachetune_check_indices(C.c_void_p(16), 4, 10, 1, None, None) == ct.CT_E_INVALID
    out = C.c_size_t(1)
    assert lib.cachetune_recompute_attn_ws(None, 100, 32, 16512, 8, 128, ct.CT_BF16, C.byref(out)) == ct.CT_OK
    assert lib.cachetune_recompute_attn_ws(None, 100, 32, 16512, 8, 100, ct.CT_BF16,
                                           C.byref(out)) == ct.CT_E_UNSUPPORTED


def test_select_topr_counts(lib, orc):
    """k = floor(r n) per chunk from the library's host query, the oracle's count."""
    import non_prefix_kv_token_amd as ct
    ns = [512, 2048, 1, 8192, 333]
    arr = (C.c_int32 * len(ns))(*ns)
    for r in [(15, 100), (0, 1), (1, 1), (1, 3)]:
        k = (C.c_int32 * len(ns))()
        assert lib.cachetune_select_topr_counts(arr, len(ns), r[0], r[1], k) == ct.CT_OK
        assert list(k) == [orc.ksel(n, *r) for n in ns]
    k = (C.c_int32 * len(ns))()
    assert lib.cachetune_select_topr_counts(arr, len(ns), 3, 2, k) == ct.CT_E_INVALID
    assert lib.cachetune_select_topr_counts(None, len(ns), 1, 2, k) == ct.CT_E_INVALID


def test_handle_calls_reject_bad_arguments(lib):
    import non_prefix_kv_token_amd as ct
    h = C.c_void_p()
    assert lib.cachetune_create(-1, C.byref(h)) in (ct.CT_E_INVALID, ct.CT_E_HIP)
    assert h.value is None
    assert lib.cachetune_create(0, None) == ct.CT_E_INVALID
    lib.cachetune_destroy(None)  # ignored
    n = (C.c_int32 * 1)(2048)
    assert lib.cachetune_prepare_scoring(None, n, 1, 1, 16, 0, None) == ct.CT_E_INVALID


# ---- hardware-aware ratio search: host logic, callable without a GPU ---------------------

@pytest.mark.parametrize("case", [
    dict(t_c=1.0, t_i=0.25, c=0.23, r_min=0.0, half_width=0.1, eps=0.01),
    dict(t_c=0.6, t_i=0.09, c=0.10, r_min=0.15, half_width=0.1, eps=0.005),   # optimum below the floor
    dict(t_c=1.0, t_i=1.0, c=0.62, r_min=0.0, half_width=0.2, eps=1e-4),
])
def test_calibrate_ratio_matches_oracle(lib, orc, case):
    """The library's search makes the oracle's probes, in the same order, and
    returns the oracle's ratio."""
    import non_prefix_kv_token_amd as ct
    c = case["c"]
    cost = lambda r: (r - c) ** 2 + 0.1 * abs(r - c)  # noqa: E731
    kw = dict(r_min=case["r_min"], half_width=case["half_width"], eps=case["eps"])
    seen = []
    r_lib, n = ct.cachetune_calibrate_ratio(case["t_c"], case["t_i"], lambda r: (seen.append(r), cost(r))[1],
                                            **kw)
    r_orc, probes, _ = orc.calibrate_ratio(case["t_c"], case["t_i"], cost, **kw)
    assert n == len(probes) == len(seen)
    assert max(abs(x - p[0]) for x, p in zip(seen, probes)) <= 1e-12
    assert abs(r_lib - r_orc) <= 1e-12


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fit_cost_model_matches_oracle(lib, orc, seed):
    """The library's App. C.1 fit equals the oracle's (numpy least squares) on
    noisy probes, and refuses what the oracle finds no fit for."""
    import numpy as np
    import non_prefix_kv_token_amd as ct
    rng = np.random.default_rng(seed)
    r = np.array([0.02, 0.05, 0.10, 0.15, 0.20, 0.30, 0.12, 0.25])
    L, N = 32, 65536
    times = orc.cost_model_time(r, 0.6e-3 * (1 + 0.3 * rng.random()), 0.09e-3, 0.9, L, N) * \
        (1 + 0.02 * rng.standard_normal(r.shape))
    want = orc.fit_cost_model(r, times, L, N)
    got = ct.cachetune_fit_cost_model(r, times, L, N)
    assert want is not None
    assert np.allclose(got, want, rtol=1e-9, atol=1e-12)
    one_sided = L * (0.5 + (1 - r) * N * 1e-4)
    assert orc.fit_cost_model(r, one_sided, L, N) is None
    with pytest.raises(RuntimeError):
        ct.cachetune_fit_cost_model(r, one_sided, L, N)
    with pytest.raises(RuntimeError):
        ct.cachetune_fit_cost_model(r[:3], times[:3], L, N)


def test_calibrate_ratio_rejects_bad_arguments(lib):
    import non_prefix_kv_token_amd as ct
    good = lambda r: r  # noqa: E731
    for kw in [dict(t_c=-1.0, t_i=1.0), dict(t_c=0.0, t_i=0.0), dict(t_c=1.0, t_i=1.0, r_min=0.6, r_max=0.5),
               dict(t_c=1.0, t_i=1.0, r_max=1.5), dict(t_c=1.0, t_i=1.0, eps=0.0),
               dict(t_c=1.0, t_i=1.0, half_width=-0.1), dict(t_c=float("nan"), t_i=1.0)]:
        with pytest.raises(RuntimeError):
            ct.cachetune_calibrate_ratio(cost=good, **kw)
    with pytest.raises(RuntimeError):   # a non-finite measurement stops the search
        ct.cachetune_calibrate_ratio(1.0, 1.0, lambda r: float("nan"))
    with pytest.raises(ZeroDivisionError):   # the callback's own exception comes back
        ct.cachetune_calibrate_ratio(1.0, 1.0, lambda r: 1 / 0)


def test_score_variant_ws(lib):
    import non_prefix_kv_token_amd as ct
    n = (C.c_int32 * 2)(2048, 700)
    sz = {}
    for v in (ct.CT_SCORE_LOWPASS, ct.CT_SCORE_L2, ct.CT_SCORE_HIGHPASS):
        out = C.c_size_t(0)
        assert lib.cachetune_score_variant_ws(None, n, 2, 4, 8, 128, 1, 16, 0, v, C.byref(out)) == ct.CT_OK
        sz[v] = out.value
    # the high-frequency view runs the band path first: same workspace; L2 needs only energies
    assert sz[ct.CT_SCORE_HIGHPASS] == sz[ct.CT_SCORE_LOWPASS]
    assert 0 < sz[ct.CT_SCORE_L2] < sz[ct.CT_SCORE_LOWPASS]
    out = C.c_size_t(0)
    assert lib.cachetune_score_variant_ws(None, n, 2, 4, 8, 128, 1, 16, 0, 3, C.byref(out)) == ct.CT_E_INVALID
    assert b"unknown variant" in lib.cachetune_last_error()


def test_band_energy_validation(lib):
    import non_prefix_kv_token_amd as ct
    n = (C.c_int32 * 2)(2048, 9)
    out = C.c_size_t(0)
    assert lib.cachetune_band_energy_ws(n, 2, 4, 8, 128, 0, C.byref(out)) == ct.CT_OK
    # every bin's coefficients: 4 layers x 2 tensors x padded 2*nb rows x 1024 channels x 4 bytes
    assert out.value >= 4 * 2 * (2080 + 32) * 1024 * 4
    arr = (ct.ct_chunk * 2)()
    for i, m in enumerate((2048, 9)):  # pointers are only checked for NULL before device work
        arr[i].k, arr[i].v, arr[i].n = 256, 512, m
    fake = C.c_void_p(1024)
    for nb in (0, 6, 2000):  # 9 tokens have 5 bins
        assert lib.cachetune_band_energy(arr, 2, 4, 8, 128, ct.CT_BF16, 0, nb, fake, None, fake,
                                         1 << 40, None) == ct.CT_E_INVALID
    assert lib.cachetune_band_energy(arr, 2, 4, 8, 128, ct.CT_BF16, 0, 5, None, None, fake,
                                     1 << 40, None) == ct.CT_E_INVALID
    assert lib.cachetune_band_energy(arr, 2, 4, 8, 128, ct.CT_BF16, 0, 5, fake, None, None,
                                     0, None) == ct.CT_E_WORKSPACE


def test_layer_calls_reject_bad_arguments(lib):
    import non_prefix_kv_token_amd as ct
    fake = C.c_void_p(4096)  # only checked for NULL and alignment before device work
    assert lib.cachetune_rmsnorm(fake, fake, 4, 4096, C.c_float(1e-5), ct.CT_F32, fake, None) == ct.CT_E_UNSUPPORTED
    assert lib.cachetune_rmsnorm(fake, fake, 4, 100, C.c_float(1e-5), ct.CT_BF16, fake, None) == ct.CT_E_INVALID
    assert lib.cachetune_rmsnorm(None, fake, 4, 64, C.c_float(1e-5), ct.CT_BF16, fake, None) == ct.CT_E_INVALID
    assert lib.cachetune_rmsnorm(C.c_void_p(4098), fake, 4, 64, C.c_float(1e-5), ct.CT_BF16, fake,
                                 None) == ct.CT_E_INVALID
    assert lib.cachetune_silu_mul(fake, 3, 12, ct.CT_BF16, fake, None) == ct.CT_E_INVALID
    assert lib.cachetune_linear(fake, fake, None, 4, 12, 64, ct.CT_BF16, fake, None) == ct.CT_E_INVALID
    assert lib.cachetune_linear(fake, fake, None, 4, 16, 64, ct.CT_F32, fake, None) == ct.CT_E_UNSUPPORTED
    assert lib.cachetune_linear(None, fake, None, 4, 16, 64, ct.CT_BF16, fake, None) == ct.CT_E_INVALID
    assert lib.cachetune_linear(fake, fake, C.c_void_p(4100), 4, 16, 64, ct.CT_BF16, fake,
                                None) == ct.CT_E_INVALID
    assert lib.cachetune_qkv_proj(fake, fake, 4, 64, 12, 8, ct.CT_BF16, fake, fake, fake, None) == ct.CT_E_INVALID
    assert lib.cachetune_qkv_proj(fake, fake, 4, 64, 16, 8, ct.CT_BF16, fake, None, fake, None) == ct.CT_E_INVALID

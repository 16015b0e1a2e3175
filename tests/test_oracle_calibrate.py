"""Pins of the oracle's hardware-aware ratio search (CacheTune page, App. C.1
cost model and App. C.2 warm-started golden-section search), against
properties the mathematics fixes: the balance point of the cost model, the
golden-section invariants (one new probe per step, width shrinking by the
golden ratio, the minimiser of a unimodal cost kept inside the interval), and a
brute-force grid minimum."""
import math

import numpy as np
import pytest

PHI = (math.sqrt(5.0) - 1.0) / 2.0


def test_warm_start_is_the_balance_point(orc):
    # r*N*t_c == (1 - r)*N*t_i at r = t_i / (t_c + t_i), clamped
    for t_c, t_i in [(1.0, 1.0), (3.0, 1.0), (0.5, 2.0), (7.0, 0.0)]:
        r = orc.warm_start_ratio(t_c, t_i, 0.0, 1.0)
        assert math.isclose(r * t_c, (1.0 - r) * t_i, abs_tol=1e-15)
    assert orc.warm_start_ratio(1.0, 0.01, 0.15, 1.0) == 0.15
    assert orc.warm_start_ratio(0.01, 1.0, 0.0, 0.6) == 0.6


def test_first_probes_are_the_golden_points_around_the_warm_start(orc):
    r, probes, widths = orc.calibrate_ratio(3.0, 1.0, lambda r: 0.0, r_min=0.0, r_max=1.0, half_width=0.1,
                                            eps=0.05)
    a, b = 0.25 - 0.1, 0.25 + 0.1
    assert math.isclose(probes[0][0], a + (1 - PHI) * (b - a), rel_tol=1e-12)
    assert math.isclose(probes[1][0], a + PHI * (b - a), rel_tol=1e-12)
    assert math.isclose(widths[0], b - a, rel_tol=1e-12)


@pytest.mark.parametrize("c", [0.18, 0.2371, 0.31])
def test_unimodal_minimum_within_half_eps(orc, c):
    eps = 1e-3
    r, probes, widths = orc.calibrate_ratio(1.0, 0.25, lambda r: (r - c) ** 2, r_min=0.0, half_width=0.15,
                                            eps=eps)
    assert abs(r - c) <= eps / 2
    assert widths[-1] < eps


def test_one_probe_per_step_and_golden_shrink(orc):
    eps, hw = 1e-4, 0.2
    r, probes, widths = orc.calibrate_ratio(1.0, 1.0, lambda r: abs(r - 0.4321), r_min=0.0, half_width=hw,
                                            eps=eps)
    steps = len(widths) - 1
    assert len(probes) == 2 + steps
    # the first k with (2 hw) phi^k < eps
    assert steps == math.ceil(math.log(eps / (2 * hw)) / math.log(PHI))
    for w0, w1 in zip(widths[:-1], widths[1:]):
        assert math.isclose(w1 / w0, PHI, rel_tol=1e-9)


def test_monotone_costs_end_at_the_interval_edges(orc):
    eps = 1e-3
    r, _, _ = orc.calibrate_ratio(1.0, 0.2, lambda r: r, r_min=0.15, half_width=0.2, eps=eps)
    assert 0.15 <= r <= 0.15 + eps   # increasing cost: the quality floor r_min
    r, _, _ = orc.calibrate_ratio(1.0, 1.0, lambda r: -r, r_min=0.0, half_width=0.2, eps=eps)
    assert 0.7 - eps <= r <= 0.7     # decreasing cost: the upper end r0 + half_width


def test_cost_model_optimum_is_found(orc):
    # per-layer time of the pages' cost model: compute and load overlap, plus overhead
    t_c, t_i, t_o, N = 4.0e-6, 1.0e-6, 3.0e-5, 2048
    cost = lambda r: max(r * N * t_c, (1 - r) * N * t_i) + t_o  # noqa: E731
    r, _, _ = orc.calibrate_ratio(t_c, t_i, cost, r_min=0.0, half_width=0.1, eps=1e-4)
    assert abs(r - t_i / (t_c + t_i)) <= 1e-4


def test_matches_grid_search(orc):
    rng = np.random.default_rng(7)
    for _ in range(20):
        c, p = rng.uniform(0.2, 0.5), rng.uniform(1.0, 3.0)
        cost = lambda r: abs(r - c) ** p  # noqa: E731
        r, _, _ = orc.calibrate_ratio(1.0, 0.5, cost, r_min=0.1, half_width=0.25, eps=1e-3)
        grid = np.linspace(0.1, 0.5833333333333334, 200001)
        best = grid[np.argmin(np.abs(grid - c) ** p)]
        assert abs(r - best) <= 1e-3


# ---- App. C.1 cost model with the fixed per-layer overhead t_o ----------------------

SWEEP = [0.02, 0.05, 0.10, 0.15, 0.20, 0.30]


@pytest.mark.parametrize("t_c,t_i,t_o", [(0.636e-3, 0.085e-3, 1.0), (1.17e-3, 0.12e-3, 0.4),
                                          (2.0e-3, 0.3e-3, 0.05)])
def test_fit_recovers_exact_costs(orc, t_c, t_i, t_o):
    """Times made by the model from known costs (probes on both sides of the
    balance) give back those costs."""
    L, N = 32, 65536
    times = orc.cost_model_time(np.array(SWEEP), t_c, t_i, t_o, L, N)
    got = orc.fit_cost_model(SWEEP, times, L, N)
    assert got is not None
    for a, b in zip(got, (t_c, t_i, t_o)):
        assert abs(a - b) <= 1e-9 * max(1.0, abs(b))


def test_fit_invariances(orc):
    """Scaling every time scales all three costs; adding c*L to every time
    adds c to t_o only; the order of the probes does not matter."""
    L, N = 32, 65536
    rng = np.random.default_rng(3)
    times = orc.cost_model_time(np.array(SWEEP), 0.7e-3, 0.1e-3, 0.8, L, N) * (1 + 0.01 * rng.standard_normal(len(SWEEP)))
    t_c, t_i, t_o = orc.fit_cost_model(SWEEP, times, L, N)
    s = orc.fit_cost_model(SWEEP, 3.0 * times, L, N)
    assert np.allclose(s, (3 * t_c, 3 * t_i, 3 * t_o), rtol=1e-9)
    a = orc.fit_cost_model(SWEEP, times + 0.25 * L, L, N)
    assert np.allclose(a, (t_c, t_i, t_o + 0.25), rtol=1e-9)
    perm = rng.permutation(len(SWEEP))
    p = orc.fit_cost_model(np.array(SWEEP)[perm], times[perm], L, N)
    assert np.allclose(p, (t_c, t_i, t_o), rtol=1e-12)


def test_fit_is_the_best_split_by_brute_force(orc):
    """With noise, the fitted costs give the smallest residual among all
    (split, positive costs) candidates found by a brute-force grid around the
    fit, and the model's balance point lies between the two parts."""
    L, N = 32, 65536
    rng = np.random.default_rng(11)
    times = orc.cost_model_time(np.array(SWEEP), 0.64e-3, 0.085e-3, 1.0, L, N) * (1 + 0.02 * rng.standard_normal(len(SWEEP)))
    t_c, t_i, t_o = orc.fit_cost_model(SWEEP, times, L, N)
    base = np.sum((times - orc.cost_model_time(np.array(SWEEP), t_c, t_i, t_o, L, N)) ** 2)
    for dc in (0.97, 1.0, 1.03):
        for di in (0.97, 1.0, 1.03):
            for do in (-0.05, 0.0, 0.05):
                res = np.sum((times - orc.cost_model_time(np.array(SWEEP), t_c * dc, t_i * di, t_o + do, L, N)) ** 2)
                assert res >= base * (1 - 1e-12)
    rb = t_i / (t_c + t_i)
    assert SWEEP[0] <= rb <= SWEEP[-1]


def test_fit_rejects_one_sided_probes(orc):
    """Probes that are all loading-bound (times falling with r) have no split
    with positive costs on both sides."""
    L, N = 32, 65536
    times = L * (0.5 + (1 - np.array(SWEEP)) * N * 1e-4)
    assert orc.fit_cost_model(SWEEP, times, L, N) is None

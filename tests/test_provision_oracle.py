"""Pins of the provisioning oracle (oracle/provision.py): kappa_r against its
closed forms and a seeded Monte Carlo, the barrier overhead against the
CLT column printed in the pages' Table 1 (tests/golden), the trace moments
against Corollary 4.5 on long geometric traces and against hand sums, the
slot timeline against a step-by-step walk, and the fit against exact lines.
Planted mistakes at the end check that the pins bite."""
import json
import math
import os

import numpy as np
import pytest

from oracle import provision as pv
import workloads.slots as slots

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "barrier_overhead_table1.json")


def test_kappa_closed_forms():
    assert abs(pv.kappa(1)) < 1e-12                       # the mean of one standard normal
    assert abs(pv.kappa(2) - 1 / math.sqrt(math.pi)) < 1e-12
    assert abs(pv.kappa(3) - 3 / (2 * math.sqrt(math.pi))) < 1e-12


@pytest.mark.parametrize("r", [4, 8, 16])
def test_kappa_against_monte_carlo(r):
    rng = np.random.default_rng(100 + r)
    m = rng.standard_normal((400000, r)).max(axis=1)
    se = m.std() / math.sqrt(m.size)
    assert abs(pv.kappa(r) - m.mean()) < 4 * se


def test_barrier_overhead_reproduces_the_printed_clt_column():
    g = json.load(open(GOLDEN))
    B, mu_p, mu_d = g["setting"]["B"], g["setting"]["mu_P"], g["setting"]["mu_D"]
    var_p = mu_p * (mu_p + 1)                              # geometric prompts (reading 17)
    theta = mu_p + mu_d
    nu = math.sqrt(var_p + mu_d * (mu_d + 1))
    for row in g["rows"]:
        ours = 100 * pv.barrier_overhead(B, theta, nu, row["r"])
        if row["r"] == 24:
            # the printed 11.01 % is kappa_32's value, not kappa_24's (10.36 %)
            assert abs(ours - 10.36) < 0.005
            assert abs(100 * pv.barrier_overhead(B, theta, nu, 32) - row["clt"]) < 0.01
            continue
        assert abs(ours - row["clt"]) <= 0.005 + 1e-9, (row, ours)


def test_monte_carlo_overhead_matches_the_printed_mc_column_at_r2():
    """Each worker sums B stationary slot loads; with geometric lifetimes the
    stationary load is P + A, A the age of the request in service: a length-
    biased uniform age, drawn here from simulated slot timelines."""
    g = json.load(open(GOLDEN))
    B, r, trials = 256, 2, 6000
    P, D = slots.draw_slot_traces(1, 20000, "geometric:100", "geometric:500", k=9)
    y = pv.slot_timeline(P[0], D[0])                      # one long stationary timeline
    rng = np.random.default_rng(7)
    draws = y[rng.integers(0, y.size, size=(trials, r, B))]
    loads = draws.sum(axis=2)                             # [trials][r]
    over = 100 * (loads.max(axis=1).mean() / loads.mean() - 1)
    se = 100 * loads.max(axis=1).std() / loads.mean() / math.sqrt(trials)
    assert abs(over - g["rows"][0]["mc"]) < 4 * se + 0.02, (over, se)


def test_trace_moments_meet_corollary_4_5_on_long_geometric_traces():
    P, D = slots.draw_slot_traces(1, 30000, "geometric:100", "geometric:500", k=3)
    theta, q, var = pv.stationary_moments(P[0], D[0])
    th, v = pv.geometric_slot_moments(100.0, 100.0 * 101.0, 500.0)
    assert abs(theta - th) / th < 0.02
    assert abs(var - v) / v < 0.05


@pytest.mark.parametrize("mu_d", [1.0, 2.0, 37.5, 500.0])
def test_corollary_4_5_against_exact_sums_over_the_lifetime_law(mu_d):
    """Stationary load Y = P + A, P independent of the request's age A.  A
    uniformly random decode step lands in a request with probability
    proportional to its lifetime D (length biasing), at an age uniform on
    0..D-1: E[A] = E[D(D-1)/2] / E[D], E[A^2] = E[(D-1)D(2D-1)/6] / E[D].  For
    geometric D on {1, 2, ...} these sums are taken term by term over the pmf
    (truncated where the tail is below 1e-30), not sampled."""
    p = 1.0 / mu_d
    d = np.arange(1, 200001, dtype=np.float64)
    pmf = p * (1.0 - p) ** (d - 1)
    assert pmf[-1] < 1e-30 and abs(pmf.sum() - 1) < 1e-12
    ed = (pmf * d).sum()
    ea = (pmf * d * (d - 1) / 2).sum() / ed
    ea2 = (pmf * (d - 1) * d * (2 * d - 1) / 6).sum() / ed
    mu_p, var_p = 100.0, 100.0 * 101.0
    theta, nu2 = pv.geometric_slot_moments(mu_p, var_p, mu_d)
    assert abs(theta - (mu_p + ea)) < 1e-9 * max(1.0, theta)
    assert abs(nu2 - (var_p + ea2 - ea * ea)) < 1e-9 * max(1.0, nu2)


def test_trace_moments_by_hand():
    # requests (P, D): (3, 2) -> loads 3, 4; (0, 3) -> 0, 1, 2; (5, 1) -> 5
    theta, q, var = pv.stationary_moments([3, 0, 5], [2, 3, 1])
    assert theta == (3 + 4 + 0 + 1 + 2 + 5) / 6
    assert q == (9 + 16 + 0 + 1 + 4 + 25) / 6
    assert abs(var - (q - theta ** 2)) < 1e-12


def test_load_at_step_walks_the_timeline():
    P, D = slots.draw_slot_traces(1, 50, "lognormal:300:0.8:0:4000", "geometric:20", k=4)
    y = pv.slot_timeline(P[0], D[0])
    for step in [0, 1, int(D[0, 0]) - 1, int(D[0, 0]), y.size // 2, y.size - 1]:
        assert pv.load_at_step(P[0], D[0], step) == y[step]
    with pytest.raises(IndexError):
        pv.load_at_step(P[0], D[0], y.size)


def test_fit_recovers_an_exact_line():
    T = np.array([1000, 5000, 20000, 80000, 320000], dtype=float)
    a, b = pv.fit_linear(T, 3.5e-9 * T + 4e-6)
    assert abs(a - 3.5e-9) < 1e-18 and abs(b - 4e-6) < 1e-15


def _pins():
    """The pins above as callables, so that a planted mistake can be run
    through them; each raises AssertionError when its check fails."""
    return {
        "kappa closed forms": test_kappa_closed_forms,
        "printed CLT column": test_barrier_overhead_reproduces_the_printed_clt_column,
        "Corollary 4.5": test_trace_moments_meet_corollary_4_5_on_long_geometric_traces,
        "exact lifetime sums": lambda: [test_corollary_4_5_against_exact_sums_over_the_lifetime_law(m)
                                        for m in (1.0, 2.0, 37.5, 500.0)],
        "hand sums": test_trace_moments_by_hand,
        "timeline walk": test_load_at_step_walks_the_timeline,
        "exact line": test_fit_recovers_an_exact_line,
    }


def _failing_pins():
    failed = []
    for name, pin in _pins().items():
        try:
            pin()
        except AssertionError:
            failed.append(name)
    return failed


def test_pins_pass_on_the_oracle_as_written():
    assert _failing_pins() == []


def _wrong_kappa(r):
    # integrand with Phi^r instead of Phi^(r-1)
    import scipy.integrate
    import scipy.stats
    f = lambda z: z * r * scipy.stats.norm.pdf(z) * scipy.stats.norm.cdf(z) ** r
    return scipy.integrate.quad(f, -np.inf, np.inf, epsabs=1e-13, epsrel=1e-13, limit=200)[0]


def _timeline_ages_from_one(P, D):
    out = []
    for p, d in zip(np.asarray(P).tolist(), np.asarray(D).tolist()):
        out.extend(range(p + 1, p + d + 1))
    return np.array(out, dtype=np.int64)


def _fit_without_intercept(T, t):
    T = np.asarray(T, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    return float((T * t).sum() / (T * T).sum()), 0.0


@pytest.mark.parametrize("name,fn,caught_by", [
    # the sqrt(B) of the worker-load spread dropped from the overhead
    ("barrier_overhead", lambda B, th, nu, r: nu * pv.kappa(r) / (B * th), "printed CLT column"),
    # the spread counted per slot instead of per worker (B instead of sqrt(B))
    ("barrier_overhead", lambda B, th, nu, r: B * nu * pv.kappa(r) / (B * th), "printed CLT column"),
    ("kappa", _wrong_kappa, "kappa closed forms"),
    # Corollary 4.5 with mu_out = E[D] instead of E[D] - 1
    ("geometric_slot_moments", lambda mp, vp, md: (mp + md, vp + md * (md + 1.0)), "exact lifetime sums"),
    # the age variance dropped (nu^2 = sigma_P^2 only)
    ("geometric_slot_moments", lambda mp, vp, md: (mp + md - 1.0, vp), "Corollary 4.5"),
    ("slot_timeline", _timeline_ages_from_one, "hand sums"),
    ("fit_linear", _fit_without_intercept, "exact line"),
])
def test_planted_mistakes_in_the_oracle_are_caught(monkeypatch, name, fn, caught_by):
    """Plant a plausible mistake into oracle/provision.py itself and run the
    pins: the named pin must fail."""
    monkeypatch.setattr(pv, name, fn)
    failed = _failing_pins()
    assert caught_by in failed, f"planting a wrong {name} left every pin green: {failed}"

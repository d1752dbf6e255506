"""Stationary decode-slot load, barrier overhead and the linear attention
latency model (oracle; test infrastructure only).

Follows "Analytical Provisioning for Attention-FFN Disaggregated LLM Serving
under Stochastic Workloads":

* §3.1 (Attention): the step reads the KV cache of every request; the total
  token load is T = sum_b (s_b + i_b) and the latency is linear in it,
  t_A(T) = alpha_A * T + beta_A.  App. B.2.1 derives alpha_A from bytes per
  token over effective bandwidth and leaves beta_A to regression.
* §4.1: one decode slot serves requests one after another; request n has a
  prompt P_n and a lifetime of D_n decode steps, and at age a in 0..D_n-1 its
  load is P_n + a.  Y is the slot's load at a uniformly random decode step,
  theta = E[Y], nu^2 = Var(Y).
* §4.2: with r workers of B slots each, the step waits for the largest worker
  load; its mean is B*theta + sqrt(B)*nu*kappa_r with kappa_r = E[max of r
  independent standard normals] = integral of z r phi(z) Phi(z)^(r-1) dz.
* Corollary 4.5 (geometric lifetimes): theta = mu_P + mu_out and
  nu^2 = sigma_P^2 + mu_out (mu_out + 1), mu_out = E[D] - 1.

Readings where the pages are silent (numbered after those of rows.py):

16. "A uniformly random decode step" of a trace is a uniformly random step
    of the slot's whole timeline, so theta and E[Y^2] of a finite trace are
    plain averages over every decode step it contains.
17. App. A.3 does not state sigma_P; its printed CLT column is reproduced
    with P geometric on {0, 1, ...} with mean 100, sigma_P^2 = 100 * 101,
    and s = sqrt(B (sigma_P^2 + mu_D (mu_D + 1))), m = B (mu_P + mu_D), as
    that appendix writes them.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.integrate
import scipy.stats


def slot_timeline(P, D) -> np.ndarray:
    """Token load of one slot at each of its decode steps, in time order: request
    n contributes P_n, P_n + 1, ..., P_n + D_n - 1."""
    out = []
    for p, d in zip(np.asarray(P).tolist(), np.asarray(D).tolist()):
        out.extend(range(p, p + d))
    return np.array(out, dtype=np.int64)


def stationary_moments(P, D):
    """(theta, E[Y^2], nu^2) of a trace as averages over every decode step (reading 16).
    Exact integer sums, divided once."""
    y = slot_timeline(P, D)
    n = int(y.size)
    s1 = int(y.sum())
    if n and int(y.max()) ** 2 * n < 2 ** 62:
        s2 = int((y * y).sum())                   # exact in int64 under this bound
    else:
        s2 = int((y.astype(object) ** 2).sum())
    theta = s1 / n
    q = s2 / n
    return theta, q, q - theta * theta


def load_at_step(P, D, step: int) -> int:
    """Load of one slot at decode step `step` (0-based), walking its requests."""
    t = 0
    for p, d in zip(np.asarray(P).tolist(), np.asarray(D).tolist()):
        if step < t + d:
            return p + (step - t)
        t += d
    raise IndexError("the trace ends before this step")


def geometric_slot_moments(mu_p: float, var_p: float, mu_d: float):
    """Corollary 4.5: (theta, nu^2) for geometric lifetimes of mean mu_d."""
    mu_out = mu_d - 1.0
    return mu_p + mu_out, var_p + mu_out * (mu_out + 1.0)


def kappa(r: int) -> float:
    """E[max of r independent standard normals] as the integral of z r phi Phi^(r-1)."""
    f = lambda z: z * r * scipy.stats.norm.pdf(z) * scipy.stats.norm.cdf(z) ** (r - 1)
    val, _ = scipy.integrate.quad(f, -np.inf, np.inf, epsabs=1e-13, epsrel=1e-13, limit=200)
    return val


def barrier_overhead(B: int, theta: float, nu: float, r: int) -> float:
    """Relative synchronization overhead (sqrt(B) nu kappa_r) / (B theta) (§4.2)."""
    return math.sqrt(B) * nu * kappa(r) / (B * theta)


def fit_linear(T, t):
    """Least-squares (alpha, beta) of t = alpha * T + beta."""
    T = np.asarray(T, dtype=np.float64)
    A = np.stack([T, np.ones_like(T)], axis=1)
    (alpha, beta), *_ = np.linalg.lstsq(A, np.asarray(t, dtype=np.float64), rcond=None)
    return float(alpha), float(beta)

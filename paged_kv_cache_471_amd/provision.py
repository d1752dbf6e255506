"""Slot-load statistics and the attention latency model (host side).

Continuous batching keeps B decode slots per worker busy; each slot serves
requests one after another, request n with prompt P_n and lifetime D_n, and at
age a its load is P_n + a tokens ("Analytical Provisioning for Attention-FFN
Disaggregated LLM Serving under Stochastic Workloads", §4.1).  The attention
step's time is linear in the total token load, t_A(T) = alpha_A T + beta_A
(§3.1; App. B.2.1 gives alpha_A as bytes per token over effective bandwidth
and leaves beta_A to regression).  With r workers the step waits for the
largest worker load, whose mean is B theta + sqrt(B) nu kappa_r (§4.2).

This module computes, on the host:

* ``trace_moments``: the trace estimator of theta = E[Y] and E[Y^2] (App.
  A.6), closed-form sums over requests, exact in integers;
* ``kappa``: E[max of r standard normals], by composite Simpson quadrature
  of r z phi(z) Phi(z)^(r-1) on [-12, 12];
* ``barrier_load`` / ``barrier_overhead``;
* ``slot_loads``: every slot's load at a given decode step of its trace;
* ``fit_latency``: least-squares (alpha_A, beta_A) from measured step times.

``bench.py`` measures t_A on the GPU over batches whose lengths are
stationary slot loads and fits alpha_A and beta_A with these functions.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def trace_moments(P: Sequence[int], D: Sequence[int]) -> Tuple[float, float, float]:
    """(theta_hat, q_hat, nu2_hat) of a request trace: request i adds D_i decode
    steps with loads P_i .. P_i + D_i - 1, so
        theta_hat = sum[D P + D(D-1)/2] / sum D,
        q_hat     = sum[D P^2 + P D(D-1) + D(D-1)(2D-1)/6] / sum D,
        nu2_hat   = q_hat - theta_hat^2."""
    Pi = [int(x) for x in np.asarray(P).ravel()]
    Di = [int(x) for x in np.asarray(D).ravel()]
    if len(Pi) != len(Di) or not Di:
        raise ValueError("P and D must be non-empty and of one length")
    if min(Di) < 1 or min(Pi) < 0:
        raise ValueError("lifetimes are >= 1 and prompts >= 0")
    n = sum(Di)
    s1 = sum(d * p + d * (d - 1) // 2 for p, d in zip(Pi, Di))
    s2 = sum(d * p * p + p * d * (d - 1) + d * (d - 1) * (2 * d - 1) // 6 for p, d in zip(Pi, Di))
    theta = s1 / n
    q = s2 / n
    return theta, q, q - theta * theta


def kappa(r: int, nodes: int = 4801) -> float:
    """E[max of r independent standard normals]."""
    if r < 1:
        raise ValueError("r >= 1")
    if nodes % 2 == 0:
        nodes += 1
    z = np.linspace(-12.0, 12.0, nodes)
    h = z[1] - z[0]
    phi = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    Phi = 0.5 * (1.0 + np.array([math.erf(x / math.sqrt(2.0)) for x in z]))
    f = z * r * phi * Phi ** (r - 1)
    w = np.ones(nodes)
    w[1:-1:2] = 4.0
    w[2:-1:2] = 2.0
    return float(h / 3.0 * np.dot(w, f))


def barrier_load(B: int, theta: float, nu: float, r: int) -> float:
    """Mean largest worker load over r workers of B slots: B theta + sqrt(B) nu kappa_r."""
    return B * theta + math.sqrt(B) * nu * kappa(r)


def barrier_overhead(B: int, theta: float, nu: float, r: int) -> float:
    """Relative synchronization overhead (nu / theta) (kappa_r / sqrt(B))."""
    return barrier_load(B, theta, nu, r) / (B * theta) - 1.0


def slot_loads(P: np.ndarray, D: np.ndarray, step: int) -> np.ndarray:
    """Load of every slot at decode step `step` of its trace.  P, D [slots][requests];
    raises if some slot's trace ends before that step."""
    P = np.asarray(P, dtype=np.int64)
    D = np.asarray(D, dtype=np.int64)
    ends = np.cumsum(D, axis=1)                       # step after each request's last
    if np.any(ends[:, -1] <= step):
        raise ValueError("a slot's trace ends before this step")
    n = (ends <= step).sum(axis=1)                    # requests finished before `step`
    start = np.where(n > 0, ends[np.arange(len(n)), np.maximum(n - 1, 0)], 0)
    return P[np.arange(len(n)), n] + (step - start)


def fit_latency(T: Sequence[float], t: Sequence[float]) -> Tuple[float, float, float]:
    """(alpha, beta, r2) of t = alpha T + beta by ordinary least squares."""
    T = np.asarray(T, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if T.size < 2:
        raise ValueError("need two points at least")
    Tm, tm = T.mean(), t.mean()
    sxx = float(((T - Tm) ** 2).sum())
    sxy = float(((T - Tm) * (t - tm)).sum())
    alpha = sxy / sxx
    beta = float(tm - alpha * Tm)
    res = t - (alpha * T + beta)
    sst = float(((t - tm) ** 2).sum())
    r2 = 1.0 - float((res ** 2).sum()) / sst if sst > 0 else 1.0
    return alpha, beta, r2


__all__ = ["trace_moments", "kappa", "barrier_load", "barrier_overhead", "slot_loads", "fit_latency"]

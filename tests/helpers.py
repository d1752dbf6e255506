"""Shared test helpers: move seeded cases to the GPU and compare with the oracle."""
import numpy as np
import torch

import oracle
import workloads as wl

TOL_OUT = {wl.F32: 1e-5, wl.BF16: 1.5e-2, wl.FP8: 5e-2}


def out_bound(ref: np.ndarray, kvd: int, out_bf16: bool):
    """Per-element bound on |out - oracle|.  The max-abs tolerance of the KV
    dtype, except where a bf16 output's own rounding already exceeds it: the
    output is the fp32 result rounded to nearest even, whose error is up to
    half an ulp, 2^(floor(log2 |ref|) - 8), which passes 1.5e-2 from |ref| = 4
    up.  There the bound is that half ulp plus 2^-12 |ref| for the fp32
    computation before the rounding.  fp32 outputs keep the plain tolerance."""
    tol = TOL_OUT[kvd]
    if not out_bf16:
        return np.full(np.shape(ref), tol)
    mag = np.abs(np.asarray(ref, dtype=np.float64))
    half_ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 8)
    return np.maximum(tol, half_ulp + mag * 2.0 ** -12)


def assert_out_close(o: np.ndarray, ro: np.ndarray, kvd: int, out_bf16: bool, label: str = "") -> float:
    """Every element of o within out_bound of the oracle ro; returns max |o - ro|."""
    if o.size == 0:
        return 0.0
    err = np.abs(o - ro)
    bound = out_bound(ro, kvd, out_bf16)
    if not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{label}: |out - oracle| = {err.flat[i]:.3e} > {bound.flat[i]:.3e} at "
                             f"|oracle| = {abs(ro.flat[i]):.3f} (max |out - oracle| = {err.max():.3e})")
    return float(err.max())
# lse bound relative to max(1, |lse|): fp32 KV 1e-5, otherwise 1e-4
TOL_LSE = {wl.F32: 1e-5, wl.BF16: 1e-4, wl.FP8: 1e-4}


def to_dev_storage(x: np.ndarray, dtype: int, dev="cuda"):
    if dtype == wl.F32:
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    if dtype == wl.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(dev).view(torch.float8_e4m3fn)


def gqa_to_dev(case: wl.GQACase, dev="cuda"):
    cfg = case.cfg
    t = dict(
        q=to_dev_storage(case.q, cfg.q_dtype, dev),
        kv=to_dev_storage(case.kv, cfg.kv_dtype, dev),
        page_table=torch.from_numpy(case.page_table).to(dev),
        seq_lens=torch.from_numpy(case.seq_lens).to(dev),
        k_scale=None if case.k_scale is None else torch.from_numpy(case.k_scale).to(dev),
        v_scale=None if case.v_scale is None else torch.from_numpy(case.v_scale).to(dev),
    )
    return t


def mla_to_dev(case: wl.MLACase, dev="cuda"):
    return dict(q=to_dev_storage(case.q, wl.BF16, dev), kv=to_dev_storage(case.kv, wl.BF16, dev),
                page_table=torch.from_numpy(case.page_table).to(dev),
                seq_lens=torch.from_numpy(case.seq_lens).to(dev))


def out_to_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def gqa_oracle(case: wl.GQACase, requests=None):
    cfg = case.cfg
    return oracle.paged_decode_attention(case.q, cfg.q_dtype, case.kv, cfg.kv_dtype, case.page_table,
                                         case.seq_lens, cfg.page_size, case.scale, case.k_scale, case.v_scale,
                                         requests=requests)


def assert_close_gqa(case, out, lse, ref_out, ref_lse, requests=None, label=""):
    kvd = case.cfg.kv_dtype
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    # every request, checked against the oracle or not, gives finite outputs
    # and a log-sum-exp that is finite or, for an empty history, -inf
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    assert not np.any(np.isnan(l)) and not np.any(l == np.inf), f"{label}: NaN or +inf lse"
    rows = list(range(len(case.seq_lens))) if requests is None else list(requests)
    o, l, ro, rl = o[rows], l[rows], ref_out[rows], ref_lse[rows]
    err = assert_out_close(o, ro, kvd, case.cfg.q_dtype == wl.BF16, label)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l)), f"{label}: lse finiteness differs"
    assert np.all(l[~fin] == rl[~fin])
    if fin.any():
        rel = np.max(np.abs(l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin])))
        assert rel <= TOL_LSE[kvd], f"{label}: lse rel err {rel:.3e}"
    return err

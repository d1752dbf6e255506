"""Shared test helpers: move seeded cases to the GPU and compare with the oracle."""
import numpy as np
import torch

import oracle
import workloads as wl

TOL_OUT = {wl.F32: 1e-5, wl.BF16: 1.5e-2, wl.FP8: 5e-2}
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
    err = np.max(np.abs(o - ro)) if o.size else 0.0
    assert err <= TOL_OUT[kvd], f"{label}: max |out - oracle| = {err:.3e} > {TOL_OUT[kvd]}"
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l)), f"{label}: lse finiteness differs"
    assert np.all(l[~fin] == rl[~fin])
    if fin.any():
        rel = np.max(np.abs(l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin])))
        assert rel <= TOL_LSE[kvd], f"{label}: lse rel err {rel:.3e}"
    return err

"""The largest batch the library offers (8192 requests), on both paths, every
output compared with the oracle: many short and empty histories, so that
the planner's shares hold many streams each and empty requests are spread
over all workers."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import gqa_to_dev, mla_to_dev, gqa_oracle, assert_close_gqa, assert_out_close, out_to_f64, TOL_LSE

pytestmark = pytest.mark.gpu

da = None
MAX_BATCH = 8192


def setup_module(module):
    global da
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_471_amd as _da
    da = _da


def _short_lengths(seed, hi):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, hi, size=MAX_BATCH).astype(np.int32)
    lens[rng.random(MAX_BATCH) < 0.1] = 0
    return lens


@pytest.mark.parametrize("kd", [wl.BF16, wl.FP8])
def test_gqa_at_the_batch_limit(kd):
    cfg = wl.GQAConfig("maxbatch", 21, MAX_BATCH, 8, 2, 64, 16, wl.BF16, kd, "fixed:1")
    case = wl.make_gqa_case(cfg, seq_lens=_short_lengths(81, 60), poison=True, seed=82)
    t = gqa_to_dev(case)
    out, lse = da.decode_attn_paged(t["q"], t["kv"], t["page_table"], t["seq_lens"], case.scale,
                                    k_scale=t["k_scale"], v_scale=t["v_scale"])
    torch.cuda.synchronize()
    ro, rl = gqa_oracle(case)
    assert_close_gqa(case, out, lse, ro, rl, label=f"batch {MAX_BATCH}")


def test_mla_at_the_batch_limit():
    cfg = wl.MLAConfig("maxbatch", 22, MAX_BATCH, 128, 576, 512, 64, "fixed:1")
    case = wl.make_mla_case(cfg, seq_lens=_short_lengths(83, 65), seed=84)
    t = mla_to_dev(case)
    out, lse = da.decode_attn_mla(t["q"], t["kv"], t["page_table"], t["seq_lens"], case.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode_attention(case.q, case.kv, case.page_table, case.seq_lens, cfg.page_size,
                                         case.scale, 512)
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    assert_out_close(o, ro, wl.BF16, True, f"batch {MAX_BATCH}")
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin) and np.all(l[~fin] == -np.inf), "empty requests: lse -inf"
    rel = np.abs(l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))
    assert float(rel.max()) <= TOL_LSE[wl.BF16], f"lse rel err {rel.max():.3e}"

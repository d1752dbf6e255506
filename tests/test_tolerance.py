"""The per-element output bound the GPU tests use (helpers.out_bound).

The pages fix max-abs tolerances per KV dtype (1e-5 fp32, 1.5e-2 bf16, 5e-2
fp8).  A bf16 output is the fp32 result rounded to nearest even, and that
rounding alone is off by up to half an ulp, which passes 1.5e-2 from |out| = 4
up; there the bound is the half ulp plus 2^-12 |out|.  These tests pin the
bound: the pages' tolerance below that magnitude, every correctly rounded
bf16 value accepted at any magnitude, and a value one ulp off rejected."""
import numpy as np
import torch

import workloads as wl
from helpers import out_bound, assert_out_close, TOL_OUT


def _bf16_rne(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_pages_tolerance_below_four():
    ref = np.linspace(-3.99, 3.99, 20001)
    assert np.all(out_bound(ref, wl.BF16, True) == TOL_OUT[wl.BF16])
    assert np.all(out_bound(ref * 4, wl.FP8, True) == TOL_OUT[wl.FP8])
    assert np.all(out_bound(ref * 1000, wl.F32, False) == TOL_OUT[wl.F32])


def test_correct_rounding_always_passes():
    rng = np.random.default_rng(5)
    ref = np.concatenate([rng.uniform(-64, 64, 200000), rng.standard_normal(200000) * 3])
    # just below and above the rounding midpoints of [4, 8), where the error peaks
    ulp = 2.0 ** -5
    mids = 4.0 + ulp * (np.arange(128) + 0.5)
    ref = np.concatenate([ref, mids - 1e-9, mids + 1e-9, -(mids - 1e-9)])
    rounded = _bf16_rne(ref)
    assert np.max(np.abs(rounded - ref)) > TOL_OUT[wl.BF16]        # the plain tolerance cannot hold there
    assert np.all(np.abs(rounded - ref) <= out_bound(ref, wl.BF16, True))
    assert_out_close(rounded, ref, wl.BF16, True, "correctly rounded")


def test_one_ulp_off_fails():
    ref = np.array([4.5, -6.25, 12.0, 0.75])
    ulp = np.array([2.0 ** -5, 2.0 ** -5, 2.0 ** -4, 2.0 ** -8])
    bad = _bf16_rne(ref) + ulp
    bound = out_bound(ref, wl.BF16, True)
    assert np.all(np.abs(bad[:3] - ref[:3]) > bound[:3])
    try:
        assert_out_close(bad[:3], ref[:3], wl.BF16, True, "one ulp off")
    except AssertionError:
        pass
    else:
        raise AssertionError("an output one ulp off the correctly rounded value was accepted")
    # below 4 the pages' tolerance itself decides
    assert np.abs(bad[3] - ref[3]) <= TOL_OUT[wl.BF16] and bound[3] == TOL_OUT[wl.BF16]

"""GPU parity of the absorbed-MLA path against the float64 oracle (through the C ABI).

Bound: max |out - oracle| <= 1.5e-2 over every output element (bf16 latent);
lse within 1e-4 relative to max(1, |lse|).  The kernel rounds the softmax
weights to bf16 as the MFMA operand and accumulates in fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import mla_to_dev, out_to_f64, assert_out_close

pytestmark = pytest.mark.gpu

TOL_LSE = 1e-4

da = None


def setup_module(module):
    global da
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_471_amd as _da
    da = _da


def _cfg(H=128, P=64, lengths="uniform:1:700", B=4):
    return wl.MLAConfig("t", 9, B, H, 576, 512, P, lengths)


def run(case, **kw):
    t = mla_to_dev(case)
    out, lse = da.decode_attn_mla(t["q"], t["kv"], t["page_table"], t["seq_lens"], case.scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_of(case, requests=None):
    return oracle.mla_decode_attention(case.q, case.kv, case.page_table, case.seq_lens, case.cfg.page_size,
                                       case.scale, 512, requests=requests)


def assert_close(case, out, lse, ro, rl, requests=None, label=""):
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    # every request, checked against the oracle or not, gives finite outputs
    # and a log-sum-exp that is finite or, for an empty history, -inf
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    assert not np.any(np.isnan(l)) and not np.any(l == np.inf), f"{label}: NaN or +inf lse"
    rows = list(range(len(case.seq_lens))) if requests is None else list(requests)
    o, l, ro, rl = o[rows], l[rows], ro[rows], rl[rows]
    err = assert_out_close(o, ro, wl.BF16, True, label)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l)), f"{label}: lse finiteness differs"
    assert np.all(l[~fin] == rl[~fin])
    if fin.any():
        rel = float(np.max(np.abs(l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))))
        assert rel <= TOL_LSE, f"{label}: lse rel err {rel:.3e}"
    return err


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("P", [32, 64])
def test_heads_and_pages(H, P):
    case = wl.make_mla_case(_cfg(H, P), poison=True, extra_pages=2, seed=300 + H + P)
    out, lse = run(case)
    ro, rl = oracle_of(case)
    assert_close(case, out, lse, ro, rl, label=f"H{H} P{P}")


@pytest.mark.parametrize("lens", [[1], [31], [32], [33], [63], [64], [65], [1, 0, 2], [0], [0, 0, 70],
                                  [4096], [64 * 9 + 17, 3, 64 * 20]])
def test_edge_lengths(lens):
    case = wl.make_mla_case(_cfg(), seq_lens=np.array(lens, dtype=np.int32), poison=True, extra_pages=1, seed=5)
    out, lse = run(case)
    ro, rl = oracle_of(case)
    assert_close(case, out, lse, ro, rl, label=f"lens {lens}")


@pytest.mark.parametrize("workers", [1, 2, 3, 7, 64, 300, 2048])
def test_partitions(workers):
    """Any number of workers gives the same result (pieces merged in token order)."""
    case = wl.make_mla_case(_cfg(lengths="lognormal:400:1.0:1:3000", B=7), poison=True, seed=77)
    case.seq_lens[2] = 0
    out, lse = run(case, workers=workers)
    ro, rl = oracle_of(case)
    assert_close(case, out, lse, ro, rl, label=f"G={workers}")


def test_repeated_calls_reuse_counters():
    cases = [wl.make_mla_case(_cfg(lengths="lognormal:900:1.0:1:6000", B=9), poison=True, seed=400 + i)
             for i in range(2)]
    refs = [oracle_of(c) for c in cases]
    for rep in range(3):
        for c, (ro, rl) in zip(cases, refs):
            out, lse = run(c, workers=50 + 13 * rep)
            assert_close(c, out, lse, ro, rl, label=f"rep {rep}")


def test_one_token_returns_latent_prefix_exactly():
    case = wl.make_mla_case(_cfg(), seq_lens=np.array([1, 1, 1], dtype=np.int32), poison=True, seed=3)
    out, lse = run(case)
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(3):
        lat = case.kv[case.page_table[b, 0], 0, :512]
        assert np.array_equal(o[b], np.broadcast_to(lat, o[b].shape))


def test_sharp_scores():
    """An 8x larger scale exercises the running maximum and its rescaling."""
    case = wl.make_mla_case(_cfg(lengths="uniform:200:900"), poison=True, seed=12)
    case.scale *= 8.0
    out, lse = run(case)
    ro, rl = oracle_of(case)
    assert_close(case, out, lse, ro, rl, label="sharp")


def test_page_permutation_bitwise():
    case = wl.make_mla_case(_cfg(lengths="lognormal:500:0.8:1:4000", B=6), poison=True, extra_pages=4, seed=11)
    out0, lse0 = run(case)
    perm = np.random.default_rng(2).permutation(case.num_pages)
    kv = np.empty_like(case.kv)
    kv[perm] = case.kv
    table = case.page_table.copy()
    m = table >= 0
    table[m] = perm[table[m]]
    case.kv, case.page_table = kv, table
    out1, lse1 = run(case)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_deterministic_across_runs():
    case = wl.make_mla_case(wl.MLA, batch=12, seed=4)
    a, la = run(case)
    b, lb = run(case)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_gather_bitwise():
    case = wl.make_mla_case(_cfg(lengths="uniform:1:200", B=5), poison=True, extra_pages=2, seed=9)
    t = mla_to_dev(case)
    dense = da.paged_kv_gather(t["kv"], t["page_table"], t["seq_lens"], mla=True)
    torch.cuda.synchronize()
    raw = dense.cpu().view(torch.int16).numpy().view(np.uint16)
    for b, L in enumerate(case.seq_lens):
        ref = oracle.gather_history(case.kv, case.page_table, b, int(L), 64, mla=True)
        assert np.array_equal(raw[b, :L], ref)


def test_full_size_whole():
    """The 128-request MLA workload at full size (lognormal lengths up to 64k)
    in the default launch: every output and log-sum-exp against the oracle."""
    case = wl.make_mla_case(wl.MLA)
    out, lse = run(case)
    ro, rl = oracle_of(case)
    assert_close(case, out, lse, ro, rl, label="mla full")


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("workers", [0, 3, 11])
def test_running_max_jumps_every_chunk(H, workers):
    """Scores that rise by more than the kernels' raise margin at every chunk
    boundary: the running maximum moves on every chunk, so the 128-head kernel
    folds its accumulators into the piece's slot and restarts on every chunk
    (and the 64-head kernel rescales on every chunk).  The growth sits in the
    64 rope dims of the latent, which are keys only: rope part of latent row t
    is (t / 2) u, every head's query rope part is u, so scores rise by about 15
    (base 2) per 32 tokens while the values stay N(0, 0.5)."""
    cfg = _cfg(H=H, lengths="uniform:150:700", B=3)
    case = wl.make_mla_case(cfg, poison=True, extra_pages=1, seed=91 + H)
    rng = np.random.default_rng(5)
    u = rng.standard_normal(64) * 0.5
    for b, L in enumerate(case.seq_lens):
        for t in range(int(L)):
            pg, r = case.page_table[b, t // cfg.page_size], t % cfg.page_size
            case.kv[pg, r, 512:] = wl.to_bf16_bits(u * (t / 2.0))
    case.q[:, :, 512:] = wl.to_bf16_bits(np.broadcast_to(u, case.q[:, :, 512:].shape))
    out, lse = run(case, workers=workers)
    ro, rl = oracle_of(case)
    assert_close(case, out, lse, ro, rl, label=f"jumps H{H} G{workers}")

"""Pins for the CPU oracle: each checks it against something other than itself.

Brute force with Python loops and scipy's softmax/logsumexp on tiny inputs,
closed forms, invariants, special cases that reduce to another routine, the
fp8/bf16 decoders against torch's own casts, and the latent byte count the
pages print.  The mutation tests at the end plant plausible mistakes in the
oracle (on the CPU) and check that at least one pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as oatt
from oracle import formats as ofmt
import workloads as wl
from workloads import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers

def _tiny_case(B=3, Hq=4, Hkv=2, D=None, P=None, lens=(1, 5, 9), seed=7, kv_dtype=wl.F32, q_dtype=wl.F32,
               poison=True, extra=2):
    # an fp8 cache's tiled V blocks need head_dim a multiple of 64 and pages of 16k tokens
    if D is None:
        D = 64 if kv_dtype == wl.FP8 else 8
    if P is None:
        P = 16 if kv_dtype == wl.FP8 else 4
    cfg = wl.GQAConfig("t", 0, B, Hq, Hkv, D, P, q_dtype, kv_dtype, "uniform:1:16")
    return wl.make_gqa_case(cfg, seq_lens=np.array(lens, dtype=np.int32), seed=seed,
                            poison=poison, extra_pages=extra, scale=0.37)


def _run(case):
    return oracle.paged_decode_attention(case.q, case.cfg.q_dtype, case.kv, case.cfg.kv_dtype,
                                         case.page_table, case.seq_lens, case.cfg.page_size,
                                         case.scale, case.k_scale, case.v_scale)


def _brute_force(case):
    """Independent statement: Python loops over tokens for the gather and the dot
    products (math.fsum), scipy for softmax and logsumexp."""
    cfg = case.cfg
    qf = ofmt.decode_storage(case.q, cfg.q_dtype)
    B, Hq, D = qf.shape
    g = Hq // cfg.kv_heads
    # an fp8 cache keeps V in tiles; read it back in token order with the
    # input generator's inverse of its storage map
    vlog = wl.fp8_v_from_storage(case.kv[:, 1]) if cfg.kv_dtype == wl.FP8 else case.kv[:, 1]
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(case.seq_lens[b])
        for h in range(Hq):
            j = h // g
            if L == 0:
                lse[b, h] = -np.inf
                continue
            ks, vs = [], []
            for t in range(L):
                page = int(case.page_table[b][t // cfg.page_size])
                slot = t % cfg.page_size
                k = ofmt.decode_storage(case.kv[page, 0, j, slot], cfg.kv_dtype)
                v = ofmt.decode_storage(vlog[page, j, slot], cfg.kv_dtype)
                if cfg.kv_dtype == wl.FP8:
                    k = k * float(case.k_scale[j])
                    v = v * float(case.v_scale[j])
                ks.append(k)
                vs.append(v)
            s = np.array([case.scale * math.fsum(float(qf[b, h, d]) * float(k[d]) for d in range(D))
                          for k in ks])
            p = scipy.special.softmax(s)
            lse[b, h] = scipy.special.logsumexp(s)
            for d in range(D):
                out[b, h, d] = math.fsum(float(p[t]) * float(vs[t][d]) for t in range(L))
    return out, lse


# ----------------------------------------------------------------------------- formats

def test_fp8_table_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = ofmt.fp8_e4m3fn_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.nanmax(mine) == 448.0 and np.nanmin(mine) == -448.0
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isnan(mine).sum() == 2


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = ofmt.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("kv_dtype,q_dtype", [(wl.F32, wl.F32), (wl.BF16, wl.BF16), (wl.FP8, wl.BF16)])
def test_oracle_matches_brute_force(kv_dtype, q_dtype):
    case = _tiny_case(kv_dtype=kv_dtype, q_dtype=q_dtype, lens=(1, 5, 9, 16, 3), B=5)
    out, lse = _run(case)
    bo, bl = _brute_force(case)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_two_token_closed_form():
    case = _tiny_case(B=1, Hq=1, Hkv=1, lens=(2,), poison=False, extra=0)
    out, lse = _run(case)
    q = case.q[0, 0].astype(np.float64)
    pg = case.page_table[0]
    k0, k1 = case.kv[pg[0], 0, 0, 0].astype(np.float64), case.kv[pg[0], 0, 0, 1].astype(np.float64)
    v0, v1 = case.kv[pg[0], 1, 0, 0].astype(np.float64), case.kv[pg[0], 1, 0, 1].astype(np.float64)
    s0, s1 = case.scale * float(q @ k0), case.scale * float(q @ k1)
    e0, e1 = math.exp(s0), math.exp(s1)
    np.testing.assert_allclose(out[0, 0], (e0 * v0 + e1 * v1) / (e0 + e1), rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - math.log(e0 + e1)) < 1e-14


# ----------------------------------------------------------------------------- invariants

def test_one_token_returns_its_value_exactly():
    case = _tiny_case(lens=(1, 1, 1))
    out, lse = _run(case)
    for b in range(3):
        pg = case.page_table[b, 0]
        for h in range(4):
            assert np.array_equal(out[b, h], case.kv[pg, 1, h // 2, 0].astype(np.float64))
            qk = float(case.q[b, h].astype(np.float64) @ case.kv[pg, 0, h // 2, 0].astype(np.float64))
            assert abs(lse[b, h] - case.scale * qk) < 1e-14


def test_constant_value_returns_it():
    case = _tiny_case(lens=(7, 12, 3), poison=True)
    const = np.linspace(-2, 2, case.cfg.head_dim).astype(np.float32)
    for b, L in enumerate(case.seq_lens):
        for t in range(L):
            case.kv[case.page_table[b, t // 4], 1, :, t % 4] = const
    out, _ = _run(case)
    np.testing.assert_allclose(out, np.broadcast_to(const, out.shape), rtol=0, atol=1e-15)


def test_logit_shift_changes_only_lse():
    case = _tiny_case(lens=(6, 11, 2), poison=False, extra=0)
    # keys on a 1/64 grid and shifts on a 1/8 grid keep k + u exact in float32
    case.kv[:, 0] = np.round(case.kv[:, 0] * 64) / 64
    out0, lse0 = _run(case)
    u = np.round(np.random.default_rng(3).standard_normal((2, case.cfg.head_dim)) * 4) / 8
    shifted = case.kv.copy()
    shifted[:, 0] = case.kv[:, 0] + u[None, :, None, :].astype(np.float32)
    assert np.array_equal(shifted[:, 0].astype(np.float64) - case.kv[:, 0].astype(np.float64),
                          np.broadcast_to(u[None, :, None, :], shifted[:, 0].shape))
    case.kv = shifted
    out1, lse1 = _run(case)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-12)
    qf = case.q.astype(np.float64)
    for h in range(4):
        delta = case.scale * (qf[:, h] @ u[h // 2])
        np.testing.assert_allclose(lse1[:, h] - lse0[:, h], delta, rtol=0, atol=1e-12)


def test_page_permutation_is_bitwise_invariant():
    case = _tiny_case(lens=(13, 4, 9), extra=3)
    out0, lse0 = _run(case)
    perm = np.random.default_rng(11).permutation(case.num_pages)
    new_kv = np.empty_like(case.kv)
    new_kv[perm] = case.kv                         # page p moves to perm[p]
    table = case.page_table.copy()
    m = table >= 0
    table[m] = perm[table[m]]
    case.kv, case.page_table = new_kv, table
    out1, lse1 = _run(case)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_token_permutation_within_history():
    case = _tiny_case(lens=(13,), B=1, poison=False, extra=0)
    out0, lse0 = _run(case)
    L = 13
    perm = np.random.default_rng(5).permutation(L)
    P = case.cfg.page_size
    src = [(case.page_table[0, t // P], t % P) for t in range(L)]
    vals = [case.kv[pg, :, :, s].copy() for pg, s in src]
    for t in range(L):
        pg, s = src[t]
        case.kv[pg, :, :, s] = vals[perm[t]]
    out1, lse1 = _run(case)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("cuts", [[0, 5, 13], [0, 1, 2, 3, 13], [0, 12, 13], [0, 4, 4, 8, 13]])
def test_split_merge_equals_unsplit(cuts):
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 16))
    k = rng.standard_normal((13, 16))
    v = rng.standard_normal((13, 16))
    full_o, full_l = oracle.dense_attention(q, k, v, 0.25)
    parts = [oracle.attention_over_range(q, k, v, 0.25, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = oracle.lse_merge(parts)
    np.testing.assert_allclose(o, full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, full_l, rtol=0, atol=1e-12)


def test_merge_of_empty_parts():
    o, l = oracle.lse_merge([(np.zeros((2, 4)), np.full(2, -np.inf))] * 3)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_empty_history():
    case = _tiny_case(lens=(0, 3, 0))
    out, lse = _run(case)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(out[2] == 0) and np.all(lse[2] == -np.inf)
    assert np.all(np.isfinite(out[1]))


def test_gqa_equals_mha_with_repeated_heads():
    case = _tiny_case(lens=(9, 2, 16), poison=False)
    out0, lse0 = _run(case)
    g = 2
    mha = wl.GQAConfig("m", 0, 3, 4, 4, 8, 4, wl.F32, wl.F32, "uniform:1:16")
    kv = np.repeat(case.kv, g, axis=2)             # KV head h//g copied to head h
    rep = wl.GQACase(mha, case.seq_lens, case.page_table, case.num_pages, case.q, kv, None, None,
                     case.scale, case.unreferenced)
    out1, lse1 = _run(rep)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse1, lse0, rtol=0, atol=1e-14)


def test_fp8_scales_apply_per_kv_head():
    """fp8 K/V with power-of-two per-head scales equals the fp32 path fed the exact
    dequantised values (the product is exact in float32)."""
    case = _tiny_case(kv_dtype=wl.FP8, q_dtype=wl.F32, lens=(7, 10, 16), poison=False)
    case.k_scale = np.array([0.5, 4.0], dtype=np.float32)
    case.v_scale = np.array([2.0, 0.25], dtype=np.float32)
    out0, lse0 = _run(case)
    table = ofmt.fp8_e4m3fn_table()
    logical = case.kv.copy()
    logical[:, 1] = wl.fp8_v_from_storage(case.kv[:, 1])        # V in token order
    kv32 = table[logical].astype(np.float32)
    kv32[:, 0] *= case.k_scale[None, :, None, None]
    kv32[:, 1] *= case.v_scale[None, :, None, None]
    f32cfg = wl.GQAConfig("f", 0, 3, 4, 2, case.cfg.head_dim, case.cfg.page_size, wl.F32, wl.F32, "uniform:1:16")
    ref = wl.GQACase(f32cfg, case.seq_lens, case.page_table, case.num_pages, case.q, kv32, None, None,
                     case.scale, case.unreferenced)
    out1, lse1 = _run(ref)
    np.testing.assert_allclose(out0, out1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse0, lse1, rtol=0, atol=1e-14)


def test_mla_equals_single_kv_head_gqa_with_value_prefix():
    cfg = wl.MLAConfig("m", 0, 3, 4, 24, 16, 4, "uniform:1:16")
    case = wl.make_mla_case(cfg, seq_lens=np.array([5, 1, 12], dtype=np.int32), seed=3, poison=True,
                            extra_pages=2, scale=0.2)
    out, lse = oracle.mla_decode_attention(case.q, case.kv, case.page_table, case.seq_lens, 4, 0.2,
                                           v_dim=16)
    # the same history as a one-KV-head GQA cache whose K and V are both the latent
    kv = np.stack([case.kv, case.kv], axis=1)[:, :, None]          # [np][2][1][P][24]
    gcfg = wl.GQAConfig("g", 0, 3, 4, 1, 24, 4, wl.BF16, wl.BF16, "uniform:1:16")
    g = wl.GQACase(gcfg, case.seq_lens, case.page_table, case.num_pages, case.q, kv, None, None,
                   0.2, case.unreferenced)
    gout, glse = _run(g)
    np.testing.assert_allclose(out, gout[..., :16], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, glse, rtol=0, atol=1e-14)


def test_mla_brute_force():
    cfg = wl.MLAConfig("m", 0, 2, 3, 12, 8, 4, "uniform:1:16")
    case = wl.make_mla_case(cfg, seq_lens=np.array([6, 3], dtype=np.int32), seed=4, poison=True,
                            extra_pages=1, scale=0.3)
    out, lse = oracle.mla_decode_attention(case.q, case.kv, case.page_table, case.seq_lens, 4, 0.3,
                                           v_dim=8)
    qf = ofmt.bf16_bits_to_f64(case.q)
    for b in range(2):
        L = int(case.seq_lens[b])
        lat = [ofmt.bf16_bits_to_f64(case.kv[case.page_table[b, t // 4], t % 4]) for t in range(L)]
        for h in range(3):
            s = np.array([0.3 * math.fsum(qf[b, h] * c) for c in lat])
            p = scipy.special.softmax(s)
            ref = [math.fsum(p[t] * lat[t][d] for t in range(L)) for d in range(8)]
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
            assert abs(lse[b, h] - scipy.special.logsumexp(s)) < 1e-12


def test_poison_never_reaches_result():
    case = _tiny_case(lens=(3, 6, 1), poison=True, extra=4)
    out, lse = _run(case)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


# ----------------------------------------------------------------------------- accounting

def test_mla_bytes_per_token_matches_page():
    with open(os.path.join(GOLDEN, "mla_latent_bytes.json")) as f:
        g = json.load(f)
    assert g["d_c"] + g["d_rope"] == g["latent_dim"] == wl.MLA.latent_dim
    assert accounting.mla_kv_bytes_per_token(g["latent_dim"], g["bytes_per_element"]) == g["bytes_per_token"]
    assert wl.MLA.v_dim == g["d_c"]


def test_token_units():
    with open(os.path.join(GOLDEN, "token_units.json")) as f:
        g = json.load(f)
    assert wl.LONGFP8.lengths == f"fixed:{g['examples']['128K']}"
    assert wl.SKEWED.lengths.endswith(f"{g['examples']['32K']}:{g['examples']['64K']}")


# ----------------------------------------------------------------------------- planted mistakes

def _pins_fail(monkeypatch, target, name, bad):
    monkeypatch.setattr(target, name, bad)
    case = _tiny_case(lens=(1, 5, 9, 16, 3), B=5)
    out, lse = _run(case)
    bo, bl = _brute_force(case)
    return not (np.allclose(out, bo, atol=1e-12, rtol=0) and np.allclose(lse, bl, atol=1e-12, rtol=0))


def test_planted_mistakes_are_caught(monkeypatch):
    good_dense = oatt.dense_attention
    good_gather = oatt.gather_history

    def no_max_shift_wrong_lse(q, k, v, scale):          # drops the max term from lse
        o, l = good_dense(q, k, v, scale)
        s = scale * (q @ k.T)
        return o, l - s.max(axis=1) if k.shape[0] else l

    def transposed_scale(q, k, v, scale):                # scale applied to the output, not logits
        o, l = good_dense(q, k, v, 1.0)
        return o * scale, l

    def off_by_one_gather(kv, table, b, length, page_size, mla=False):
        t = np.arange(length, dtype=np.int64)
        pg = table[b, t // page_size].astype(np.int64)
        r = (t + 1) % page_size
        return kv[pg, 0, :, r, :], kv[pg, 1, :, r, :]

    def swapped_kv(kv, table, b, length, page_size, mla=False):
        k, v = good_gather(kv, table, b, length, page_size, mla)
        return v, k

    for name, bad, target in [("dense_attention", no_max_shift_wrong_lse, oatt),
                              ("dense_attention", transposed_scale, oatt),
                              ("gather_history", off_by_one_gather, oatt),
                              ("gather_history", swapped_kv, oatt)]:
        with monkeypatch.context() as m:
            assert _pins_fail(m, target, name, bad), name


def test_planted_head_map_mistake_is_caught(monkeypatch):
    good = oatt.paged_decode_attention

    def interleaved(q, q_dtype, kv, kv_dtype, table, lens, P, scale, ks=None, vs=None, requests=None):
        # maps head h to KV head h % Hkv instead of h // g
        Hkv = kv.shape[2]
        Hq = q.shape[1]
        g = Hq // Hkv
        order = np.array([(h % Hkv) * g + h // Hkv for h in range(Hq)])
        inv = np.argsort(order)
        o, l = good(q[:, order], q_dtype, kv, kv_dtype, table, lens, P, scale, ks, vs, requests)
        return o[:, inv], l[:, inv]

    monkeypatch.setattr(oracle, "paged_decode_attention", interleaved)
    case = _tiny_case(lens=(4, 5, 9), B=3)
    out, lse = _run(case)
    bo, bl = _brute_force(case)
    assert not np.allclose(out, bo, atol=1e-12, rtol=0)

"""Pins of the multi-row decode oracle (oracle/rows.py) against what it does
not compute itself: torch's causal scaled-dot-product attention (a library
routine) when every history token is a query row, numpy's triangular mask
with scipy's softmax / logsumexp on histories gathered here by a loop of this
file's own, the single-row oracle (pinned on its own in test_oracle.py) at
n = 1, and empty rows.  Planted mistakes at the end check that the pins bite."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import rows as orows
from oracle.formats import F32, BF16, FP8
import workloads as wl


def _case(rng, B, n, Hq, Hkv, D, lens, kv_dtype=F32, P=16):
    """Random paged inputs: q [B][n][Hq][D] and a cache holding the given lengths."""
    q_dtype = F32 if kv_dtype == F32 else BF16
    lens = np.asarray(lens, dtype=np.int32)
    npg = (lens + P - 1) // P
    num_pages = int(npg.sum()) + 3
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, max(1, int(npg.max()))), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        table[b, :npg[b]] = perm[at:at + npg[b]]
        at += npg[b]
    q32 = rng.standard_normal((B, n, Hq, D)).astype(np.float32)
    kv32 = rng.standard_normal((num_pages, 2, Hkv, P, D)).astype(np.float32)
    ks = vs = None
    if kv_dtype == F32:
        kv = kv32
    elif kv_dtype == BF16:
        kv = wl.to_bf16_bits(kv32)
    else:
        kc, ks = wl.quantize_fp8_per_head(kv32[:, 0], head_axis=1)
        vc, vs = wl.quantize_fp8_per_head(kv32[:, 1], head_axis=1)
        kv = np.stack([kc, wl.fp8_v_to_storage(vc)], axis=1)     # V blocks in the tiled fp8 format
    q = q32 if q_dtype == F32 else wl.to_bf16_bits(q32)
    return dict(q=q, q_dtype=q_dtype, kv=kv, kv_dtype=kv_dtype, table=table, lens=lens, P=P, ks=ks, vs=vs)


def _dense_history(c, b):
    """K, V [L][Hkv][D] float64 of request b, gathered slot by slot."""
    L, P = int(c["lens"][b]), c["P"]
    dec = oracle.decode_storage
    Hkv, D = c["kv"].shape[2], c["kv"].shape[4]
    K = np.zeros((L, Hkv, D))
    V = np.zeros((L, Hkv, D))
    vlog = wl.fp8_v_from_storage(c["kv"][:, 1]) if c["kv_dtype"] == FP8 else c["kv"][:, 1]
    for t in range(L):
        pg = c["table"][b, t // P]
        K[t] = dec(c["kv"][pg, 0, :, t % P, :], c["kv_dtype"])
        V[t] = dec(vlog[pg, :, t % P, :], c["kv_dtype"])
    if c["kv_dtype"] == FP8:
        K *= c["ks"].astype(np.float64)[None, :, None]
        V *= c["vs"].astype(np.float64)[None, :, None]
    return K, V


def _run(c, scale):
    return oracle.paged_decode_attention_rows(c["q"], c["q_dtype"], c["kv"], c["kv_dtype"], c["table"], c["lens"],
                                              c["P"], scale, c["ks"], c["vs"])


def _tril_reference(c, scale):
    """Bottom-right-aligned causal mask as numpy's tril with offset L - n, softmax
    and logsumexp from scipy, over every (request, row, head)."""
    qf = oracle.decode_storage(c["q"], c["q_dtype"])
    B, n, Hq, D = qf.shape
    Hkv = c["kv"].shape[2]
    g = Hq // Hkv
    out = np.zeros((B, n, Hq, D))
    lse = np.full((B, n, Hq), -np.inf)
    for b in range(B):
        L = int(c["lens"][b])
        if L == 0:
            continue
        K, V = _dense_history(c, b)
        keep = np.tril(np.ones((n, L), dtype=bool), k=L - n)
        for h in range(Hq):
            S = scale * (qf[b, :, h, :] @ K[:, h // g, :].T)          # [n][L]
            S = np.where(keep, S, -np.inf)
            for i in range(n):
                if not keep[i].any():
                    continue
                p = scipy.special.softmax(S[i])
                out[b, i, h] = p @ V[:, h // g, :]
                lse[b, i, h] = scipy.special.logsumexp(S[i])
    return out, lse


@pytest.mark.parametrize("kv_dtype", [F32, BF16, FP8])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1)])
def test_every_token_a_row_equals_torch_causal_sdpa(kv_dtype, Hq, Hkv):
    """n = L: the step is causal self-attention over the whole sequence, which
    torch's scaled_dot_product_attention(is_causal=True) computes."""
    rng = np.random.default_rng(11 + Hq + Hkv + kv_dtype)
    n = 21
    c = _case(rng, 2, n, Hq, Hkv, 64 if kv_dtype == FP8 else 32, [n, n], kv_dtype)
    scale = 0.3
    out, lse = _run(c, scale)
    qf = oracle.decode_storage(c["q"], c["q_dtype"])
    for b in range(2):
        K, V = _dense_history(c, b)
        g = Hq // Hkv
        qt = torch.from_numpy(qf[b].transpose(1, 0, 2).copy())[None]                      # [1][Hq][n][D]
        kt = torch.from_numpy(K.transpose(1, 0, 2).copy()).repeat_interleave(g, dim=0)[None]
        vt = torch.from_numpy(V.transpose(1, 0, 2).copy()).repeat_interleave(g, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
        ref = ref[0].numpy().transpose(1, 0, 2)                                             # [n][Hq][D]
        assert np.max(np.abs(out[b] - ref)) < 1e-12


@pytest.mark.parametrize("kv_dtype", [F32, BF16, FP8])
def test_rows_match_triangular_mask_brute_force(kv_dtype):
    rng = np.random.default_rng(5 + kv_dtype)
    n, Hq, Hkv = 3, 8, 2
    lens = [3, 4, 17, 40, 16, 33]
    c = _case(rng, len(lens), n, Hq, Hkv, 64, lens, kv_dtype)
    out, lse = _run(c, 0.125)
    ro, rl = _tril_reference(c, 0.125)
    assert np.max(np.abs(out - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_rows_without_visible_positions_are_empty():
    """L < n: the first n - L rows see nothing (out 0, lse -inf); the rest are
    ordinary rows; L = 0 empties every row."""
    rng = np.random.default_rng(3)
    n = 4
    lens = [0, 1, 2, 3, 4]
    c = _case(rng, len(lens), n, 4, 2, 32, lens)
    out, lse = _run(c, 0.2)
    ro, rl = _tril_reference(c, 0.2)
    for b, L in enumerate(lens):
        for i in range(n):
            if i < n - L:
                assert np.all(out[b, i] == 0.0) and np.all(lse[b, i] == -np.inf)
            else:
                assert np.max(np.abs(out[b, i] - ro[b, i])) < 1e-12
                assert np.max(np.abs(lse[b, i] - rl[b, i])) < 1e-12


def test_single_row_is_the_decode_oracle():
    rng = np.random.default_rng(9)
    lens = [1, 15, 16, 17, 50]
    c = _case(rng, len(lens), 1, 8, 2, 64, lens, BF16)
    out, lse = _run(c, 0.1)
    ro, rl = oracle.paged_decode_attention(c["q"][:, 0], c["q_dtype"], c["kv"], c["kv_dtype"], c["table"], c["lens"],
                                           c["P"], 0.1)
    assert np.array_equal(out[:, 0], ro) and np.array_equal(lse[:, 0], rl)


def test_last_row_sees_the_whole_history():
    """The last row is the newest token: it attends the whole history, as the
    single query of a plain decode step does."""
    rng = np.random.default_rng(10)
    lens = [5, 16, 31]
    c = _case(rng, len(lens), 3, 4, 4, 32, lens)
    out, lse = _run(c, 0.25)
    ro, rl = oracle.paged_decode_attention(c["q"][:, 2], c["q_dtype"], c["kv"], c["kv_dtype"], c["table"], c["lens"],
                                           c["P"], 0.25)
    assert np.max(np.abs(out[:, 2] - ro)) < 1e-13


@pytest.mark.parametrize("planted", [lambda L, n, i: max(0, L - n + i),          # own position left out
                                     lambda L, n, i: min(L, i + 1)])             # mask aligned to the first token
def test_planted_mask_mistakes_are_caught(monkeypatch, planted):
    rng = np.random.default_rng(12)
    n = 5
    lens = [n, 23]
    c = _case(rng, 2, n, 4, 2, 32, lens)
    good = _tril_reference(c, 0.2)
    monkeypatch.setattr(orows, "visible_tokens", planted)
    out, lse = _run(c, 0.2)
    bad = np.nanmax(np.abs(out - good[0]))
    assert not np.isfinite(bad) or bad > 1e-6


# ---- MLA: every row over the head-shared latent, keys 576 wide, values its first 512

def _mla_case(rng, B, n, H, lens, P=64, Dk=576):
    lens = np.asarray(lens, dtype=np.int32)
    npg = (lens + P - 1) // P
    num_pages = int(npg.sum()) + 2
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, max(1, int(npg.max()))), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        table[b, :npg[b]] = perm[at:at + npg[b]]
        at += npg[b]
    q = wl.to_bf16_bits((0.5 * rng.standard_normal((B, n, H, Dk))).astype(np.float32))
    kv = wl.to_bf16_bits((0.5 * rng.standard_normal((num_pages, P, Dk))).astype(np.float32))
    return q, kv, table, lens, P


def _mla_latent(kv, table, b, L, P):
    C = np.zeros((L, kv.shape[2]))
    for t in range(L):
        C[t] = oracle.decode_storage(kv[table[b, t // P], t % P], BF16)
    return C


def test_mla_every_token_a_row_equals_torch_causal_sdpa():
    rng = np.random.default_rng(31)
    n, H = 19, 8
    q, kv, table, lens, P = _mla_case(rng, 2, n, H, [n, n], P=16)
    scale = 1 / np.sqrt(576)
    out, lse = oracle.mla_decode_attention_rows(q, kv, table, lens, P, scale)
    qf = oracle.decode_storage(q, BF16)
    for b in range(2):
        C = _mla_latent(kv, table, b, n, P)
        qt = torch.from_numpy(qf[b].transpose(1, 0, 2).copy())[None]                     # [1][H][n][576]
        kt = torch.from_numpy(C).expand(H, n, 576)[None]
        vt = torch.from_numpy(C[:, :512].copy()).expand(H, n, 512)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
        assert np.max(np.abs(out[b] - ref[0].numpy().transpose(1, 0, 2))) < 1e-12


def test_mla_rows_match_triangular_mask_brute_force():
    rng = np.random.default_rng(32)
    n, H = 2, 4
    lens = [0, 1, 2, 64, 65, 130]
    q, kv, table, lens, P = _mla_case(rng, len(lens), n, H, lens)
    scale = 0.05
    out, lse = oracle.mla_decode_attention_rows(q, kv, table, lens, P, scale)
    qf = oracle.decode_storage(q, BF16)
    for b, L in enumerate(lens):
        C = _mla_latent(kv, table, b, int(L), P)
        keep = np.tril(np.ones((n, int(L)), dtype=bool), k=int(L) - n)
        for h in range(H):
            S = np.where(keep, scale * (qf[b, :, h, :] @ C.T), -np.inf) if L else np.zeros((n, 0))
            for i in range(n):
                if L == 0 or not keep[i].any():
                    assert np.all(out[b, i, h] == 0.0) and lse[b, i, h] == -np.inf
                    continue
                p = scipy.special.softmax(S[i])
                assert np.max(np.abs(out[b, i, h] - p @ C[:, :512])) < 1e-12
                assert abs(lse[b, i, h] - scipy.special.logsumexp(S[i])) < 1e-12


def test_mla_single_row_is_the_decode_oracle():
    rng = np.random.default_rng(33)
    q, kv, table, lens, P = _mla_case(rng, 3, 1, 8, [1, 64, 100])
    out, lse = oracle.mla_decode_attention_rows(q, kv, table, lens, P, 0.04)
    ro, rl = oracle.mla_decode_attention(q[:, 0], kv, table, lens, P, 0.04)
    assert np.array_equal(out[:, 0], ro) and np.array_equal(lse[:, 0], rl)

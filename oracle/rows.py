"""Multi-row decode queries, float64 (oracle; test infrastructure only).

A request's query rows in one step are its chunk length in prefill and one in
plain decode (SPLASH, §4.2 "Transition-aware scheduling": the per-request
q_i beside the live context s_i).  With multi-token prediction of depth 1 a
decode step processes 1 + 1 = 2 tokens per request (Analytical Provisioning,
App. B.1 "Model Configuration" and the batch-size mapping that counts
k * (1 + MTP depth) tokens per request).  Each row attends like the single
row of attention.py, except that it sees the history only up to its own
position.

Readings where the pages are silent (numbered after those of append.py):

13. A request with n rows brings the last n tokens of its history, already
    appended (reading 4): row i, 0 <= i < n, is the token at position
    L - n + i and attends positions t <= L - n + i.  Every row sees the older
    history whole; among the new rows the mask is causal.
14. q and out are [B][n][Hq][D] (a request's rows in position order, heads
    inside a row as in the single-row case), lse is [B][n][Hq]; one call has
    one n for every request.  MLA likewise: q [B][n][H][576], out
    [B][n][H][512], every row over the head-shared latent.
15. A row that sees no position (L - n + i < 0, possible only when L < n)
    gives out = 0 and lse = -inf, as an empty history does (reading 5).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import gather_history, dense_attention, _dequant
from .formats import decode_storage, BF16


def visible_tokens(L: int, n: int, i: int) -> int:
    """Number of history positions row i of n sees in a history of L tokens (reading 13)."""
    return max(0, L - n + i + 1)


def paged_decode_attention_rows(q, q_dtype: int, kv_pages, kv_dtype: int, page_table, seq_lens,
                                page_size: int, scale: float, k_scale=None, v_scale=None,
                                requests: Optional[Sequence[int]] = None):
    """GQA paged decode attention with n query rows per request.  q [B][n][Hq][D];
    returns float64 out [B][n][Hq][D] and lse [B][n][Hq] (requests not listed in
    ``requests`` are left NaN)."""
    qf = decode_storage(q, q_dtype)
    B, n, Hq, D = qf.shape
    Hkv = kv_pages.shape[2]
    g = Hq // Hkv
    out = np.full((B, n, Hq, D), np.nan)
    lse = np.full((B, n, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(seq_lens[b])
        if L > 0:
            k_raw, v_raw = gather_history(kv_pages, page_table, b, L, page_size)
            K = _dequant(k_raw, kv_dtype, k_scale)          # [L][Hkv][D]
            V = _dequant(v_raw, kv_dtype, v_scale)
        for i in range(n):
            vis = visible_tokens(L, n, i)
            if vis == 0:
                out[b, i] = 0.0
                lse[b, i] = -np.inf
                continue
            for j in range(Hkv):
                o, l = dense_attention(qf[b, i, j * g:(j + 1) * g], K[:vis, j, :], V[:vis, j, :], scale)
                out[b, i, j * g:(j + 1) * g] = o
                lse[b, i, j * g:(j + 1) * g] = l
    return out, lse


def mla_decode_attention_rows(q_bits, kv_bits, page_table, seq_lens, page_size: int, scale: float,
                              v_dim: int = 512, requests: Optional[Sequence[int]] = None):
    """Absorbed MLA decode with n query rows per request (readings 13-15).  q
    [B][n][H][576] and pages [num_pages][P][576] as bf16 bit patterns; returns
    float64 out [B][n][H][v_dim] and lse [B][n][H]."""
    qf = decode_storage(q_bits, BF16)
    B, n, H, Dk = qf.shape
    out = np.full((B, n, H, v_dim), np.nan)
    lse = np.full((B, n, H), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(seq_lens[b])
        if L > 0:
            C = decode_storage(gather_history(kv_bits, page_table, b, L, page_size, mla=True), BF16)
        for i in range(n):
            vis = visible_tokens(L, n, i)
            if vis == 0:
                out[b, i] = 0.0
                lse[b, i] = -np.inf
                continue
            o, l = dense_attention(qf[b, i], C[:vis], C[:vis, :v_dim], scale)
            out[b, i] = o
            lse[b, i] = l
    return out, lse

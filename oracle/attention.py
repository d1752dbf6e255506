"""Paged decode attention, float64, two passes (oracle; test infrastructure only).

Definition followed.  A decode step gives each request b exactly one query row
per head and attends over the request's whole cached history, the token
appended in this step included (OpWeave, App. A.2; Analytical Provisioning,
§2 and Fig. 1; SPLASH, §4.1 "Handoff" and §4.2).  Every query head attends
the complete history (SPLASH, §3 "Computation").  For each b < B, h < Hq:

    L = seq_lens[b];  j = h // (Hq // Hkv)
    k_t, v_t = gathered K and V of KV head j for token t < L
    s_t = scale * <q[b, h], k_t>
    m = max_t s_t;  w_t = exp(s_t - m);  Z = sum_t w_t
    out[b, h] = sum_t w_t v_t / Z;  lse[b, h] = m + ln Z

MLA (absorbed): one head-shared latent c_t of 576 values per token (SPLASH, §2:
the latent cache has no head axis; Analytical Provisioning, App. B.1:
512 + 64 = 576); every head uses k_t = c_t and v_t = c_t[:512].

Readings where the pages are silent (each is a choice, stated once here):

1. ``scale`` multiplies q.k before a natural-exponential softmax.
2. ``lse`` is the natural log of sum_t exp(s_t), max included.
3. Query head h uses KV head h // (Hq / Hkv) (contiguous groups).
4. seq_lens[b] counts every cached token including this step's; the only
   mask is t < L (the single query is the last position).
5. L = 0 gives out = 0 and lse = -inf.
6. page_table is int32 [B][max_pages]; entries at or past ceil(L/P) are
   never read (they may hold -1).
7. Slots of the last page at or past L are not history; their contents
   (possibly NaN) never reach the result.
8. GQA pages are laid out [num_pages][2 (K, V)][Hkv][P][D]; MLA pages
   [num_pages][P][576].  Only gather_history knows the layout.  In an fp8
   cache (uint8 storage) each V block [P][D] is kept in 16-token tiles;
   with DL = D / 16, token s of the tile (s = slot % 16) and dim d sit at byte
       1024 * ((d mod DL) div 4) + 256 * (s div 4) + 16 * (d div DL)
       + 4 * (d mod 4) + (s mod 4)
   of the tile, the tile at byte 16 * D * (slot div 16) of the block: the
   codes of four consecutive tokens for one dim are adjacent.  K blocks and
   bf16 / fp32 caches are row-major [P][D].
9. fp8 K/V dequantise as e4m3fn(code) * scale[j], one fp32 scale per KV head
   for K and one for V (SPLASH, App. B.1 mentions the scales traveling with
   the FP8 cache; the granularity is a reading).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .formats import decode_storage, FP8


def fp8_v_byte(slot, d, head_dim: int):
    """Byte of (slot, dim d) within an fp8 V block of one (page, KV head)
    (reading 8).  Works elementwise on integer arrays."""
    if head_dim % 64 != 0:
        raise ValueError("the tiled fp8 V layout is defined for head_dim a multiple of 64")
    DL = head_dim // 16
    tile, s = slot // 16, slot % 16
    within = 1024 * ((d % DL) // 4) + 256 * (s // 4) + 16 * (d // DL) + 4 * (d % 4) + (s % 4)
    return 16 * head_dim * tile + within


def gather_history(kv_pages: np.ndarray, page_table: np.ndarray, b: int, length: int,
                   page_size: int, mla: bool = False):
    """Explicitly gather request b's first ``length`` tokens, in logical order, still
    in storage format.  GQA: returns (K, V) each [L][Hkv][D]; MLA: C [L][576]."""
    t = np.arange(length, dtype=np.int64)
    pg = page_table[b, t // page_size].astype(np.int64)
    r = t % page_size
    if mla:
        return kv_pages[pg, r, :]
    k = kv_pages[pg, 0, :, r, :]
    if kv_pages.dtype != np.uint8:
        return k, kv_pages[pg, 1, :, r, :]
    # fp8: V blocks are tiled (reading 8); pick each (token, dim) byte
    Hkv, D = kv_pages.shape[2], kv_pages.shape[4]
    if page_size % 16 != 0:
        raise ValueError("the tiled fp8 V layout is defined for pages of a multiple of 16 tokens")
    blocks = kv_pages[pg, 1].reshape(length, Hkv, page_size * D)          # [L][Hkv][P*D]
    byte = fp8_v_byte(r[:, None], np.arange(D, dtype=np.int64)[None, :], D)  # [L][D]
    v = np.take_along_axis(blocks, np.broadcast_to(byte[:, None, :], (length, Hkv, D)), axis=2)
    return k, v


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """One head group against dense float64 history: q [g][Dk], k [L][Dk], v [L][Dv].
    Two passes: the max first, then the weights, their sum and the weighted values."""
    g = q.shape[0]
    L = k.shape[0]
    if L == 0:
        return np.zeros((g, v.shape[1])), np.full(g, -np.inf)
    s = scale * (q @ k.T)                       # [g][L]
    m = s.max(axis=1, keepdims=True)            # pass 1
    w = np.exp(s - m)                           # pass 2
    z = w.sum(axis=1, keepdims=True)
    out = (w @ v) / z
    lse = (m + np.log(z))[:, 0]
    return out, lse


def _dequant(x, dtype, scale_vec):
    y = decode_storage(x, dtype)
    if dtype == FP8:
        y = y * np.asarray(scale_vec, dtype=np.float32).astype(np.float64)[None, :, None]
    return y


def paged_decode_attention(q, q_dtype: int, kv_pages, kv_dtype: int, page_table, seq_lens,
                           page_size: int, scale: float, k_scale=None, v_scale=None,
                           requests: Optional[Sequence[int]] = None):
    """GQA/MQA/MHA paged decode attention.  Returns float64 out [B][Hq][D] and lse [B][Hq]
    (rows of requests not listed in ``requests`` are left NaN)."""
    qf = decode_storage(q, q_dtype)
    B, Hq, D = qf.shape
    Hkv = kv_pages.shape[2]
    g = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(seq_lens[b])
        if L == 0:
            out[b] = 0.0
            lse[b] = -np.inf
            continue
        k_raw, v_raw = gather_history(kv_pages, page_table, b, L, page_size)
        K = _dequant(k_raw, kv_dtype, k_scale)          # [L][Hkv][D]
        V = _dequant(v_raw, kv_dtype, v_scale)
        for j in range(Hkv):
            o, l = dense_attention(qf[b, j * g:(j + 1) * g], K[:, j, :], V[:, j, :], scale)
            out[b, j * g:(j + 1) * g] = o
            lse[b, j * g:(j + 1) * g] = l
    return out, lse


def mla_decode_attention(q_bits, kv_bits, page_table, seq_lens, page_size: int, scale: float,
                         v_dim: int = 512, requests: Optional[Sequence[int]] = None):
    """Absorbed MLA decode over the head-shared bf16 latent.  q [B][H][576] and pages
    [num_pages][P][576] as bf16 bit patterns.  Returns float64 out [B][H][v_dim], lse [B][H]."""
    qf = decode_storage(q_bits, 1)
    B, H, Dk = qf.shape
    out = np.full((B, H, v_dim), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(seq_lens[b])
        if L == 0:
            out[b] = 0.0
            lse[b] = -np.inf
            continue
        C = decode_storage(gather_history(kv_bits, page_table, b, L, page_size, mla=True), 1)
        o, l = dense_attention(qf[b], C, C[:, :v_dim], scale)
        out[b] = o
        lse[b] = l
    return out, lse


def attention_over_range(qf: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, t0: int, t1: int):
    """Attention of one head group over tokens [t0, t1) of a dense float64 history:
    the partial result that a split of the history produces."""
    return dense_attention(qf, k[t0:t1], v[t0:t1], scale)


def lse_merge(parts):
    """Combine partial results (o_i [g][Dv], lse_i [g]) of disjoint token ranges.
    lse = ln sum_i exp(lse_i); o = sum_i exp(lse_i - lse) o_i.  Empty parts carry
    lse_i = -inf and weigh nothing; if every part is empty the result is (0, -inf)."""
    lses = np.stack([p[1] for p in parts])                 # [n][g]
    os_ = np.stack([p[0] for p in parts])                  # [n][g][Dv]
    m = lses.max(axis=0)
    g = lses.shape[1]
    out = np.zeros(os_.shape[1:])
    lse = np.full(g, -np.inf)
    for h in range(g):
        if not math.isfinite(m[h]):
            continue
        w = np.exp(lses[:, h] - m[h])
        z = w.sum()
        lse[h] = m[h] + math.log(z)
        out[h] = (w[:, None] * os_[:, h, :]).sum(axis=0) / z
    return out, lse

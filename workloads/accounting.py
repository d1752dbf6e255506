"""Algorithmic byte and FLOP counts of one decode-attention call.

"Algorithmic" means what the method itself has to move: every cached K/V (or
latent) element of every live token read once, plus q, the outputs, the page
table entries that are used, seq_lens and the fp8 scales.  Workspace partials
and any re-reads are implementation overhead and are not counted.

The per-token KV volume follows "Analytical Provisioning for Attention-FFN
Disaggregated LLM Serving under Stochastic Workloads", App. B.2.1 (data volume
per token of the MLA latent: (d_c + d_rope) values of 2 bytes each).
"""
from __future__ import annotations

import numpy as np

from . import ELEM_BYTES, F32, FP8


def gqa_kv_bytes_per_token(kv_heads: int, head_dim: int, kv_dtype: int) -> int:
    return 2 * kv_heads * head_dim * ELEM_BYTES[kv_dtype]


def mla_kv_bytes_per_token(latent_dim: int, elem_bytes: int = 2) -> int:
    return latent_dim * elem_bytes


def gqa_bytes(seq_lens, page_size, q_heads, kv_heads, head_dim, q_dtype, kv_dtype, rows: int = 1) -> int:
    """With ``rows`` query rows per request, q, out and lse grow by that factor;
    the K/V history is still read once."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B = len(L)
    pages = int(((L + page_size - 1) // page_size).sum())
    kv = int(L.sum()) * gqa_kv_bytes_per_token(kv_heads, head_dim, kv_dtype)
    qb = rows * B * q_heads * head_dim * ELEM_BYTES[q_dtype]
    ob = qb                                   # out has q's dtype
    lse = rows * B * q_heads * 4
    scales = 2 * kv_heads * 4 if kv_dtype == FP8 else 0
    return kv + qb + ob + lse + 4 * pages + 4 * B + scales


def gqa_flops(seq_lens, q_heads, head_dim, rows: int = 1) -> int:
    """Row i of n sees L - n + 1 + i positions."""
    L = np.asarray(seq_lens, dtype=np.int64)
    seen = sum(int(np.maximum(L - rows + 1 + i, 0).sum()) for i in range(rows))
    return seen * q_heads * 2 * (head_dim + head_dim)


def mla_bytes(seq_lens, page_size, q_heads, latent_dim, v_dim, rows: int = 1) -> int:
    """With ``rows`` query rows per request, q, out and lse grow by that factor;
    the latent history is counted once, as the method needs it once."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B = len(L)
    pages = int(((L + page_size - 1) // page_size).sum())
    kv = int(L.sum()) * mla_kv_bytes_per_token(latent_dim)
    qb = rows * B * q_heads * latent_dim * 2
    ob = rows * B * q_heads * v_dim * 2
    lse = rows * B * q_heads * 4
    return kv + qb + ob + lse + 4 * pages + 4 * B


def mla_flops(seq_lens, q_heads, latent_dim, v_dim, rows: int = 1) -> int:
    """Row i of n sees L - n + 1 + i positions."""
    L = np.asarray(seq_lens, dtype=np.int64)
    seen = sum(int(np.maximum(L - rows + 1 + i, 0).sum()) for i in range(rows))
    return seen * q_heads * 2 * (latent_dim + v_dim)


__all__ = ["gqa_kv_bytes_per_token", "mla_kv_bytes_per_token", "gqa_bytes", "gqa_flops",
           "mla_bytes", "mla_flops", "F32"]

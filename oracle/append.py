"""Paged KV append (oracle; test infrastructure only).

Every decode step appends the new token's K/V (or, for MLA, its latent) to the
request's history before the history is read whole (Analytical Provisioning
for Attention-FFN Disaggregated LLM Serving, §2 and Fig. 1; OpWeave, §8
"paged KV-cache management").  FP8 E4M3 KV is stored with scales (SPLASH,
App. C.1 "FP8 E4M3 KV" and App. B.1).

Readings where the pages are silent (numbered after those of attention.py):

10. The new token of request b is written at logical position t = positions[b]:
    page page_table[b][t // P], slot t % P (the layouts of reading 8).  A
    negative position means no append for that request.
11. The new K/V (or latent) arrive in the query dtype; when the cache has the
    same dtype their bits are copied unchanged.
12. bf16 into an fp8 cache: y = fp32(x) / scale[j] with the division in fp32
    (round to nearest even), then the code of the e4m3fn value nearest to y,
    ties to the even code; |y| > 448 (infinity included) saturates to the
    largest finite magnitude with y's sign; NaN gives the code 0x7F.  The
    stored code then dequantises as e4m3fn(code) * scale[j] (reading 9).
"""
from __future__ import annotations

import numpy as np

from .attention import fp8_v_byte
from .formats import F32, BF16, FP8, fp8_e4m3fn_table

_TABLE = fp8_e4m3fn_table()
_POS = _TABLE[:0x7F]                      # codes 0x00 .. 0x7E: 0 .. 448, increasing


def fp8_e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each float32 value (reading 12), by search over
    the finite non-negative values; exact because every candidate and every
    midpoint between neighbours is representable in float64."""
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat.astype(np.float64)):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        sign = 0x80 if np.signbit(flat[i]) else 0x00
        a = abs(v)
        if a >= 448.0:
            out[i] = sign | 0x7E
            continue
        hi = int(np.searchsorted(_POS, a, side="left"))      # first value >= a
        if _POS[hi] == a:
            out[i] = sign | hi
            continue
        lo = hi - 1
        dl, dh = a - _POS[lo], _POS[hi] - a
        if dl < dh:
            c = lo
        elif dh < dl:
            c = hi
        else:
            c = lo if lo % 2 == 0 else hi
        out[i] = sign | c
    return out.reshape(y.shape)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _convert(x: np.ndarray, new_dtype: int, kv_dtype: int, scale) -> np.ndarray:
    """New values (storage format of new_dtype) to the cache's storage format."""
    if new_dtype == kv_dtype:
        return np.array(x, copy=True)
    if new_dtype == BF16 and kv_dtype == FP8:
        with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
            y = _bf16_bits_to_f32(x) / np.float32(scale)
        return fp8_e4m3fn_encode(y)
    raise ValueError(f"append from dtype {new_dtype} into a {kv_dtype} cache is not offered")


def kv_append(kv_pages, kv_dtype: int, k_new, v_new, new_dtype: int, page_table, positions,
              page_size: int, k_scale=None, v_scale=None) -> np.ndarray:
    """GQA cache [num_pages][2][Hkv][P][D] with request b's k_new[b] / v_new[b]
    ([Hkv][D] each) written at position positions[b]; returns a new array."""
    kv = np.array(kv_pages, copy=True)
    B, Hkv = k_new.shape[0], k_new.shape[1]
    for b in range(B):
        t = int(positions[b])
        if t < 0:
            continue
        pg = int(page_table[b, t // page_size])
        r = t % page_size
        for j in range(Hkv):
            ks = None if k_scale is None else k_scale[j]
            vs = None if v_scale is None else v_scale[j]
            kv[pg, 0, j, r, :] = _convert(k_new[b, j], new_dtype, kv_dtype, ks)
            v = _convert(v_new[b, j], new_dtype, kv_dtype, vs)
            if kv_dtype == FP8:
                # V blocks of an fp8 cache are tiled (attention.py, reading 8)
                D = kv.shape[4]
                block = kv[pg, 1, j].reshape(-1)
                block[fp8_v_byte(r, np.arange(D, dtype=np.int64), D)] = v
                kv[pg, 1, j] = block.reshape(kv.shape[3], D)
            else:
                kv[pg, 1, j, r, :] = v
    return kv


def mla_kv_append(kv_pages, latent_new, page_table, positions, page_size: int) -> np.ndarray:
    """MLA cache [num_pages][P][576] (bf16 bits) with request b's latent
    latent_new[b] written at position positions[b]; returns a new array."""
    kv = np.array(kv_pages, copy=True)
    for b in range(latent_new.shape[0]):
        t = int(positions[b])
        if t < 0:
            continue
        kv[int(page_table[b, t // page_size]), t % page_size, :] = latent_new[b]
    return kv

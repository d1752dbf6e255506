"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out in the storage formats
the library and the oracle both read (fp32, bf16 bit patterns, fp8-e4m3 codes
with per-head fp32 scales).  It holds none of the attention arithmetic: no dot
products, no softmax, no merging, no partitioning.

Workloads (one decode step of one attention layer on one rank):

* ``tiny``   - batch 4, 8 query / 2 KV heads, head_dim 64, page 16, lengths
               uniform in [1, 256], fp32 everywhere.
* ``llama8b``- batch 64, 32 / 8 heads, head_dim 128, page 16, bf16, lengths
               lognormal (median 2048, sigma 0.8) clipped to [16, 32768].
* ``skewed`` - batch 256, 32 / 8 heads, head_dim 128, page 16, bf16, 98 % of
               lengths lognormal (median 512, sigma 0.8) and 2 % uniform in
               [32768, 65536] placed at seeded positions.
* ``mla``    - batch 128, 128 query heads over one head-shared latent of
               512 + 64 = 576 values per token (values = first 512), page 64,
               bf16, lengths lognormal (median 4096, sigma 0.8) clipped to
               [64, 65536], latent and q ~ N(0, 0.5) (0.5 = standard deviation).
* ``longfp8``- batch 2, 64 / 8 heads, head_dim 128, page 16, 131072 tokens each,
               fp8-e4m3 K/V with one fp32 scale per KV head for K and one for V,
               bf16 q and output.

The latent width 512 + 64 follows the DeepSeek-V3 configuration in "Analytical
Provisioning for Attention-FFN Disaggregated LLM Serving under Stochastic
Workloads", App. B.1; "1K tokens = 1024" follows the SPLASH paper, §5.2.

Seeds: numpy ``Generator(PCG64(20260922 + k))`` for workload k = 1..5.  Draw
order: lengths, positions of long requests (skewed only), page permutation, q,
K/V (or latent).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BASE_SEED = 20260922

# storage dtype tags shared with the C ABI (include/decode_attn.h)
F32, BF16, FP8 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3"}
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1}

FP8_MAX = 448.0          # largest finite e4m3fn magnitude
FP8_POISON = 0x7F        # e4m3fn NaN (S.1111.111)


@dataclasses.dataclass(frozen=True)
class GQAConfig:
    name: str
    index: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: int
    kv_dtype: int
    lengths: str                # law tag, see draw_lengths
    value_std: float = 1.0

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass(frozen=True)
class MLAConfig:
    name: str
    index: int
    batch: int
    q_heads: int
    latent_dim: int             # d_c + d_rope = 576
    v_dim: int                  # d_c = 512
    page_size: int
    lengths: str
    value_std: float = 0.5

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.latent_dim)


TINY = GQAConfig("tiny", 1, 4, 8, 2, 64, 16, F32, F32, "uniform:1:256")
LLAMA8B = GQAConfig("llama8b", 2, 64, 32, 8, 128, 16, BF16, BF16,
                    "lognormal:2048:0.8:16:32768")
SKEWED = GQAConfig("skewed", 3, 256, 32, 8, 128, 16, BF16, BF16,
                   "skewed:512:0.8:16:32768:0.02:32768:65536")
MLA = MLAConfig("mla", 4, 128, 128, 576, 512, 64, "lognormal:4096:0.8:64:65536")
LONGFP8 = GQAConfig("longfp8", 5, 2, 64, 8, 128, 16, BF16, FP8, "fixed:131072")

CONFIGS = {c.name: c for c in (TINY, LLAMA8B, SKEWED, MLA, LONGFP8)}


def draw_lengths(rng: np.random.Generator, batch: int, law: str) -> np.ndarray:
    """Per-request history lengths (tokens already in the cache, this step's included)."""
    parts = law.split(":")
    kind = parts[0]
    if kind == "uniform":
        lo, hi = int(parts[1]), int(parts[2])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    if kind == "fixed":
        return np.full(batch, int(parts[1]), dtype=np.int32)
    if kind == "lognormal":
        med, sigma, lo, hi = float(parts[1]), float(parts[2]), int(parts[3]), int(parts[4])
        x = np.rint(rng.lognormal(mean=math.log(med), sigma=sigma, size=batch))
        return np.clip(x, lo, hi).astype(np.int32)
    if kind == "skewed":
        med, sigma, lo, hi = float(parts[1]), float(parts[2]), int(parts[3]), int(parts[4])
        frac, llo, lhi = float(parts[5]), int(parts[6]), int(parts[7])
        n_long = int(round(frac * batch))
        short = np.clip(np.rint(rng.lognormal(math.log(med), sigma, size=batch - n_long)), lo, hi)
        long_ = rng.integers(llo, lhi + 1, size=n_long)
        where = rng.permutation(batch)[:n_long]
        out = np.empty(batch, dtype=np.int64)
        mask = np.zeros(batch, dtype=bool)
        mask[where] = True
        out[mask] = long_
        out[~mask] = short
        return out.astype(np.int32)
    raise ValueError(f"unknown length law {law!r}")


def pages_needed(seq_lens: np.ndarray, page_size: int) -> np.ndarray:
    return (seq_lens.astype(np.int64) + page_size - 1) // page_size


def build_page_table(rng: np.random.Generator, seq_lens: np.ndarray, page_size: int,
                     extra_pages: int = 0, pad_to: Optional[int] = None):
    """Random physical placement: ids = permutation of all referenced (+ extra) pages,
    handed to (request, logical page) in row-major order.  Unused entries are -1."""
    npg = pages_needed(seq_lens, page_size)
    total = int(npg.sum())
    num_pages = total + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    width = int(npg.max()) if len(npg) else 0
    if pad_to is not None:
        width = max(width, pad_to)
    width = max(width, 1)
    table = np.full((len(seq_lens), width), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    unreferenced = perm[total:]
    return table, num_pages, unreferenced


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_fp8_per_head(x: np.ndarray, head_axis: int):
    """Per-head symmetric e4m3fn quantiser: scale = amax / 448 over the head's values,
    code = RNE(clamp(x / scale, +-448)).  Returns (uint8 codes, float32 scales)."""
    import torch
    xm = np.moveaxis(x, head_axis, 0)
    amax = np.abs(xm.reshape(xm.shape[0], -1)).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    shape = [1] * x.ndim
    shape[head_axis] = -1
    y = (x.astype(np.float32) / scale.reshape(shape)).astype(np.float32)
    y = np.clip(y, -FP8_MAX, FP8_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclasses.dataclass
class GQACase:
    cfg: GQAConfig
    seq_lens: np.ndarray        # int32 [B]
    page_table: np.ndarray      # int32 [B][max_pages], -1 padded
    num_pages: int
    q: np.ndarray               # [B][Hq][D]: float32, or uint16 bf16 bits
    kv: np.ndarray              # [num_pages][2][Hkv][P][D]: float32 / uint16 bf16 / uint8 fp8
    k_scale: Optional[np.ndarray]   # float32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray]
    scale: float
    unreferenced: np.ndarray    # physical ids of pages no request uses


@dataclasses.dataclass
class MLACase:
    cfg: MLAConfig
    seq_lens: np.ndarray
    page_table: np.ndarray
    num_pages: int
    q: np.ndarray               # uint16 bf16 bits [B][Hq][576]
    kv: np.ndarray              # uint16 bf16 bits [num_pages][P][576]
    scale: float
    unreferenced: np.ndarray


def _normal(rng, shape, std, dtype=np.float32):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def fp8_v_tile_index(page_size: int, head_dim: int) -> np.ndarray:
    """Storage format of an fp8 cache's V blocks: the [P][D] block of one
    (page, KV head) is kept in 16-token tiles, and within a tile the code of
    token t and dim d (with DL = D / 16) sits at byte
        1024 * ((d % DL) // 4) + 16 * (16 * ((t % 16) // 4) + d // DL) + 4 * (d % 4) + t % 4,
    i.e. for each group of four tokens and each dim their four codes are
    adjacent.  Returns the storage byte of every (t, d), shape [P][D]."""
    P, D = page_size, head_dim
    if D % 64 != 0 or P % 16 != 0:
        raise ValueError("the tiled fp8 V format needs head_dim a multiple of 64 and pages of 16k tokens")
    DL = D // 16
    t = np.arange(P)[:, None]
    d = np.arange(D)[None, :]
    return ((t // 16) * 16 * D + 1024 * ((d % DL) // 4) + 16 * (16 * ((t % 16) // 4) + d // DL)
            + 4 * (d % 4) + t % 4).astype(np.int64)


def fp8_v_to_storage(v: np.ndarray) -> np.ndarray:
    """Logical fp8 V codes [..][P][D] -> the tiled storage of the same shape.
    The byte formula of fp8_v_tile_index is an axis permutation: with
    t = 16 a + 4 b + c and d = DL e + 4 f + g, storage is ordered
    [a][f][b][e][g][c], so one transpose lays it out."""
    P, D = v.shape[-2:]
    fp8_v_tile_index(P, D)                                   # validates the shape
    DL = D // 16
    lead = v.shape[:-2]
    x = v.reshape(lead + (P // 16, 4, 4, 16, DL // 4, 4))   # a, b, c, e, f, g
    n = len(lead)
    x = x.transpose(tuple(range(n)) + (n, n + 4, n + 1, n + 3, n + 5, n + 2))
    return np.ascontiguousarray(x).reshape(v.shape)


def fp8_v_from_storage(v: np.ndarray) -> np.ndarray:
    """Tiled storage of fp8 V codes [..][P][D] -> logical [..][P][D] (token-major)."""
    P, D = v.shape[-2:]
    idx = fp8_v_tile_index(P, D).reshape(-1)
    flat = v.reshape(v.shape[:-2] + (P * D,))
    return flat[..., idx].reshape(v.shape)


def _poison_tail_gqa(kv, seq_lens, table, page_size, kv_dtype, unreferenced):
    for b, L in enumerate(seq_lens):
        r = int(L) % page_size
        if L > 0 and r:
            pg = table[b, (int(L) - 1) // page_size]
            _poison(kv, (pg, slice(None), slice(None), slice(r, None)), kv_dtype)
    for pg in unreferenced:
        _poison(kv, (pg,), kv_dtype)


def _poison(arr, idx, kv_dtype):
    if kv_dtype == F32:
        arr[idx] = np.float32(np.nan)
    elif kv_dtype == BF16:
        arr[idx] = np.uint16(0x7FC0)
    else:
        arr[idx] = np.uint8(FP8_POISON)


def make_gqa_case(cfg: GQAConfig, *, seq_lens: Optional[np.ndarray] = None, batch: Optional[int] = None,
                  seed: Optional[int] = None, poison: bool = False, extra_pages: int = 0,
                  pad_to: Optional[int] = None, scale: Optional[float] = None) -> GQACase:
    """Draw one paged GQA decode input.  ``seq_lens`` overrides the length law (edge cases);
    ``poison`` fills tail slots and unreferenced pages with NaN (fp8: 0x7F)."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    B = cfg.batch if batch is None else batch
    if seq_lens is None:
        seq_lens = draw_lengths(rng, B, cfg.lengths)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    table, num_pages, unref = build_page_table(rng, seq_lens, cfg.page_size, extra_pages, pad_to)
    num_pages = max(num_pages, 1)
    q32 = _normal(rng, (B, cfg.q_heads, cfg.head_dim), cfg.value_std)
    kv32 = _normal(rng, (num_pages, 2, cfg.kv_heads, cfg.page_size, cfg.head_dim), cfg.value_std)
    q = q32 if cfg.q_dtype == F32 else to_bf16_bits(q32)
    k_scale = v_scale = None
    if cfg.kv_dtype == F32:
        kv = kv32
    elif cfg.kv_dtype == BF16:
        kv = to_bf16_bits(kv32)
    else:
        kc, k_scale = quantize_fp8_per_head(kv32[:, 0], head_axis=1)
        vc, v_scale = quantize_fp8_per_head(kv32[:, 1], head_axis=1)
        kv = np.stack([kc, vc], axis=1)
    del kv32
    if poison:
        _poison_tail_gqa(kv, seq_lens, table, cfg.page_size, cfg.kv_dtype, unref)
    if cfg.kv_dtype == FP8:
        kv[:, 1] = fp8_v_to_storage(kv[:, 1])
    return GQACase(cfg, seq_lens, table, num_pages, q, kv, k_scale, v_scale,
                   cfg.scale if scale is None else float(scale), unref)


def make_mla_case(cfg: MLAConfig, *, seq_lens: Optional[np.ndarray] = None, batch: Optional[int] = None,
                  seed: Optional[int] = None, poison: bool = False, extra_pages: int = 0,
                  pad_to: Optional[int] = None, scale: Optional[float] = None,
                  q_heads: Optional[int] = None) -> MLACase:
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    B = cfg.batch if batch is None else batch
    if seq_lens is None:
        seq_lens = draw_lengths(rng, B, cfg.lengths)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    H = cfg.q_heads if q_heads is None else q_heads
    table, num_pages, unref = build_page_table(rng, seq_lens, cfg.page_size, extra_pages, pad_to)
    num_pages = max(num_pages, 1)
    q = to_bf16_bits(_normal(rng, (B, H, cfg.latent_dim), cfg.value_std))
    kv = to_bf16_bits(_normal(rng, (num_pages, cfg.page_size, cfg.latent_dim), cfg.value_std))
    if poison:
        for b, L in enumerate(seq_lens):
            r = int(L) % cfg.page_size
            if L > 0 and r:
                kv[table[b, (int(L) - 1) // cfg.page_size], r:] = np.uint16(0x7FC0)
        for pg in unref:
            kv[pg] = np.uint16(0x7FC0)
    return MLACase(cfg, seq_lens, table, num_pages, q, kv,
                   cfg.scale if scale is None else float(scale), unref)

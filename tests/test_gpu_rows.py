"""GPU parity of multi-row decode attention (decode_attn_paged_rows, through
the C ABI) with the oracle: max-abs on out and lse within the tolerances of
the single-row path, over dtypes, head shapes, row counts, lengths shorter
than the row count, poisoned tails and forced splits (where a piece may hold
no position some row sees)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import to_dev_storage, out_to_f64, assert_out_close, TOL_LSE
from oracle.formats import F32, BF16, FP8

pytestmark = pytest.mark.gpu

da = None


def setup_module(module):
    global da
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_471_amd as _da
    da = _da


def _run_case(q_dtype, kv_dtype, D, Hq, Hkv, n, lens, workers=0, seed=0, scale=None):
    cfg = wl.GQAConfig("rows", 40 + seed, len(lens), Hq, Hkv, D, 16, q_dtype, kv_dtype, "fixed:1")
    case = wl.make_gqa_case(cfg, seq_lens=np.asarray(lens, dtype=np.int32), poison=True, extra_pages=3,
                            seed=1000 + seed, scale=scale)
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal((len(lens), n, Hq, D)).astype(np.float32)
    q = q32 if q_dtype == F32 else wl.to_bf16_bits(q32)
    ro, rl = oracle.paged_decode_attention_rows(q, q_dtype, case.kv, kv_dtype, case.page_table, case.seq_lens,
                                                16, case.scale, case.k_scale, case.v_scale)
    dev = lambda x: None if x is None else torch.from_numpy(x).cuda()
    out, lse = da.decode_attn_paged_rows(to_dev_storage(q, q_dtype), to_dev_storage(case.kv, kv_dtype),
                                         dev(case.page_table), dev(case.seq_lens), case.scale,
                                         k_scale=dev(case.k_scale), v_scale=dev(case.v_scale), workers=workers)
    torch.cuda.synchronize()
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    err = assert_out_close(o, ro, kv_dtype, q_dtype == BF16, "rows")
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin) and np.all(l[~fin] == -np.inf), "empty rows must give lse = -inf"
    rel = np.abs(l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))
    assert (rel.max() if rel.size else 0.0) <= TOL_LSE[kv_dtype], f"lse rel err {rel.max():.3e}"
    return out, lse


LENS = [0, 1, 2, 3, 15, 16, 17, 18, 31, 33, 64, 100, 257, 1000]

SHAPES = [  # (Hq, Hkv, rows): members = rows * Hq / Hkv, padded to a power of two
    (8, 8, 2),     # g 1, 2 members
    (8, 2, 2),     # g 4, 8 members (the llama-8B grouping with MTP depth 1)
    (16, 8, 3),    # g 2, 6 members padded to 8
    (4, 4, 8),     # g 1, 8 rows
    (8, 4, 4),     # g 2, 8 members
    (8, 8, 3),     # g 1, 3 members padded to 4
    (8, 2, 4),     # g 4, 16 members (bf16: the matrix-core kernel's full tile)
    (4, 4, 12),    # g 1, 12 members padded to 16
]


@pytest.mark.parametrize("q_dtype,kv_dtype", [(F32, F32), (BF16, BF16), (BF16, FP8)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", SHAPES)
def test_rows_parity(q_dtype, kv_dtype, D, shape):
    # fp32 queries with more than 8 (row, head) pairs run in row blocks
    Hq, Hkv, n = shape
    _run_case(q_dtype, kv_dtype, D, Hq, Hkv, n, LENS, seed=Hq + 3 * Hkv + n + D)


# more (row, head) pairs than a kernel tile holds (16 on the matrix cores, 8 on
# the vector ALUs): the rows run in blocks, each block a request of its own
# over the same pages with its history cut where its last row's view ends
# (Hq, Hkv, rows, q dtype, kv dtype)
BLOCKED = [
    (32, 2, 2, BF16, BF16),    # g 16 x 2 rows: blocks of 1 row
    (128, 8, 2, BF16, FP8),    # the 128/8 head shape with MTP depth 1, fp8 cache
    (16, 2, 3, BF16, BF16),    # g 8 x 3 rows: blocks of 1 (2 does not divide 3)
    (8, 2, 8, BF16, BF16),     # g 4 x 8 rows: blocks of 4
    (12, 4, 6, BF16, BF16),    # g 3 x 6 rows: blocks of 3 (9 pairs)
    (8, 2, 4, F32, F32),       # fp32, g 4 x 4 rows: blocks of 2
    (8, 1, 16, F32, F32),      # fp32, g 8 x 16 rows: blocks of 1
]


@pytest.mark.parametrize("workers", [0, 7])
@pytest.mark.parametrize("shape", BLOCKED)
def test_rows_in_blocks(shape, workers):
    Hq, Hkv, n, qd, kd = shape
    _run_case(qd, kd, 128, Hq, Hkv, n, LENS, workers=workers, seed=11 * Hq + Hkv + 3 * n + workers)


# groups that are not a power of two (bf16 queries, the matrix-core kernel):
# (Hq, Hkv, rows), members = rows * Hq / Hkv padded to a power of two
ODD_GROUPS = [
    (28, 4, 1),    # g 7 (a 28/4 head shape), 7 members padded to 8
    (40, 8, 1),    # g 5
    (12, 2, 1),    # g 6
    (24, 2, 1),    # g 12, padded to 16
    (3, 1, 1),     # g 3, one KV head
    (28, 4, 2),    # g 7, 14 members (MTP depth 1)
    (15, 5, 3),    # g 3, 9 members padded to 16
    (10, 2, 3),    # g 5, 15 members
]


@pytest.mark.parametrize("kv_dtype", [BF16, FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", ODD_GROUPS)
def test_groups_not_a_power_of_two(kv_dtype, D, shape):
    Hq, Hkv, n = shape
    _run_case(BF16, kv_dtype, D, Hq, Hkv, n, LENS, seed=5 * Hq + Hkv + 7 * n + D)


@pytest.mark.parametrize("workers", [1, 5, 333])
def test_group_of_seven_under_forced_splits(workers):
    _run_case(BF16, BF16, 128, 28, 4, 2, LENS, workers=workers, seed=70 + workers)


@pytest.mark.parametrize("workers", [1, 3, 64, 2000])
@pytest.mark.parametrize("shape", [(8, 2, 2), (4, 4, 8), (16, 8, 3), (8, 2, 4)])
def test_rows_parity_under_forced_splits(workers, shape):
    """Many workers give every page its own piece, so the last page of a
    history is a piece that the earlier rows see nothing of; one worker runs
    every stream whole."""
    Hq, Hkv, n = shape
    _run_case(BF16, BF16, 128, Hq, Hkv, n, [1, 2, 7, 16, 17, 18, 23, 32, 33, 500], workers=workers, seed=workers)


def test_single_row_equals_decode_attn_paged():
    cfg = wl.GQAConfig("r1", 61, 9, 32, 8, 128, 16, BF16, BF16, "uniform:1:700")
    case = wl.make_gqa_case(cfg, poison=True)
    dev = lambda x: torch.from_numpy(x).cuda()
    q = to_dev_storage(case.q, BF16)
    kv = to_dev_storage(case.kv, BF16)
    o1, l1 = da.decode_attn_paged(q, kv, dev(case.page_table), dev(case.seq_lens), case.scale)
    o2, l2 = da.decode_attn_paged_rows(q[:, None].contiguous(), kv, dev(case.page_table), dev(case.seq_lens),
                                       case.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2[:, 0].view(torch.int16)) and torch.equal(l1, l2[:, 0])


def test_mtp2_at_full_llama8b_size_whole():
    """The llama-8B-shaped batch (64 requests, lognormal lengths up to 32k) with
    two rows per request, in the default launch: every row of every request
    against the oracle."""
    cfg = wl.LLAMA8B
    case = wl.make_gqa_case(cfg)
    rng = np.random.default_rng(77)
    B = cfg.batch
    q = wl.to_bf16_bits(rng.standard_normal((B, 2, cfg.q_heads, cfg.head_dim)).astype(np.float32))
    dev = lambda x: torch.from_numpy(x).cuda()
    out, lse = da.decode_attn_paged_rows(to_dev_storage(q, BF16), to_dev_storage(case.kv, BF16),
                                         dev(case.page_table), dev(case.seq_lens), case.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode_attention_rows(q, BF16, case.kv, BF16, case.page_table, case.seq_lens, 16,
                                                case.scale)
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "non-finite output or lse"
    assert_out_close(o, ro, BF16, True, "rows")
    assert np.max(np.abs(l - rl) / np.maximum(1.0, np.abs(rl))) <= TOL_LSE[BF16]

"""The seeded generators: reproducible, and drawn from the stated laws."""
import math

import numpy as np

import workloads as wl


def test_reproducible():
    a = wl.make_gqa_case(wl.TINY)
    b = wl.make_gqa_case(wl.TINY)
    assert np.array_equal(a.seq_lens, b.seq_lens) and np.array_equal(a.kv, b.kv)
    assert np.array_equal(a.page_table, b.page_table) and np.array_equal(a.q, b.q)
    assert wl.TINY.seed == 20260923 and wl.LONGFP8.seed == 20260927


def test_length_laws():
    rng = np.random.default_rng(0)
    x = wl.draw_lengths(rng, 40000, wl.LLAMA8B.lengths)
    assert abs(np.median(x) / 2048 - 1) < 0.03 and x.min() >= 16 and x.max() <= 32768
    x = wl.draw_lengths(rng, 256, wl.SKEWED.lengths)
    assert (x >= 32768).sum() == 5 and x.max() <= 65536
    x = wl.draw_lengths(rng, 40000, wl.MLA.lengths)
    assert abs(np.median(x) / 4096 - 1) < 0.03 and x.min() >= 64
    x = wl.draw_lengths(rng, 1000, wl.TINY.lengths)
    assert x.min() >= 1 and x.max() <= 256


def test_page_table_is_a_permutation():
    c = wl.make_gqa_case(wl.TINY, extra_pages=5)
    npg = (c.seq_lens + 15) // 16
    used = np.concatenate([c.page_table[b, :n] for b, n in enumerate(npg)])
    assert sorted(np.concatenate([used, c.unreferenced]).tolist()) == list(range(c.num_pages))
    assert np.all(c.page_table[c.page_table >= 0] < c.num_pages)
    for b, n in enumerate(npg):
        assert np.all(c.page_table[b, n:] == -1)


def test_fp8_quantiser_uses_full_range_per_head():
    cfg = wl.GQAConfig("f", 5, 2, 4, 2, 64, 16, wl.BF16, wl.FP8, "fixed:40")
    c = wl.make_gqa_case(cfg)
    from oracle.formats import fp8_e4m3fn_to_f64
    for kv_i, sc in ((0, c.k_scale), (1, c.v_scale)):
        for j in range(2):
            v = fp8_e4m3fn_to_f64(c.kv[:, kv_i, j])
            assert np.nanmax(np.abs(v)) == 448.0
            assert sc[j] > 0


def test_fp8_poison_lands_outside_history_in_the_tiled_v_format():
    """With an fp8 cache the V blocks are stored tiled; read back in token
    order, every history token is finite and every slot past it is the NaN code."""
    cfg = wl.GQAConfig("p", 6, 3, 8, 2, 128, 16, wl.BF16, wl.FP8, "uniform:1:60")
    c = wl.make_gqa_case(cfg, poison=True, extra_pages=1)
    v = wl.fp8_v_from_storage(c.kv[:, 1])
    for b, L in enumerate(c.seq_lens):
        for t in range(int(L)):
            assert np.all(v[c.page_table[b, t // 16], :, t % 16] != wl.FP8_POISON)
        r = int(L) % 16
        if r:
            assert np.all(v[c.page_table[b, (int(L) - 1) // 16], :, r:] == wl.FP8_POISON)


def test_poison_only_outside_history():
    c = wl.make_gqa_case(wl.TINY, poison=True, extra_pages=3)
    for b, L in enumerate(c.seq_lens):
        for t in range(int(L)):
            assert np.all(np.isfinite(c.kv[c.page_table[b, t // 16], :, :, t % 16]))
    assert np.all(np.isnan(c.kv[c.unreferenced]))
    m = wl.make_mla_case(wl.MLAConfig("m", 4, 3, 2, 576, 512, 64, "uniform:1:200"), poison=True, extra_pages=1)
    assert np.all(m.kv[m.unreferenced] == 0x7FC0)

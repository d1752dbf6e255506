"""Pins of the KV-append oracle (oracle/append.py) against facts it does not
compute itself: the e4m3fn code table, torch's float8_e4m3fn cast (a library
routine, used where it is defined: finite values up to 448), round-to-nearest-
even ties worked out by hand, saturation, and the page layout read back
through gather_history.  Planted mistakes at the end check that the pins bite."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle import append as ap
from oracle.formats import F32, BF16, FP8

TABLE = oracle.fp8_e4m3fn_table()


def enc(x):
    return oracle.fp8_e4m3fn_encode(np.asarray(x, dtype=np.float32))


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = TABLE[codes].astype(np.float32)
    assert np.array_equal(enc(vals), codes)          # includes +0 -> 0x00 and -0 -> 0x80


def test_ties_go_to_the_even_code_and_neighbours_to_the_nearer():
    for c in range(0x7E):
        lo, hi = TABLE[c], TABLE[c + 1]
        mid = np.float32((lo + hi) / 2)               # exact: at most 5 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert enc(mid) == even, c
        assert enc(np.nextafter(mid, np.float32(0))) == c
        assert enc(np.nextafter(mid, np.float32(1e9))) == c + 1
        assert enc(-mid) == 0x80 | even


def test_hand_worked_values():
    # 2^-9 is the smallest subnormal (code 1); half of it ties to 0 (even)
    assert enc(2.0 ** -9) == 0x01 and enc(2.0 ** -10) == 0x00 and enc(1.5 * 2.0 ** -10) == 0x01
    # 1.0 = exponent field 7, mantissa 0; 1.0625 is halfway to 1.125 -> even code 0x38
    assert enc(1.0) == 0x38 and enc(1.0625) == 0x38 and enc(1.1875) == 0x3A
    # 240 = 1.875 * 2^7 -> 0x77; 448 = 1.75 * 2^8 is the largest finite value
    assert enc(240.0) == 0x77 and enc(448.0) == 0x7E


def test_saturation_and_nan():
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e30, np.inf], dtype=np.float32)
    assert np.all(enc(big) == 0x7E)
    assert np.all(enc(-big) == 0xFE)
    assert enc(np.float32(np.nan)) == 0x7F


def test_agrees_with_torch_cast_on_finite_range():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000)]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc(y), ref)


def _cache(num_pages, Hkv, P, D, dtype, rng):
    if dtype == F32:
        return rng.standard_normal((num_pages, 2, Hkv, P, D)).astype(np.float32)
    if dtype == BF16:
        return rng.integers(0, 1 << 16, (num_pages, 2, Hkv, P, D)).astype(np.uint16)
    return rng.integers(0, 256, (num_pages, 2, Hkv, P, D)).astype(np.uint8)


@pytest.mark.parametrize("new_dtype,kv_dtype", [(F32, F32), (BF16, BF16), (BF16, FP8)])
def test_append_lands_at_its_position_and_nowhere_else(new_dtype, kv_dtype):
    rng = np.random.default_rng(11)
    B, Hkv, P, D, maxp, npages = 5, 2, 16, 64, 4, 24
    kv = _cache(npages, Hkv, P, D, kv_dtype, rng)
    pt = rng.permutation(npages)[:B * maxp].reshape(B, maxp).astype(np.int32)
    pos = np.array([0, 15, 16, 63, -1], dtype=np.int32)
    if new_dtype == F32:
        kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
        vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    else:
        kn = (rng.standard_normal((B, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        vn = (rng.standard_normal((B, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ks = np.array([0.5, 2.0], dtype=np.float32)
    vs = np.array([0.25, 1.0], dtype=np.float32)
    out = oracle.kv_append(kv, kv_dtype, kn, vn, new_dtype, pt, pos, P, ks, vs)
    touched = np.zeros(kv.shape, dtype=bool)
    for b in range(B):
        t = int(pos[b])
        if t < 0:
            continue
        k_hist, v_hist = oracle.gather_history(out, pt, b, t + 1, P)
        if kv_dtype == new_dtype:
            assert np.array_equal(k_hist[t], kn[b]) and np.array_equal(v_hist[t], vn[b])
        else:
            # the stored code is the nearest e4m3 value of x / scale (checked by value)
            for hist, new, sc in ((k_hist, kn, ks), (v_hist, vn, vs)):
                x = oracle.bf16_bits_to_f64(new[b]) / sc[:, None]
                got = oracle.fp8_e4m3fn_to_f64(hist[t])
                lo_err = np.abs(got - x)
                # no other finite code is closer
                others = np.abs(TABLE[None, None, :0x7F] - np.abs(x)[..., None]).min(axis=-1)
                assert np.all(lo_err <= others + 1e-12)
        pg, r = int(pt[b, t // P]), t % P
        touched[pg, 0, :, r, :] = True
        if kv_dtype == FP8:
            # V of an fp8 cache is tiled: token r's codes sit at the generator's
            # storage bytes of (r, d)
            vt = touched[pg, 1].reshape(Hkv, P * D)
            vt[:, wl.fp8_v_tile_index(P, D)[r]] = True
            touched[pg, 1] = vt.reshape(Hkv, P, D)
        else:
            touched[pg, 1, :, r, :] = True
    assert np.array_equal(out[~touched], kv[~touched])


def test_fp8_v_tile_layout_matches_its_definition():
    """The oracle's byte map of a tiled fp8 V block: hand-worked bytes from the
    definition (16-token tiles; within a tile, DL = D / 16,
    byte = 1024 ((d mod DL) div 4) + 256 (s div 4) + 16 (d div DL) + 4 (d mod 4) + s mod 4),
    a bijection onto the block, and the same map as the input generator's."""
    from oracle.attention import fp8_v_byte
    assert fp8_v_byte(5, 9, 128) == 256 + 16 + 4 + 1
    # dim 7 of slot 0 at D = 128: (7 mod 8) div 4 = 1 -> 1024; 7 div 8 = 0; 7 mod 4 = 3 -> 12
    assert fp8_v_byte(0, 7, 128) == 1024 + 12
    assert fp8_v_byte(19, 0, 128) == 16 * 128 + 3            # second tile, s = 3
    assert fp8_v_byte(15, 63, 64) == 256 * 3 + 16 * 15 + 4 * 3 + 3
    for P, D in ((16, 64), (32, 128), (64, 64)):
        t = np.arange(P)[:, None]
        d = np.arange(D)[None, :]
        m = fp8_v_byte(t, d, D)
        assert sorted(m.reshape(-1).tolist()) == list(range(P * D))
        assert np.array_equal(m, wl.fp8_v_tile_index(P, D))
    with pytest.raises(ValueError):
        fp8_v_byte(0, 0, 32)


def test_mla_append():
    rng = np.random.default_rng(3)
    kv = rng.integers(0, 1 << 16, (10, 64, 576)).astype(np.uint16)
    pt = np.array([[3, 7], [1, 2], [9, 0]], dtype=np.int32)
    pos = np.array([64, 0, -1], dtype=np.int32)
    lat = rng.integers(0, 1 << 16, (3, 576)).astype(np.uint16)
    out = oracle.mla_kv_append(kv, lat, pt, pos, 64)
    assert np.array_equal(out[7, 0], lat[0]) and np.array_equal(out[1, 0], lat[1])
    mask = np.ones(kv.shape, dtype=bool)
    mask[7, 0] = mask[1, 0] = False
    assert np.array_equal(out[mask], kv[mask])


# ---- planted mistakes: a wrong tie rule or no saturation must fail a pin


def _encode_ties_up(y):
    y = np.asarray(y, dtype=np.float32)
    out = []
    for v in y.reshape(-1).astype(np.float64):
        a = abs(v)
        if a >= 448:
            c = 0x7E
        else:
            hi = int(np.searchsorted(ap._POS, a, side="left"))
            c = hi if ap._POS[hi] == a or (ap._POS[hi] - a) <= (a - ap._POS[hi - 1]) else hi - 1
        out.append((0x80 if v < 0 else 0) | c)
    return np.array(out, dtype=np.uint8)


def test_planted_tie_mistake_is_caught():
    mid = np.float32((TABLE[0x38] + TABLE[0x39]) / 2)     # 1.0625: the even code is 0x38
    assert _encode_ties_up(mid)[0] != 0x38 and enc(mid) == 0x38


def test_planted_overflow_mistake_is_caught():
    wrapped = np.float32(470.0)      # above the 448|480 midpoint
    # a converter that rounds without saturating lands on the NaN pattern
    naive = (np.float32(wrapped).view(np.uint32) + 0x7FFFF + ((np.float32(wrapped).view(np.uint32) >> 20) & 1)) >> 20
    assert int(naive) - (120 << 3) == 0x7F and enc(wrapped) == 0x7E

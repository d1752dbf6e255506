"""Storage formats decoded exactly to float64 (oracle; test infrastructure only).

* fp32: exact.
* bf16: the upper 16 bits of an IEEE binary32; decoding appends 16 zero bits.
* fp8 E4M3 as used for the KV cache (SPLASH, App. C.1 "FP8 E4M3 KV"): the OCP
  "E4M3FN" encoding - 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 is subnormal (m * 2^-9); there is no infinity and the single
  NaN pattern per sign is exponent 15 with mantissa 7; the largest finite
  magnitude is 1.75 * 2^8 = 448.  The pages name only "FP8 E4M3"; reading the
  OCP finite variant is an interpretation (it is the format the hardware
  converts natively).
"""
from __future__ import annotations

import numpy as np

F32, BF16, FP8 = 0, 1, 2


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3FN = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_e4m3fn_table() -> np.ndarray:
    return _E4M3FN.copy()


def fp8_e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3FN[np.asarray(codes, dtype=np.uint8)]


def decode_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(x)
    if dtype == FP8:
        return fp8_e4m3fn_to_f64(x)
    raise ValueError(f"unknown storage dtype {dtype}")

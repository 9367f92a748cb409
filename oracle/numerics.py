"""Exact bf16 <-> float64 conversion and rounding to bf16 (oracle; test-only).

bf16 is IEEE binary32 with the low 16 mantissa bits dropped: 1 sign bit,
8 exponent bits, 7 stored mantissa bits (froggydisk "LLM에서 KV 캐시는 얼마나
생길까", FP8 format table, BF16 row).  Every bf16 value is therefore exact in
float32 and float64.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float((2.0 - 2.0 ** -7) * 2.0 ** 127)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to the nearest bf16, ties to even; return bits.

    The quantum of a bf16 number with leading bit 2^k is 2^(k-7), but never
    below the subnormal quantum 2^-133.  Dividing by a power of two is exact
    in float64, so ``rint`` (which rounds half to even) does the rounding.
    Results beyond the largest finite bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = (a > 0) & np.isfinite(a)
    _, e = np.frexp(a[nz])              # a = f * 2^e, f in [0.5, 1): leading bit 2^(e-1)
    quantum = np.ldexp(1.0, np.maximum(e - 1 - 7, -133))
    r = np.rint(a[nz] / quantum) * quantum
    r[r > BF16_MAX] = np.inf
    out[nz] = r
    out[np.isinf(a)] = np.inf
    out = np.copysign(out, x)
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(x)] = np.uint16(0x7FC0)
    return bits


def round_to_bf16(x) -> np.ndarray:
    """float64 values rounded to bf16 (nearest-even), returned as float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x|: 2^(e-7) for |x| in [2^e, 2^(e+1)), at least 2^-133."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.ldexp(1.0, np.maximum(e - 1 - 7, -133))

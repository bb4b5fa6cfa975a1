"""Oracle widening and rounding between fp32 and the 16-bit formats.

The pages keep fp16/bf16 copies of the parameters and gradients next to fp32
master weights ("论文专题讲解：ZeRO：…", section "显存账"); they do not say how
the fp32 result is rounded back.  Reading taken: IEEE round-to-nearest, ties to
even (parity pinned against torch's CPU casts, a library routine).

Each function works from the formats' definitions with exact float64 arithmetic:
  bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits;
  fp16: 1 sign, 5 exponent (bias 15), 10 fraction bits, max finite 65504.
16-bit values travel as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)
F16_QNAN = np.uint16(0x7E00)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32: the 16 bits are the top half of the fp32 pattern."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def widen_f16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> fp32 (exact)."""
    h = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(h >> 15, -1.0, 1.0)
    e = (h >> 10) & 0x1F
    f = (h & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(f, -24),                      # subnormal: f * 2^-24
                   np.ldexp(1024.0 + f, (e - 25).astype(np.int32)))  # normal: (1 + f/1024) * 2^(e-15)
    mag = np.where(e == 0x1F, np.where(f == 0, np.inf, np.nan), mag)
    return (sign * mag).astype(np.float32)


def _round_even(x32: np.ndarray, frac_bits: int, emin: int, max_finite: float) -> np.ndarray:
    """Round fp32 values to the nearest value with `frac_bits` fraction bits and
    minimum normal exponent `emin` (ties to even); results beyond max_finite
    become +-inf.  Returns float64 values that the target format holds exactly
    (NaN stays NaN)."""
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.asarray(x32, dtype=np.float32).astype(np.float64)   # exact (sNaN -> NaN)
        _, e = np.frexp(np.abs(x))           # |x| = mant * 2^e, mant in [0.5, 1)
        binade = np.maximum(e - 1, emin)     # spacing is fixed below the normal range
        ulp = np.ldexp(1.0, (binade - frac_bits).astype(np.int32))
        q = np.rint(x / ulp)                 # x / ulp is exact; rint ties to even
        r = q * ulp
        r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, x), r)
    return np.where(np.isnan(x), np.nan, r)


def round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    r = _round_even(x32, 7, -126, float.fromhex("0x1.fep127"))
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(r), BF16_QNAN, bits).astype(np.uint16)


def round_to_f16(x32: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit patterns, round to nearest even."""
    r = _round_even(x32, 10, -14, 65504.0)
    a = np.abs(r)
    sign = np.where(np.signbit(r), 0x8000, 0).astype(np.int64)
    with np.errstate(invalid="ignore", divide="ignore"):
        _, e = np.frexp(np.where(np.isfinite(a), a, 1.0))
        binade = e - 1
        normal = a >= 2.0 ** -14
        exp_field = np.where(normal, binade + 15, 0)
        frac = np.where(normal, a / np.ldexp(1.0, (binade - 10).astype(np.int32)) - 1024.0,
                        a / 2.0 ** -24)
        frac = np.where(np.isfinite(frac), frac, 0).astype(np.int64)
    bits = sign | (exp_field.astype(np.int64) << 10) | frac
    bits = np.where(np.isinf(r), sign | 0x7C00, bits)
    bits = np.where(np.isnan(r), int(F16_QNAN), bits)
    return bits.astype(np.uint16)


def widen(storage: np.ndarray, kind: str) -> np.ndarray:
    """Slice storage -> fp32.  kind: 'f32' (float32 array), 'bf16' / 'f16' (uint16 bits)."""
    if kind == "f32":
        return np.asarray(storage, dtype=np.float32)
    if kind == "bf16":
        return widen_bf16(storage)
    if kind == "f16":
        return widen_f16(storage)
    raise ValueError(kind)


def narrow(x32: np.ndarray, kind: str) -> np.ndarray:
    """fp32 -> parameter storage ('f32' unchanged; 'bf16' / 'f16' rounded to nearest even)."""
    if kind == "f32":
        return np.asarray(x32, dtype=np.float32).copy()
    if kind == "bf16":
        return round_to_bf16(x32)
    if kind == "f16":
        return round_to_f16(x32)
    raise ValueError(kind)

"""Exact number-format helpers for the CSA oracle (test infrastructure only).

The oracle computes in float64.  Storage formats used by the decode path are
decoded here from their published definitions, never through a GPU library:

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.  Decoding is a
  16-bit left shift into a binary32 pattern, which is exact.  Encoding rounds
  to nearest, ties to even (RNE).  The pages store compressed KV and indexer
  keys as BF16 (page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, "Per-layer KV cache
  sizes"; page 1, dsv4/kernels/compressor/production_compress.py, the
  ``compressed.bfloat16()`` return).
* float32: numpy's own binary32 (RNE on conversion).

Nothing in this module is shared with the HIP library.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "f64_to_bf16_bits",
    "bf16_round_f64",
]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16 / int16 array) to float64 exactly."""
    b = np.asarray(bits)
    if b.dtype not in (np.uint16, np.int16):
        raise TypeError(f"bf16 bits must be uint16/int16, got {b.dtype}")
    u32 = b.view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round binary32 values to bfloat16 (RNE) and return the uint16 patterns.

    Rounding rule: add 0x7FFF plus the lowest kept bit, then truncate, which
    is round-half-to-even on the 16 discarded bits.  NaNs map to a quiet NaN.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_round_f64(x) -> np.ndarray:
    """Round float64 values directly to the nearest bfloat16 value (RNE).

    One rounding from the exact float64 value (no float32 step in between):
    a bfloat16 significand has 8 bits, so for |x| in [2^(e-1), 2^e) the spacing
    is 2^(e-8); subnormals keep the spacing of the smallest normal binade
    (2^-133).  Values beyond the largest finite bfloat16 overflow to +-inf.
    """
    v = np.asarray(x, dtype=np.float64)
    out = np.array(v, dtype=np.float64, copy=True)
    fin = np.isfinite(v) & (v != 0.0)
    if fin.any():
        _, e = np.frexp(v[fin])  # v = m * 2**e with 0.5 <= |m| < 1
        e = np.maximum(e, -125)
        spacing = np.ldexp(1.0, e - 8)
        q = np.rint(v[fin] / spacing) * spacing  # np.rint rounds half to even
        max_bf16 = float(np.ldexp(255.0, 120))  # 0x7F7F = (2 - 2^-7) * 2^127
        q = np.where(np.abs(q) > max_bf16, np.copysign(np.inf, q), q)
        out[fin] = q
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Bit patterns of :func:`bf16_round_f64` (the rounded value is exact in fp32)."""
    r = bf16_round_f64(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

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
* FP8 E4M3 (the OCP 8-bit floating point "E4M3FN" encoding): sign bit, 4
  exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; there is no
  infinity; the largest finite magnitude is 1.75 * 2^8 = 448.  The pages store
  indexer keys as FP8_E4M3 in the KV cache for the tensor-core scoring path
  (page 1, ``single_shot_inference.py``, comment "B2: FP8 tensor-core scoring
  path"); the codec below is written from the format's definition.
* FP4 E2M1 with E8M0 block scales (the element and scale formats of the OCP
  microscaling specification's MXFP4): an element is a sign bit, 2 exponent
  bits with bias 1 and 1 mantissa bit (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  exponent field 0 holds the subnormal 0.5); a scale is an unsigned 8-bit
  exponent, 2^(s - 127).  The pages plan an FP4 indexer cache paired with an
  FP4 tensor-core scoring kernel (page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md,
  C4 "Optional: Quantize indexer KV to FP4") without fixing the block
  layout; the codec below is written from the format's definition.

Nothing in this module is shared with the HIP library.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "f32_to_bf16_bits",
    "f64_to_bf16_bits",
    "bf16_round_f64",
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_e4m3_rows",
    "E2M1_MAX",
    "MX_BLOCK",
    "e2m1_decode",
    "e2m1_encode",
    "e8m0_decode",
    "quantize_mxfp4_rows",
    "mxfp4_decode_rows",
    "pack_e2m1",
    "unpack_e2m1",
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


# ---------------------------------------------------------------------------
# FP8 E4M3
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Decode FP8 E4M3 codes (uint8 array) to float64 exactly."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError(f"e4m3 codes must be uint8, got {c.dtype}")
    return _E4M3_TABLE[c]


# the non-negative finite codes in increasing order of value (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = _E4M3_TABLE[:0x7F]


def e4m3_encode(x) -> np.ndarray:
    """Round values to FP8 E4M3 codes: nearest representable magnitude, ties
    to the even code (the one whose lowest mantissa bit is 0), magnitudes
    above 448 saturated to 448, the sign kept (so -0.0 gives 0x80).  NaN is
    out of contract.  Works on the exact value of its float64 input."""
    v = np.asarray(x, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN is out of contract for the e4m3 encoder")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], code).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_e4m3_rows(x):
    """Per-row FP8 E4M3 quantisation of a [rows, d] array of float32 values.

    scale = max|row| / 448 (binary32 division; 1 for an all-zero row), then
    every element is divided by its row's scale in binary32 and encoded with
    :func:`e4m3_encode` (so the row's largest magnitude maps to 448 exactly).
    Returns (codes uint8 [rows, d], scales float32 [rows]); the decoded value
    of element j is ``e4m3_decode(codes[j]) * scales``.
    """
    f = np.asarray(x, dtype=np.float32)
    if f.ndim != 2:
        raise ValueError("rows x d expected")
    amax = np.abs(f).max(axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (f / scale[:, None]).astype(np.float32)
    return e4m3_encode(y.astype(np.float64)), scale


# ---------------------------------------------------------------------------
# FP4 E2M1 elements with E8M0 block scales
# ---------------------------------------------------------------------------

E2M1_MAX = 6.0
MX_BLOCK = 32  # elements sharing one E8M0 scale


def _e2m1_value(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m          # subnormal: m * 2^-1
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


_E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_POS_VALUES = _E2M1_TABLE[:8]           # 0, 0.5, 1, 1.5, 2, 3, 4, 6
_E2M1_POS_CODES = np.arange(8, dtype=np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    """Decode FP4 E2M1 codes (uint8 array, values 0..15) to float64 exactly."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError(f"e2m1 codes must be uint8, got {c.dtype}")
    if (c > 15).any():
        raise ValueError("e2m1 codes are 4 bits")
    return _E2M1_TABLE[c]


def e2m1_encode(x) -> np.ndarray:
    """Round values to FP4 E2M1 codes: nearest representable magnitude, ties
    to the even code (lowest bit 0), magnitudes above 6 saturated to 6, the
    sign bit set for negative values whose magnitude does not round to zero
    (a zero result is always code 0).  NaN is out of contract."""
    v = np.asarray(x, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN is out of contract for the e2m1 encoder")
    a = np.minimum(np.abs(v), E2M1_MAX)
    hi = np.clip(np.searchsorted(_E2M1_POS_VALUES, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_hi = _E2M1_POS_VALUES[hi] - a
    d_lo = a - _E2M1_POS_VALUES[lo]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_E2M1_POS_CODES[hi] & 1) == 0))
    code = np.where(take_hi, _E2M1_POS_CODES[hi], _E2M1_POS_CODES[lo]).astype(np.uint8)
    code = np.where(a == _E2M1_POS_VALUES[hi], _E2M1_POS_CODES[hi], code).astype(np.uint8)
    neg = (v < 0) & (code != 0)
    return np.where(neg, code | np.uint8(0x8), code).astype(np.uint8)


def e8m0_decode(s) -> np.ndarray:
    """Decode E8M0 scale codes (uint8, 0..254) to float64: 2^(s - 127)."""
    c = np.asarray(s)
    if c.dtype != np.uint8:
        raise TypeError(f"e8m0 codes must be uint8, got {c.dtype}")
    if (c == 255).any():
        raise ValueError("e8m0 code 255 is NaN, out of contract")
    return np.ldexp(1.0, c.astype(np.int64) - 127)


def quantize_mxfp4_rows(x):
    """FP4 E2M1 quantisation of a [rows, d] array of float32 values (d a
    multiple of 32), one E8M0 scale per block of 32 consecutive elements
    (reading R30).

    A block's scale is 2^X with X the smallest integer such that the block's
    largest magnitude is at most 6 * 2^X (so no element saturates), clamped
    to [-127, 127]; an all-zero block gets X = 0.  Each element is divided by
    2^X (exact) and encoded with :func:`e2m1_encode`.  Returns (codes uint8
    [rows, d], one code per element; scales uint8 [rows, d / 32], E8M0 codes
    X + 127); the decoded value of element j is ``e2m1_decode(codes[j]) *
    e8m0_decode(scales[j // 32])``.
    """
    f = np.asarray(x, dtype=np.float32)
    if f.ndim != 2 or f.shape[1] % MX_BLOCK != 0:
        raise ValueError("rows x d (a multiple of 32) expected")
    rows, d = f.shape
    blocks = f.astype(np.float64).reshape(rows, d // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    X = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    X[nz] = np.ceil(np.log2(amax[nz] / E2M1_MAX)).astype(np.int64)
    # settle the boundary exactly (6 * 2^X is exact in float64)
    for _ in range(2):
        up = nz & (amax > E2M1_MAX * np.ldexp(1.0, X))
        X[up] += 1
        down = nz & (amax <= E2M1_MAX * np.ldexp(1.0, X - 1))
        X[down] -= 1
    X = np.clip(X, -127, 127)
    y = blocks / np.ldexp(1.0, X)[:, :, None]
    codes = e2m1_encode(y).reshape(rows, d)
    return codes, (X + 127).astype(np.uint8)


def mxfp4_decode_rows(codes, scales) -> np.ndarray:
    """The float64 values of :func:`quantize_mxfp4_rows` output."""
    c = e2m1_decode(np.asarray(codes, dtype=np.uint8))
    s = e8m0_decode(np.asarray(scales, dtype=np.uint8))
    return c * np.repeat(s, MX_BLOCK, axis=-1)


def pack_e2m1(codes) -> np.ndarray:
    """Two E2M1 codes per byte along the last axis: element 2j in the low
    nibble, element 2j + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed) -> np.ndarray:
    """The codes of :func:`pack_e2m1`, one per element."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out

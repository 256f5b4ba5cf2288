"""Oracle: MXFP8 codec and block quantizer. TEST INFRASTRUCTURE ONLY.

[R] "Mixture-of-Kittens: a deterministic MoE megakernel for NVL72 racks",
§"Tuning the five hyperparameters before production": in MXFP8 mode the
activations enter in BF16 and the weights are quantized beforehand through a
separate quantize call. The pages name the format only ("MXFP8"); the element
and scale formats taken here are the OCP Microscaling (MX) v1.0 ones:

  * element: FP8 E4M3 ("FN" variant): 1 sign bit, 4 exponent bits with bias
    7, 3 mantissa bits; exponent field 0 is subnormal (value m/8 * 2^-6);
    codes 0x7F / 0xFF are NaN; there is no infinity; the largest finite
    magnitude is 448 (0x7E).
  * scale: E8M0, one unsigned byte per block of 32 consecutive elements along
    the contraction dimension, value 2^(byte - 127).
  * conversion of a block v[0..31]: X = floor(log2(max |v_i|)) - 8 (8 is the
    exponent of E4M3's largest normal, 448 = 1.75 * 2^8), clamped to
    [-127, 127]; a block of zeros gets X = -127. Each element is v_i / 2^X
    rounded to the nearest E4M3 value, ties to the even code, magnitudes above
    448 saturating to 448; the sign is kept (so -0 and negative values that
    round to zero give 0x80). Scale byte = X + 127.

Readings taken where the pages leave a step open: the OCP floor rule for X rather than a
round-up rule; saturation rather than NaN on overflow; sign-preserving zero.
Non-finite inputs are outside the contract (asserted finite here).
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "block_exponent",
           "quantize", "dequantize", "qdq"]

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte, from the bit fields (closed form).

    Pin: all 256 codes are compared against torch's float8_e4m3fn -> float
    conversion (a library routine) in tests/test_oracle_mxfp8.py.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * np.ldexp(1.0 + man / 8.0, (ex - 7).astype(np.int64))
    sub = sign * np.ldexp(man / 8.0, -6)
    val = np.where(ex == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# The non-negative finite grid, ascending with the code (0x00 .. 0x7E).
_GRID = e4m3_decode(np.arange(0x7F))
assert np.all(np.diff(_GRID) > 0)


def e4m3_encode(v) -> np.ndarray:
    """Round real values (already divided by the block scale) to E4M3 codes:
    nearest grid value, ties to the even code, |v| > 448 saturating to 448,
    sign kept.

    Pin: equals torch's float -> float8_e4m3fn cast (round to nearest even)
    on values clamped to +-448, over every bf16 bit pattern and over random
    float64 values, in tests/test_oracle_mxfp8.py.
    """
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite input is outside the contract"
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_GRID, a, side="left")          # first grid value >= a
    hi = np.minimum(hi, _GRID.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _GRID[hi], hi, code)              # exact hits
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Shared exponent X of a block from its largest magnitude:
    floor(log2(amax)) - 8, clamped to [-127, 127]; -127 when amax == 0.
    floor(log2) is read exactly from frexp (amax = f * 2^e, f in [0.5, 1))."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    x = (e.astype(np.int64) - 1) - 8
    x = np.where(amax == 0, -127, x)
    return np.clip(x, -127, 127)


def quantize(v, axis: int = -1):
    """MXFP8-quantize ``v`` in blocks of 32 consecutive elements along
    ``axis`` (the contraction dimension). Returns (codes uint8 with v's shape,
    scales uint8 with v's shape except that ``axis`` is divided by 32).

    Pins (tests/test_oracle_mxfp8.py): exact round trip of blocks built from
    E4M3 grid values times 2^X; hand-worked blocks in
    tests/golden/mxfp8_blocks.txt; saturation and zero-block special cases;
    exhaustive sweep of bf16 bit patterns against the library cast.
    """
    v = np.asarray(v, dtype=np.float64)
    axis = axis % v.ndim
    n = v.shape[axis]
    assert n % BLOCK == 0, "the blocked dimension must be a multiple of 32"
    vm = np.moveaxis(v, axis, -1)
    blocks = vm.reshape(vm.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    X = block_exponent(amax)
    scaled = np.ldexp(blocks, -X[..., None])             # exact: power-of-two scaling
    codes = e4m3_encode(scaled).reshape(vm.shape)
    return np.ascontiguousarray(np.moveaxis(codes, -1, axis)), \
        np.ascontiguousarray(np.moveaxis((X + 127).astype(np.uint8), -1, axis))


def dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    """value(code) * 2^(scale - 127), exact, in float64."""
    codes = np.asarray(codes)
    axis = axis % codes.ndim
    vals = e4m3_decode(codes)
    X = np.asarray(scales, dtype=np.int64) - 127
    Xe = np.repeat(X, BLOCK, axis=axis)
    return np.ldexp(vals, Xe)


def qdq(v, axis: int = -1) -> np.ndarray:
    """dequantize(quantize(v)): the value the MXFP8 path computes with."""
    c, s = quantize(v, axis)
    return dequantize(c, s, axis)

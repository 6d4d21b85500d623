"""The FP4 KV-store codec: e2m1 elements, one e8m0 scale per 16 elements along head_dim.

[DIST] "NVFP4 量化与 KV Cache 压缩的工程实现" and [PIPE] 三、NVFP4 量化 say only that the KV cache
can be stored in FP4 with a fused dequant kernel. The element and scale encodings follow
[OCP] (FP4 E2M1: values 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit; E8M0: 2^(byte-127)).

Steps for one block of 16 bf16 values x_0..x_15 (the readings taken where the pages are silent:
the OCP MX shared-exponent rule, ties to the even code, the sign copied, saturation at 6):
  1. a = max |x_i|; b = the biased exponent field of a (0 for zero and subnormals)
  2. scale byte sb = max(b - 2, 0), i.e. floor(log2 a) - 2 (2 = emax of e2m1) clamped to
     the e8m0 range; E = sb - 127. 0xFF is never produced.
  3. y_i = |x_i| * 2^-E (exact in float64)
  4. magnitude code = nearest grid point, ties to the even code, y > 6 saturates to 6
  5. sign bit (bit 3) copied from x_i (so -0 and tiny negatives encode as 0x8)
  6. bytes: element 2j in the low nibble, 2j+1 in the high nibble
Dequant: (-1)^s * grid[code & 7] * 2^E.
"""
from __future__ import annotations

import numpy as np

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 16


def _bf16_fields(bits: np.ndarray):
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = bits >> 15
    expo = (bits >> 7) & 0xFF
    mant = bits & 0x7F
    return sign, expo, mant


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (finite patterns only)."""
    sign, expo, mant = _bf16_fields(bits)
    if np.any(expo == 0xFF):
        raise ValueError("NaN/Inf inputs are not supported by the codec")
    normal = expo > 0
    mag = np.where(normal, (128 + mant) * np.exp2(expo.astype(np.float64) - 134.0),
                   mant * np.exp2(-133.0))
    return np.where(sign == 1, -mag, mag)


def scale_bytes(bits: np.ndarray) -> np.ndarray:
    """Steps 1-2 for blocks along the last axis. bits [..., L] -> [..., L/16] uint8."""
    bits = np.asarray(bits, dtype=np.uint16)
    L = bits.shape[-1]
    if L % BLOCK:
        raise ValueError("row length must be a multiple of 16")
    blk = bits.reshape(bits.shape[:-1] + (L // BLOCK, BLOCK))
    a = np.max(np.abs(bf16_value(blk)), axis=-1)
    # biased exponent field of a = floor(log2 a) + 127 for normal a, 0 below 2^-126;
    # frexp gives a = m * 2^e with m in [0.5, 1) exactly, so floor(log2 a) = e - 1
    _, e = np.frexp(a)
    b = np.where(a >= np.exp2(-126.0), e.astype(np.int64) - 1 + 127, 0)
    return np.maximum(b - 2, 0).astype(np.uint8)


def encode_magnitude(y: np.ndarray) -> np.ndarray:
    """Step 4: nearest point of GRID, ties to the even code, saturating above 6."""
    y = np.asarray(y, dtype=np.float64)
    code = np.zeros(y.shape, dtype=np.int64)
    # walk the 7 midpoints between neighbouring grid points; at a midpoint the even code
    # of the pair wins
    for c in range(7):
        mid = 0.5 * (GRID[c] + GRID[c + 1])
        upper_is_even = (c + 1) % 2 == 0
        above = (y >= mid) if upper_is_even else (y > mid)
        code = np.where(above, c + 1, code)
    return code


def quantize(bits: np.ndarray):
    """bf16 bit patterns [rows, L] -> (packed [rows, L/2] uint8, scales [rows, L/16] uint8)."""
    bits = np.asarray(bits, dtype=np.uint16)
    rows, L = bits.shape
    sb = scale_bytes(bits).astype(np.int64)                 # [rows, L/16]
    E = sb - 127
    x = bf16_value(bits)                                      # [rows, L]
    y = np.abs(x) * np.exp2(-np.repeat(E, BLOCK, axis=1).astype(np.float64))
    mag = encode_magnitude(y)
    sign = (bits.astype(np.int64) >> 15) & 1
    code = (sign << 3) | mag
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb.astype(np.uint8)


def dequantize(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(packed [rows, L/2], scales [rows, L/16]) -> float64 values [rows, L]."""
    packed = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    rows, half = packed.shape
    code = np.empty((rows, 2 * half), dtype=np.int64)
    code[:, 0::2] = packed & 0xF
    code[:, 1::2] = packed >> 4
    E = np.asarray(scales, dtype=np.int64) - 127
    mag = GRID[code & 7] * np.exp2(np.repeat(E, BLOCK, axis=1).astype(np.float64))
    return np.where(code & 8, -mag, mag)


def roundtrip(bits: np.ndarray) -> np.ndarray:
    """dequant(quant(x)) for bf16 bit patterns [..., L] (any leading shape)."""
    bits = np.asarray(bits, dtype=np.uint16)
    flat = bits.reshape(-1, bits.shape[-1])
    p, s = quantize(flat)
    return dequantize(p, s).reshape(bits.shape)

"""Decoders for the cache's storage formats, written from the format
definitions (test infrastructure; see the package docstring).

[Audit] B1: the latent's "nope" dims are stored as FP8_E4M3 and its 64 rope
dims as BF16.  [Roadmap] E1: the FP8 entries are stored with a scale kept
alongside; the reading taken here is a per-tensor multiply-to-dequantise
factor.

E4M3 is the OCP 8-bit format "E4M3FN": 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, NaN only at S.1111.111, largest finite 448.
  exponent field e > 0 : (-1)^s * 2^(e-7) * (1 + m/8)
  exponent field e = 0 : (-1)^s * 2^(-6) * (m/8)            (subnormal)
BF16 is the upper half of an IEEE-754 binary32: its value is that of the
float32 whose high 16 bits are the stored bits and low 16 bits are zero.

MXFP4 (the FP4 indexer variant, [Audit] B2 / [Roadmap] E7) is the OCP
Microscaling format with E2M1 elements and an E8M0 scale per block of 32:
  E2M1 nibble: 1 sign bit (bit 3), 2 exponent bits (bits 2-1) with bias 1,
  1 mantissa bit (bit 0); e > 0: (-1)^s * 2^(e-1) * (1 + m/2),
  e = 0: (-1)^s * m/2 (subnormal); no infinities or NaN.
  E8M0 byte x: 2^(x - 127); x = 255 is NaN.
Element 2j of a packed row sits in the low nibble of byte j, element 2j + 1
in the high nibble.
"""
import numpy as np


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN byte codes -> float64 values (NaN for the two NaN codes)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    out = np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, out)
    return out


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def e2m1_decode(nibbles: np.ndarray) -> np.ndarray:
    """E2M1 4-bit codes (0..15) -> float64 values."""
    c = np.asarray(nibbles, dtype=np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64))
    return sign * np.where(e == 0, m / 2.0, normal)


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64 powers of two (NaN for 255)."""
    x = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(x == 255, np.nan, np.ldexp(1.0, x - 127))


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed MXFP4 rows [..., D/2] bytes with E8M0 scales [..., D/32] ->
    float64 [..., D]."""
    b = np.asarray(packed, dtype=np.uint8)
    vals = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.float64)
    vals[..., 0::2] = e2m1_decode(b & 0xF)
    vals[..., 1::2] = e2m1_decode(b >> 4)
    sc = e8m0_decode(scales)
    return vals * np.repeat(sc, 32, axis=-1)

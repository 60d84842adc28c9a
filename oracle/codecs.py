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

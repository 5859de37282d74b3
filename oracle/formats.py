"""Storage-format decoders used by the oracle (test infrastructure; see ``oracle/__init__``).

The pages name an fp8 attention cache and an fp4 indexer cache (vLLM day-0 DeepSeek-V4 post,
paragraph after the "four moves" list) without fixing the encodings. Readings taken here:

* fp8 = OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7),
  3 mantissa bits, no infinities, NaN = S.1111.111, largest finite 448.
* fp4 = OCP Microscaling E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
  Values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.
* the per-32-element fp4 scale = OCP E8M0: value 2**(code - 127), code 255 = NaN.
* bf16 = the upper 16 bits of an IEEE-754 binary32.

Each decoder is written from the bit-field definition (not a table) so that the exhaustive
pins in ``tests/test_oracle_formats.py`` compare two independent descriptions.
"""

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16/int16) -> float64. Exact."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns: first to the nearest float32, then round-to-nearest-even
    on the upper 16 bits (how a bf16 cache stores a value computed in wider precision)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float64))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), r)


def e4m3fn_to_f64(code) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64. Exact."""
    c = np.asarray(code).astype(np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * np.exp2(1.0 - 7.0)
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e2m1_to_f64(code) -> np.ndarray:
    """OCP MX FP4 E2M1 codes (low 4 bits of each value) -> float64. Exact."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    subnormal = (m / 2.0) * np.exp2(1.0 - 1.0)
    return sign * np.where(e == 0, subnormal, normal)


def e8m0_to_f64(code) -> np.ndarray:
    """OCP E8M0 scale codes (uint8) -> float64: 2**(code-127); 255 is NaN."""
    c = np.asarray(code).astype(np.int64)
    val = np.exp2(c.astype(np.float64) - 127.0)
    return np.where(c == 255, np.nan, val)


def unpack_fp4_row(packed_row: np.ndarray, scales_row: np.ndarray, dim: int) -> np.ndarray:
    """One fp4 entry -> float64[dim].

    Packing reading: element 2j sits in the low nibble of byte j, element 2j+1 in the high
    nibble; element d is multiplied by the E8M0 scale of its 32-element group d // 32.
    """
    p = np.asarray(packed_row).astype(np.uint8)
    codes = np.empty(dim, dtype=np.int64)
    codes[0::2] = p & 0xF
    codes[1::2] = p >> 4
    vals = e2m1_to_f64(codes)
    sc = e8m0_to_f64(np.asarray(scales_row))
    return vals * np.repeat(sc, 32)[:dim]

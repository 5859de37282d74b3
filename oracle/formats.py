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

import math

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


# --------------------------------------------------------------------------------------------
# Encoders (quantise-on-insert and the fp8 attention output). The pages name the fp8 / fp4
# caches but not how values are quantised; readings taken here:
#   * fp8 row (one attention-cache entry, or one head's output row): scale = amax / 448 in
#     float32 (1 when the row is all zero), code = E4M3 nearest to x / scale (float32 quotient),
#     ties to the even code, magnitudes beyond 448 saturating to 448.
#   * fp4 block of 32 (indexer keys, OCP MX rule): shared exponent e = floor(log2 amax) - 2,
#     clamped to [-100, 60] (an all-zero block takes -100), stored as the E8M0 byte e + 127;
#     code = E2M1 nearest to x / 2**e, ties to the even code, saturating at 6.
# The encoders search the decoders' code tables for the nearest value (independent of how a
# kernel rounds). Float32 steps are taken as float64 operations rounded once to float32, which
# equals the float32 operation for a quotient of float32 operands (53 >= 2 * 24 + 2).
# --------------------------------------------------------------------------------------------
_E4M3_POS = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))      # codes 0..126: 0 .. 448
_E2M1_POS = e2m1_to_f64(np.arange(8))                             # codes 0..7: 0 .. 6


def _nearest_even_code(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to each magnitude; equal distances go to the even index
    (the code whose mantissa LSB is 0). Magnitudes beyond the last value take the last index."""
    mag = np.asarray(mag, dtype=np.float64)
    d = np.abs(mag[..., None] - table)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    idx = np.arange(table.size)
    even = cand & (idx % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return np.where(mag >= table[-1], table.size - 1, pick)


def f32_quotient(x, s) -> np.ndarray:
    """float32(x / s) for float32 x and s (the float32 division, correctly rounded)."""
    return (np.asarray(x, np.float32).astype(np.float64) /
            np.asarray(s, np.float32).astype(np.float64)).astype(np.float32)


def encode_e4m3fn(v) -> np.ndarray:
    """float values -> E4M3 codes (uint8): nearest, ties to even, saturating at +-448.
    Negative values (and -0) keep the sign bit."""
    v = np.asarray(v, dtype=np.float64)
    code = _nearest_even_code(np.abs(v), _E4M3_POS).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def encode_e2m1(v) -> np.ndarray:
    """float values -> E2M1 codes (low 4 bits): nearest, ties to even, saturating at +-6."""
    v = np.asarray(v, dtype=np.float64)
    code = _nearest_even_code(np.abs(v), _E2M1_POS).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x8), code).astype(np.uint8)


def quantize_fp8_row(x):
    """One row (float32 values) -> (E4M3 codes uint8[D], float32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = np.float32(np.float64(amax) / 448.0) if amax > 0 else np.float32(1.0)
    return encode_e4m3fn(f32_quotient(x, scale)), scale


def mx_exponent(amax: float) -> int:
    """Shared exponent of one fp4 block: floor(log2 amax) - 2 clamped to [-100, 60]."""
    if not amax > 0:
        return -100
    m, e = math.frexp(amax)          # amax = m * 2**e, 0.5 <= m < 1: floor(log2 amax) = e - 1
    return int(min(60, max(-100, (e - 1) - 2)))


def quantize_fp4_row(x):
    """One row (float32 values, D % 32 == 0) -> (packed uint8[D/2], E8M0 uint8[D/32]).
    Element 2j in the low nibble of byte j."""
    x = np.asarray(x, dtype=np.float32)
    d = x.size
    codes = np.empty(d, dtype=np.uint8)
    sc = np.empty(d // 32, dtype=np.uint8)
    for blk in range(d // 32):
        xb = x[32 * blk:32 * blk + 32].astype(np.float64)
        e = mx_exponent(float(np.abs(xb).max()))
        sc[blk] = e + 127
        codes[32 * blk:32 * blk + 32] = encode_e2m1(xb / 2.0 ** e)   # exact: power-of-two scale
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, sc

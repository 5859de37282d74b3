"""Pins for the oracle's storage-format decoders (CPU only).

Each decoder is checked exhaustively against an independent description: torch's own bfloat16
and float8_e4m3fn conversions (library routines) and hand values from the OCP FP8 / MX
definitions.
"""

import math

import numpy as np
import pytest
import torch

from oracle.formats import (bf16_bits_to_f64, e2m1_to_f64, e4m3fn_to_f64, e8m0_to_f64,
                            unpack_fp4_row)


def test_bf16_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_hand_values():
    assert bf16_bits_to_f64(0x3F80) == 1.0
    assert bf16_bits_to_f64(0xC000) == -2.0
    assert bf16_bits_to_f64(0x0001) == 2.0 ** -133
    assert math.isinf(bf16_bits_to_f64(0x7F80))


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x07, 7 * 2.0 ** -9), (0x3C, 1.5), (0x00, 0.0), (0x40, 2.0),
])
def test_e4m3fn_hand_values(code, value):
    assert e4m3fn_to_f64(code) == value


def test_e4m3fn_nan_codes():
    nan = np.isnan(e4m3fn_to_f64(np.arange(256)))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]


def test_e2m1_table():
    # OCP MX v1.0, FP4 E2M1: exponent bias 1, one mantissa bit, no inf or NaN.
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = e2m1_to_f64(np.arange(16))
    assert got[:8].tolist() == expect
    assert got[8:].tolist() == [-v for v in expect]
    assert np.signbit(got[8])  # code 0b1000 is -0


def test_e8m0():
    assert e8m0_to_f64(127) == 1.0
    assert e8m0_to_f64(0) == 2.0 ** -127
    assert e8m0_to_f64(254) == 2.0 ** 127
    assert e8m0_to_f64(130) == 8.0
    assert np.isnan(e8m0_to_f64(255))


def test_fp4_packing_low_nibble_first():
    dim = 64
    packed = np.zeros(dim // 2, np.uint8)
    packed[0] = 0x21           # element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    packed[16] = 0xF7          # element 32 = code 7 (6.0), element 33 = code 15 (-6.0)
    scales = np.array([127, 129], np.uint8)  # 1.0 for dims 0..31, 4.0 for dims 32..63
    row = unpack_fp4_row(packed, scales, dim)
    assert row[0] == 0.5 and row[1] == 1.0
    assert row[32] == 24.0 and row[33] == -24.0
    assert np.count_nonzero(row) == 4


def test_quantisers_decode_close():
    """The input generator's quantisers, read back by the oracle, stay within the format's
    rounding bound (this pins the generator's encoders, not the method)."""
    from sparse_attention_hyb_amd.workloads import quantize_fp4_rows, quantize_fp8_rows
    g = torch.Generator().manual_seed(7)
    x = torch.randn(40, 64, generator=g)
    codes, scale = quantize_fp8_rows(x)
    dec = e4m3fn_to_f64(codes.numpy()) * scale.numpy()[:, None].astype(np.float64)
    # e4m3 has 3 mantissa bits: relative rounding error <= 2**-4 for normal values,
    # absolute error <= half the smallest subnormal step times the scale
    err = np.abs(dec - x.numpy())
    bound = np.maximum(np.abs(x.numpy()) * 2.0 ** -4, scale.numpy()[:, None] * 2.0 ** -10)
    assert (err <= bound + 1e-12).all()
    assert (np.abs(dec).max(axis=1) <= scale.numpy() * 448 * (1 + 1e-7)).all()

    packed, sc = quantize_fp4_rows(x)
    dec4 = np.stack([unpack_fp4_row(packed[i].numpy(), sc[i].numpy(), 64) for i in range(40)])
    blk_scale = np.repeat(e8m0_to_f64(sc.numpy()), 32, axis=1)
    # grid step at the top of the E2M1 range is 2 (x scale); saturation at 6 x scale is
    # within one step of amax because amax / 2**e < 8
    err4 = np.abs(dec4 - x.numpy())
    assert (err4 <= blk_scale * 2.0 + 1e-12).all()
    # exact grid points survive unchanged
    v = torch.tensor([[0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -6.0, 0.0] * 4], dtype=torch.float32)
    p, s = quantize_fp4_rows(v)
    back = unpack_fp4_row(p[0].numpy(), s[0].numpy(), 32)
    assert np.array_equal(back, v[0].numpy().astype(np.float64))


def test_fp4_ties_round_to_even():
    from sparse_attention_hyb_amd.workloads import quantize_fp4_rows
    # amax 6 -> e = floor(log2 6) - 2 = 0: values are coded directly
    v = torch.tensor([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4], dtype=torch.float32)
    p, s = quantize_fp4_rows(v)
    back = unpack_fp4_row(p[0].numpy(), s[0].numpy(), 32)[:8]
    assert back.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]


def test_round_to_bf16_matches_torch_on_float32_values():
    from oracle.formats import round_to_bf16_bits
    g = torch.Generator().manual_seed(3)
    x = torch.cat([torch.randn(100000, generator=g) * 10,
                   torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0, 3e38, 1e-40])])
    ours = round_to_bf16_bits(x.numpy().astype(np.float64))
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ encoders (quantise-on-insert)
from oracle.formats import (encode_e2m1, encode_e4m3fn, mx_exponent, quantize_fp4_row,  # noqa: E402
                            quantize_fp8_row)


def _e4m3_test_values():
    pos = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))            # every finite magnitude
    mids = (pos[:-1] + pos[1:]) / 2                                   # every tie
    rng = np.random.default_rng(5)
    rand = np.exp2(rng.uniform(-12, np.log2(448.0), 20000)) * rng.choice([-1, 1], 20000)
    near = np.concatenate([np.nextafter(mids, 0), np.nextafter(mids, 1)])
    v = np.concatenate([pos, -pos, mids, -mids, near, rand]).astype(np.float32)
    return v[np.abs(v) <= 448.0]


def test_e4m3_encoder_matches_torch_cast():
    """Round to nearest even inside the finite range: torch's float32 -> float8_e4m3fn cast is an
    independent implementation of the same rounding."""
    v = _e4m3_test_values()
    ours = encode_e4m3fn(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_e4m3_encoder_saturates_and_keeps_sign():
    assert list(encode_e4m3fn([448.0, 449.0, 1e9, -500.0])) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert encode_e4m3fn([-0.0])[0] == 0x80 and encode_e4m3fn([0.0])[0] == 0
    # the smallest subnormal is 2^-9; half of it is a tie that goes to zero, just above goes up
    assert list(encode_e4m3fn([2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -9])) == [0, 1, 1]


def test_e2m1_encoder_hand_values():
    """OCP MX E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7): each tie goes to the code
    with mantissa bit 0, values above 6 saturate."""
    v = [0.0, 0.25, 0.26, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 5.01, 6.0, 100.0]
    want = [0, 0, 1, 1, 2, 2, 2, 3, 4, 4, 4, 5, 6, 6, 6, 7, 7, 7]
    assert list(encode_e2m1(v)) == want
    assert list(encode_e2m1([-0.75, -6.5])) == [0x8 | 2, 0x8 | 7]


def test_encoders_round_trip_every_code():
    c8 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert (encode_e4m3fn(e4m3fn_to_f64(c8)) == c8).all()
    c4 = np.arange(16, dtype=np.uint8)
    assert (encode_e2m1(e2m1_to_f64(c4)) == c4).all()


def test_mx_exponent_hand_values():
    assert mx_exponent(6.0) == 0 and mx_exponent(4.0) == 0 and mx_exponent(7.99) == 0
    assert mx_exponent(8.0) == 1 and mx_exponent(1.0) == -2 and mx_exponent(0.75) == -3
    assert mx_exponent(0.0) == -100 and mx_exponent(2.0 ** -300) == -100
    assert mx_exponent(2.0 ** 100) == 60


def test_quantize_fp8_row_error_bound_and_exact_rows():
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = (rng.standard_normal(512) * np.exp2(rng.uniform(-20, 20))).astype(np.float32)
        codes, s = quantize_fp8_row(x)
        assert s == np.float32(np.float64(np.abs(x).max()) / 448.0)
        y = e4m3fn_to_f64(codes) * np.float64(s)
        v = x.astype(np.float64) / np.float64(s)
        # half an E4M3 step at v's binade (subnormal step 2^-9), plus the float32 quotient's rounding
        step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))), -6) - 3)
        assert (np.abs(y - x) <= (0.5 * step + 2.0 ** -23 * np.abs(v)) * np.float64(s)).all()
    # a row whose maximum is 448 has scale 1 and is its own code image
    x = e4m3fn_to_f64(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float32)
    codes, s = quantize_fp8_row(x)
    assert s == 1.0 and (codes == np.arange(0, 0x7F)).all()
    codes, s = quantize_fp8_row(np.zeros(64, np.float32))
    assert s == 1.0 and (codes == 0).all()


def test_quantize_fp4_row_layout_and_error_bound():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(128) * np.repeat(np.exp2(rng.uniform(-8, 8, 4)), 32)).astype(np.float32)
    packed, sc = quantize_fp4_row(x)
    assert packed.shape == (64,) and sc.shape == (4,)
    y = unpack_fp4_row(packed, sc, 128)
    for blk in range(4):
        xb = x[32 * blk:32 * blk + 32].astype(np.float64)
        e = mx_exponent(np.abs(xb).max())
        assert sc[blk] == e + 127
        v = np.abs(xb) / 2.0 ** e
        # grid steps: 0.5 below 2, 1 in [2, 4), 2 from 4; saturation at 6 beyond
        step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
        err = np.abs(y[32 * blk:32 * blk + 32] - xb) / 2.0 ** e
        assert (err <= np.maximum(0.5 * step, v - 6.0) + 1e-12).all()
    # element 2j in the low nibble of byte j
    x = np.zeros(32, np.float32)
    x[0], x[1], x[31] = 4.0, -1.0, 0.5
    packed, sc = quantize_fp4_row(x)
    assert sc[0] == 127 and packed[0] == (0x6 | (0xA << 4)) and packed[15] == (0x1 << 4)

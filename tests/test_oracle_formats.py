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

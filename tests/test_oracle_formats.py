"""Pins of the oracle's number-format decoders (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import decode_bf16, decode_e4m3, E4M3_MAX


# Values fixed by the OCP FP8 E4M3 format definition (bias 7, 3 mantissa bits,
# subnormals m*2^-9, no infinities, S.1111.111 = NaN).
@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0x77, 240.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_e4m3_hand_values(code, value):
    assert decode_e4m3(np.uint8(code)) == value


def test_e4m3_nan_and_signed_zero():
    assert np.isnan(decode_e4m3(np.uint8(0x7F)))
    assert np.isnan(decode_e4m3(np.uint8(0xFF)))
    z = decode_e4m3(np.uint8(0x80))
    assert z == 0.0 and np.signbit(z)
    assert E4M3_MAX == 448.0
    finite = decode_e4m3(np.arange(256, dtype=np.uint8))
    assert np.nanmax(np.abs(finite)) == E4M3_MAX


def test_e4m3_matches_library_cast():
    # torch's float8_e4m3fn is the OCP E4M3 format: an independent library decoder.
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = decode_e4m3(codes)
    both_nan = np.isnan(lib) & np.isnan(ours)
    assert np.all(both_nan | (lib == ours))
    assert np.array_equal(np.signbit(lib[~both_nan]), np.signbit(ours[~both_nan]))


def test_e4m3_monotone_positive_codes():
    vals = decode_e4m3(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0)


def test_bf16_hand_values_and_library():
    assert decode_bf16(np.uint16(0x3F80)) == 1.0
    assert decode_bf16(np.uint16(0xC000)) == -2.0
    assert decode_bf16(np.uint16(0x4049)) == 3.140625
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite patterns only
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(lib, decode_bf16(bits))

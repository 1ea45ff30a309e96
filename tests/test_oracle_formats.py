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


# ---------------------------------------------------------------------------
# encoder pins
# ---------------------------------------------------------------------------

def test_e4m3_encode_matches_library_cast():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even: an independent encoder
    from oracle import encode_e4m3
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.uniform(-448, 448, 200000), rng.uniform(-0.02, 0.02, 100000),
                        rng.normal(0, 3, 100000)]).astype(np.float32)
    y = np.clip(y, -448, 448)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3(y), lib)


def test_e4m3_encode_ties_and_round_trip():
    from oracle import encode_e4m3
    # every representable value encodes to its own code
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)
    # midpoints go to the even code: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39)
    assert encode_e4m3(np.float64(1.0625)) == 0x38
    assert encode_e4m3(np.float64(1.1875)) == 0x3A          # between 1.125 (0x39) and 1.25 (0x3A)
    assert encode_e4m3(np.float64(2.0 ** -10)) == 0x00      # half the smallest subnormal: to 0
    assert encode_e4m3(np.float64(3 * 2.0 ** -10)) == 0x02  # 1.5 steps: to 2 (even)
    assert encode_e4m3(np.float64(-0.0)) == 0x80
    with pytest.raises(ValueError):
        encode_e4m3(np.float64(449.0))


def test_per_token_quantization_definition():
    from oracle import quantize_e4m3_per_token
    rng = np.random.default_rng(6)
    x = rng.normal(0, 1, (6, 3, 16)).astype(np.float32)
    x[2] = 0.0                                               # an all-zero token
    x[4] *= 2.0 ** 40                                        # scaling by 2^j is exact
    codes, scale = quantize_e4m3_per_token(x)
    assert scale[2] == 1.0 and np.all(codes[2] == 0)
    for t in (0, 1, 3, 4, 5):
        amax = np.abs(x[t]).max()
        assert scale[t] == np.float32(amax) / np.float32(448.0)
        # the largest element maps to +-448 exactly
        i = np.unravel_index(np.abs(x[t]).argmax(), x[t].shape)
        assert abs(decode_e4m3(codes[t][i])) == 448.0
    c4, s4 = quantize_e4m3_per_token(x[4:5] / np.float32(2.0 ** 40))
    assert np.array_equal(c4[0], codes[4]) and s4[0] * np.float32(2.0 ** 40) == scale[4]
    # dequantized values are within half an E4M3 step of x
    deq = decode_e4m3(codes) * scale[:, None, None]
    step = np.maximum(np.abs(deq), 2.0 ** -6 * scale[:, None, None]) * 2.0 ** -3
    assert np.all(np.abs(deq - x) <= 0.5 * step * (1 + 1e-6))

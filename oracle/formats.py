"""Exact decoders for the stored number formats (test infrastructure only).

The pages say only that the indexer is FP8-friendly (GLM-5.2 技术报告速览, section
"IndexShare": ReLU is used instead of softmax for speed and FP8-friendliness) and that
the model ships BF16 and FP8 weights (GLM 5.2: Built for Long Horizon Tasks, section 5.1
release-surface table).  They fix neither the FP8 flavour nor the scaling granularity;
the reading used here is OCP FP8 E4M3 ("e4m3fn") with one fp32 scale per token.

Both decoders are written from the bit-level format definitions, so that the oracle
sees exactly the values the stored bytes represent:

* bfloat16: the upper 16 bits of an IEEE-754 binary32 word.
* OCP E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
  encodes subnormals m * 2^-9; there are no infinities; S.1111.111 is NaN; the
  largest finite magnitude is 1.75 * 2^8 = 448.
"""

import numpy as np

E4M3_MAX = 448.0


def decode_bf16(bits):
    """uint16 bit patterns (any shape) -> float64 values, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3_table():
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = np.nan
        elif exp_field == 0:
            table[code] = sign * mant * 2.0 ** -9
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


_E4M3 = _e4m3_table()


def decode_e4m3(codes):
    """uint8 OCP E4M3 codes (any shape) -> float64 values, exactly (NaN for 0x7F/0xFF)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# Encoder (the step before the path: per-token quantization of the indexer's q^I and
# k^I).  The reading is the one the pages leave open, as above: one fp32 scale per token,
# scale = amax / 448 (1 for an all-zero token), codes = round-to-nearest-even of
# x / scale in E4M3.  Both divisions are single-precision (IEEE round to nearest), so a
# device encoder can match the codes bit for bit.
# ---------------------------------------------------------------------------

_POS_CODES = np.arange(0x7F, dtype=np.uint8)           # 0x00 .. 0x7E: the non-negative finite values
_POS_VALUES = _E4M3[_POS_CODES]                         # increasing


def encode_e4m3(y):
    """float values with |y| <= 448 (any shape) -> nearest E4M3 codes, ties to the even
    code (mantissa bit 0 clear), sign kept (including -0)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("values must be finite with |y| <= 448")
    hi = np.searchsorted(_POS_VALUES, a, side="left")   # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0)).astype(np.uint8)


def quantize_e4m3_per_token(x):
    """x: [T, ...] float32 -> (codes uint8 [T, ...], scale float32 [T])."""
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[0]
    amax = np.abs(x.reshape(T, -1)).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = x / scale.reshape((T,) + (1,) * (x.ndim - 1))            # float32 division
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return encode_e4m3(y), scale

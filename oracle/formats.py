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

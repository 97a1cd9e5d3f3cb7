"""Decoding of OCP FP8 E4M3 (the "e4m3fn" variant) to float64, from the format's
definition.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The library never
calls it and shares no code with it.

Used for a K/V cache stored in FP8 with bf16 queries and outputs (the pages name
an FP8 KV cache among the serving integrations).  The oracle attends over the
exact values the codes stand for, so the attention definition itself is
unchanged: decode the pools, then call bsr_attention.

Format (OCP 8-bit floating point specification, E4M3): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits.  Exponent 0 encodes subnormals m * 2^-9;
exponent field 15 with mantissa 7 encodes NaN (there is no infinity); every other
code is (1 + m / 8) * 2^(e - 7), so the largest finite magnitude is 448.
"""

from __future__ import annotations

import numpy as np

__all__ = ["decode_e4m3"]


def decode_e4m3(codes):
    """float64 array of the values of uint8 E4M3 codes (same shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    value = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    value = sign * value
    return np.where((e == 15) & (m == 7), np.nan, value)

"""Pins of the E4M3 decoder: values fixed by the format's definition, and the
whole code table against torch's float8_e4m3fn conversion (a library routine)."""

import numpy as np
import torch


def pin_e4m3_closed_forms(F):
    cases = {
        0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x3C: 1.5,
        0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x01: 2.0 ** -9,
    }
    got = F.decode_e4m3(np.array(list(cases), dtype=np.uint8))
    assert np.array_equal(got, np.array(list(cases.values()))), got
    assert np.signbit(F.decode_e4m3(np.array([0x80], dtype=np.uint8)))[0]
    assert np.all(np.isnan(F.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))))


def pin_e4m3_table_vs_library(F):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = F.decode_e4m3(codes.numpy())
    assert np.array_equal(got, ref, equal_nan=True)


def pin_e4m3_monotone(F):
    # positive codes 0x00..0x7E increase strictly: the exponent / mantissa split is right
    v = F.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


ALL_FP8_PINS = [pin_e4m3_closed_forms, pin_e4m3_table_vs_library, pin_e4m3_monotone]

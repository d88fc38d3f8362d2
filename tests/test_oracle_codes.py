"""Pins of the oracle's bf16 / e4m3 decoders: exhaustive tables and the OCP spec."""
import json
import math
import os

import numpy as np
import torch

from oracle import decode_bf16, decode_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


def test_bf16_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(decode_bf16(codes), ref)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(decode_e4m3(codes), ref)


def test_e4m3_spec_table():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_codes.json")))
    for code, val in g["codes"].items():
        got = float(decode_e4m3(np.array([int(code, 16)], dtype=np.uint8))[0])
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def test_e4m3_has_no_infinity_and_max_448():
    v = decode_e4m3(np.arange(256, dtype=np.uint8))
    assert not np.isinf(v).any()
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert np.isnan(v).sum() == 2


def test_every_e4m3_value_is_a_bf16_value():
    # the FP8 path widens e4m3 to bf16 before the MFMA; this is exact because
    # every finite e4m3 value has a bf16 code
    v = decode_e4m3(np.arange(256, dtype=np.uint8))
    v = v[np.isfinite(v)]
    bf = decode_bf16(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    assert np.isin(v, bf[np.isfinite(bf)]).all()

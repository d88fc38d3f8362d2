"""Exact decoders from storage codes to fp64 -- oracle (test infrastructure only).

The KV cache reaches the kernel either as bfloat16 or as FP8 codes read with
bf16 queries ("Xqa decode kernels", section "Purpose": the Hopper decode path
takes BF16/FP16 queries over an FP8 KV cache; "Test Plan" runs it with
``--kv-cache-dtype fp8``).  The pages do not name the FP8 encoding; the plain
reading, consistent with the +-448 clamp of the FP8 workload, is OCP e4m3fn.

Both decoders are written from the bit-level definitions of the formats, not
from any library conversion, and are pinned exhaustively against torch's
conversions in ``tests/test_oracle_codes.py``.
"""
import numpy as np


def decode_bf16(codes) -> np.ndarray:
    """bfloat16 code -> fp64.

    A bf16 value is the upper 16 bits of an IEEE binary32 value: sign (1),
    exponent (8, bias 127), mantissa (7).  The decode is exact.
    """
    c = np.asarray(codes).astype(np.uint32)
    sign = np.where((c >> 15) & 1, -1.0, 1.0)
    e = ((c >> 7) & 0xFF).astype(np.int64)
    m = (c & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 128.0, e - 127)
    sub = sign * np.ldexp(m / 128.0, -126)
    out = np.where(e == 0, sub, normal)
    out = np.where((e == 255) & (m == 0), sign * np.inf, out)
    out = np.where((e == 255) & (m != 0), np.nan, out)
    return out


def decode_e4m3(codes) -> np.ndarray:
    """OCP e4m3fn code -> fp64.

    Sign (1), exponent (4, bias 7), mantissa (3).  e >= 1: s * 2^(e-7) * (1 + m/8);
    e == 0: subnormal s * 2^-6 * (m/8).  Codes 0x7F and 0xFF (all exponent and
    mantissa bits set) are NaN; there are no infinities, so the largest finite
    magnitude is 2^8 * 1.75 = 448.
    """
    c = np.asarray(codes).astype(np.uint32)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = ((c >> 3) & 0xF).astype(np.int64)
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out

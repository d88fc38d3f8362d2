"""KV append: the new tokens' key/value rows written into their cache pages.

Oracle -- TEST INFRASTRUCTURE ONLY (tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may use it; the product path never does).

The decode step reads a paged cache in which logical token j of sequence b
sits in page block_table[b][j // P], slot j % P; the step before decode
writes each new token there.  An FP8 cache is read as code x scale with one
fp32 scale per tensor ("Xqa decode kernels", section "Purpose": bf16 queries
over an FP8 KV cache; "Test Plan": the cache dtype fp8 with its dequant
test).  The pages do not spell out the write side; the plainest reading,
the inverse of that read, is taken here:

    code = nearest e4m3 value of clamp(x / scale, -448, 448)   (fp32 division)

with ties going to the code whose mantissa is even and the sign kept (a
negative value that rounds to zero gives -0).  NaN gives a NaN code (this
oracle keeps the sign; the format's two NaN codes are equivalent, and parity
checks accept either).  A bf16 cache stores the bf16 codes unchanged.
"""
import numpy as np

from .codes import decode_bf16, decode_e4m3

E4M3_MAX = 448.0

# the 127 non-negative finite e4m3 values, in code order (0x00 .. 0x7E),
# which is also increasing value order
_POS_VALUES = decode_e4m3(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """float values -> OCP e4m3fn codes: saturate to +-448, nearest value, ties to even.

    Written as a search over the table of representable values: for each |x|
    take the two table entries around it and keep the nearer one (the one
    with the even code on a tie).  Inputs are compared exactly in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    nan = np.isnan(x)
    ax = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, ax, side="left")          # first value >= |x|
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = ax - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def quantise_bf16(codes, scale: float) -> np.ndarray:
    """bf16 codes -> e4m3 codes of value / scale (the division in fp32)."""
    x = decode_bf16(codes).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = x / np.float32(scale)
    return e4m3_encode(y)


def append_kv(k_cache, v_cache, k_new, v_new, block_table, positions, page_size: int,
              kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """Return copies of the caches with the new rows written.

    k_cache / v_cache: [num_pages][Hkv][P][d] codes (uint16 bf16 or uint8
    e4m3); v_cache may be None (a latent cache whose values are the first
    columns of its keys).  k_new / v_new: bf16 codes [B][T][Hkv][d].
    positions[b]: logical position of sequence b's first new token; token t
    goes to position positions[b] + t.  A token whose position is negative,
    past the block table's row, or whose page lies outside the cache is not
    written.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = None if v_cache is None else np.array(v_cache, copy=True)
    B, T, Hkv, _ = k_new.shape
    num_pages = k_cache.shape[0]
    for b in range(B):
        for t in range(T):
            pos = int(positions[b]) + t
            if pos < 0 or pos // page_size >= block_table.shape[1]:
                continue
            page = int(block_table[b, pos // page_size])
            if page < 0 or page >= num_pages:
                continue
            slot = pos % page_size
            for hk in range(Hkv):
                if kv_dtype == "bf16":
                    k_out[page, hk, slot, :] = k_new[b, t, hk, :]
                    if v_out is not None:
                        v_out[page, hk, slot, :] = v_new[b, t, hk, :]
                else:
                    k_out[page, hk, slot, :] = quantise_bf16(k_new[b, t, hk, :], k_scale)
                    if v_out is not None:
                        v_out[page, hk, slot, :] = quantise_bf16(v_new[b, t, hk, :], v_scale)
    return k_out, v_out

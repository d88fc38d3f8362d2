"""Pins of the append oracle (e4m3 quantiser and page placement), CPU only.

The quantiser is checked against what the OCP e4m3fn format fixes: every
finite code is a fixed point, the midpoint between neighbouring codes goes
to the even one and anything off the midpoint to the nearer one, magnitudes
past 448 saturate, NaN keeps its NaN code; and, as a library special case,
against torch's float8_e4m3fn conversion on every bf16 value (clamped first:
that conversion does not saturate).  The placement is checked by brute force
on small caches: exactly the target rows change.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.append import append_kv, e4m3_encode, quantise_bf16


def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.decode_e4m3(c)
    keep = ~np.isnan(v)
    return c[keep], v[keep]


def test_every_finite_code_is_a_fixed_point():
    c, v = _finite_codes()
    assert np.array_equal(e4m3_encode(v), c)
    assert e4m3_encode(np.array([-0.0]))[0] == 0x80


def test_midpoints_go_to_the_even_code_and_off_midpoints_to_the_nearer():
    for sign in (0x00, 0x80):
        lo = np.arange(0x00, 0x7E)                 # neighbours lo, lo + 1 (same sign)
        a = oracle.decode_e4m3((lo | sign).astype(np.uint8))
        b = oracle.decode_e4m3(((lo + 1) | sign).astype(np.uint8))
        mid = (a + b) / 2                          # exact: one more bit than e4m3 has
        even = np.where(lo % 2 == 0, lo, lo + 1) | sign
        assert np.array_equal(e4m3_encode(mid), even.astype(np.uint8))
        toward_a = mid + (a - b) / 64              # a little nearer a, then nearer b
        toward_b = mid + (b - a) / 64
        assert np.array_equal(e4m3_encode(toward_a), (lo | sign).astype(np.uint8))
        assert np.array_equal(e4m3_encode(toward_b), ((lo + 1) | sign).astype(np.uint8))


def test_subnormals_and_zero():
    # 2^-9 is the smallest subnormal; half of it ties between 0 and 0x01 -> 0
    assert e4m3_encode(np.array([2.0**-9]))[0] == 0x01
    assert e4m3_encode(np.array([2.0**-10]))[0] == 0x00
    assert e4m3_encode(np.array([3 * 2.0**-10]))[0] == 0x02
    assert e4m3_encode(np.array([-2.0**-11]))[0] == 0x80
    assert e4m3_encode(np.array([0.0]))[0] == 0x00


def test_saturation_and_nan():
    big = np.array([448.0, 464.0, 480.0, 1e6, np.inf, -448.0, -1e30, -np.inf])
    assert list(e4m3_encode(big)) == [0x7E] * 5 + [0xFE] * 3
    nan = np.array([np.nan, -np.nan])
    got = e4m3_encode(nan)
    assert (got & 0x7F == 0x7F).all()


def test_matches_torch_conversion_on_every_bf16_value():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.decode_bf16(codes)
    keep = ~np.isnan(x)
    xs = np.clip(x[keep], -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(xs), ref)


# 7 and 14: for 60 bf16 values each, x / scale and x * (1/scale) round to
# different codes, so these scales tell the division from a reciprocal
@pytest.mark.parametrize("scale", [1.0, 0.0625, 3.0, 7.0, 14.0, 1 / 300, 200.0])
def test_quantise_divides_in_fp32(scale):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.decode_bf16(codes).astype(np.float32)
    keep = ~np.isnan(x)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        y = x[keep] / np.float32(scale)
    ys = np.clip(y, -448.0, 448.0)
    ref = torch.from_numpy(ys.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quantise_bf16(codes[keep], scale), ref)


def _small(kv_dtype, mla=False, seed=5):
    rng = np.random.default_rng(seed)
    P, Hkv, D = 4, (1 if mla else 2), (12 if mla else 8)
    pages = 7
    dt = np.uint8 if kv_dtype == "e4m3" else np.uint16
    kc = rng.integers(0, 120, size=(pages, Hkv, P, D)).astype(dt)
    vc = None if mla else rng.integers(0, 120, size=(pages, Hkv, P, D)).astype(dt)
    B, T = 3, 2
    kn = synth.to_bf16_codes(rng.standard_normal((B, T, Hkv, D), dtype=np.float32))
    vn = None if mla else synth.to_bf16_codes(rng.standard_normal((B, T, Hkv, D), dtype=np.float32))
    bt = np.array([[3, 5, -1], [0, 6, 1], [2, 9, 4]], dtype=np.int32)   # -1 and 9: not pages
    pos = np.array([3, 6, 2], dtype=np.int32)
    return kc, vc, kn, vn, bt, pos, P


@pytest.mark.parametrize("kv_dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("mla", [False, True])
def test_append_writes_exactly_the_target_rows(kv_dtype, mla):
    kc, vc, kn, vn, bt, pos, P = _small(kv_dtype, mla)
    k2, v2 = append_kv(kc, vc, kn, vn, bt, pos, P, kv_dtype, k_scale=0.5, v_scale=2.0)
    written = set()
    for b in range(kn.shape[0]):
        for t in range(kn.shape[1]):
            j = int(pos[b]) + t
            page = int(bt[b, j // P])
            if 0 <= page < kc.shape[0]:
                written.add((page, j % P))
                for hk in range(kn.shape[2]):
                    want = kn[b, t, hk] if kv_dtype == "bf16" else quantise_bf16(kn[b, t, hk], 0.5)
                    assert np.array_equal(k2[page, hk, j % P], want)
                    if vc is not None:
                        want = vn[b, t, hk] if kv_dtype == "bf16" else quantise_bf16(vn[b, t, hk], 2.0)
                        assert np.array_equal(v2[page, hk, j % P], want)
    # sequence 0 writes positions 3 (page 3) and 4 (page 5); sequence 1
    # positions 6, 7 (page 6); sequence 2 positions 2, 3 (page 2)
    assert written == {(3, 3), (5, 0), (6, 2), (6, 3), (2, 2), (2, 3)}
    for page in range(kc.shape[0]):
        for slot in range(P):
            if (page, slot) not in written:
                assert np.array_equal(k2[page, :, slot], kc[page, :, slot])
                if vc is not None:
                    assert np.array_equal(v2[page, :, slot], vc[page, :, slot])


def test_append_skips_positions_outside_the_table_and_cache():
    kc, vc, kn, vn, bt, pos, P = _small("bf16")
    # sequence 0 at position 7: column 1 (page 5) then column 2 (-1, not a page);
    # sequence 2 at 4: column 1 holds 9, past the 7 pages; sequence 1 at -1
    # then 0: only position 0 is written
    k2, v2 = append_kv(kc, vc, kn, vn, bt, np.array([7, -1, 4], dtype=np.int32), P, "bf16")
    changed = {(p, s) for p in range(kc.shape[0]) for s in range(P)
               if not np.array_equal(k2[p, :, s], kc[p, :, s])}
    assert changed == {(5, 3), (0, 0)}

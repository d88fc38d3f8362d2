"""Pins of the oracle's e4m3-query reading (queries quantised like an FP8 cache), CPU only.

With e4m3 queries every query value is replaced by the e4m3 code of
q / q_scale (fp32 division, saturated to +-448, nearest value, ties to the
even code) read back times q_scale.  Checked here against a brute-force
search over all 256 codes, against queries that are already code x scale
(left unchanged, so attention equals the bf16-query oracle's), and at the
saturation bound.
"""
import dataclasses

import numpy as np

import oracle
import synth
from oracle.attention import dequant_q


def _case(q_scale, q_codes=None, seed=3):
    c = synth.make_case("q8", B=1, T=2, Hq=4, Hkv=2, d_qk=64, d_v=64, seq_lens=[40], page_size=16,
                        kv_dtype=synth.KV_E4M3, seed=seed)
    if q_codes is not None:
        c = dataclasses.replace(c, q=q_codes)
    return dataclasses.replace(c, q_scale=q_scale)


def _brute_nearest(x):
    """Nearest finite e4m3 value to each x (fp64 distances, ties to the even code)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.decode_e4m3(codes)
    out = np.empty_like(x, dtype=np.float64)
    for i, xv in enumerate(np.clip(x, -448.0, 448.0)):
        d = np.abs(vals - xv)
        best = np.flatnonzero(d == d.min())
        pick = [j for j in best if codes[j] % 2 == 0] or list(best)
        out[i] = vals[pick[0]] if vals[pick[0]] != 0 else 0.0
    return out


def test_queries_go_to_the_nearest_code():
    qs = float(np.float32(0.0137))
    case = _case(qs)
    for (t, h) in [(0, 0), (1, 3)]:
        x = oracle.decode_bf16(case.q[0, t, h]).astype(np.float32) / np.float32(qs)
        want = _brute_nearest(x.astype(np.float64)) * qs
        got = dequant_q(case, 0, t, h)
        assert np.array_equal(got, want), np.flatnonzero(got != want)[:5]


def test_representable_queries_are_unchanged_and_attention_matches():
    # q = (e4m3 value) x 2^-5: exact in bf16, so quantising gives back q itself
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 0x7F, size=(1, 2, 4, 64)).astype(np.uint8) | \
        (rng.integers(0, 2, size=(1, 2, 4, 64)).astype(np.uint8) << 7)
    vals = oracle.decode_e4m3(codes) * 2.0 ** -5
    q_codes = synth.to_bf16_codes(vals.astype(np.float32))
    assert np.array_equal(oracle.decode_bf16(q_codes), vals)
    case = _case(2.0 ** -5, q_codes)
    for (t, h) in [(0, 1), (1, 2)]:
        assert np.array_equal(dequant_q(case, 0, t, h), vals[0, t, h])
    O8, L8 = oracle.attend(case)
    O, L = oracle.attend(dataclasses.replace(case, q_scale=None))
    assert np.array_equal(O8, O) and np.array_equal(L8, L)


def test_queries_saturate_at_448_scales():
    qs = 2.0 ** -8
    q = synth.to_bf16_codes(np.array([[[[5.0, -5.0, 1.75, -1.0e3] * 16] * 4] * 2], dtype=np.float32))
    case = _case(qs, q)
    got = dequant_q(case, 0, 0, 0)[:4]
    assert list(got) == [448 * qs, -448 * qs, 448 * qs, -448 * qs]

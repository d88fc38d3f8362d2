"""Planted mistakes in the oracle must be caught by its pins.

Each test swaps one oracle function for a plausibly wrong variant (on the CPU,
in this process only) and checks that at least one pin then fails.
"""
import numpy as np
import pytest

import oracle.attention as A
import oracle.codes as C
import oracle.plan as P
import tests.test_oracle_attention as TA
import tests.test_oracle_codes as TC
import tests.test_oracle_plan as TP


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_wrong_e4m3_bias_is_caught(monkeypatch):
    def bad(codes):
        c = np.asarray(codes).astype(np.uint32)
        sign = np.where((c >> 7) & 1, -1.0, 1.0)
        e = ((c >> 3) & 0xF).astype(np.int64)
        m = (c & 0x7).astype(np.float64)
        out = np.where(e == 0, sign * np.ldexp(m / 8, -7), sign * np.ldexp(1 + m / 8, e - 8))
        return np.where((e == 15) & (m == 7), np.nan, out)
    monkeypatch.setattr(TC, "decode_e4m3", bad)
    _fails(TC.test_e4m3_all_codes_match_torch)
    _fails(TC.test_e4m3_spec_table)


def test_wrong_head_grouping_is_caught(monkeypatch):
    def bad_rows(case, hk):
        return [(t, h) for t in range(case.T) for h in range(case.Hq) if h % case.Hkv == hk]
    monkeypatch.setattr(A, "_rows_of_group", bad_rows)
    _fails(TA.test_attend_vs_torch_sdpa_fp64)


def test_dropped_scale_is_caught(monkeypatch):
    orig = A.attend_rows
    monkeypatch.setattr(A, "attend_rows", lambda q, K, V, sigma, lim: orig(q, K, V, 1.0, lim))
    _fails(TA.test_golden_two_key)


def test_off_by_one_causal_limit_is_caught(monkeypatch):
    orig = A.attend_rows
    monkeypatch.setattr(A, "attend_rows",
                        lambda q, K, V, s, lim: orig(q, K, V, s, [x + 1 for x in lim]))
    _fails(TA.test_attend_causal_vs_torch_sdpa_fp64)


def test_unweighted_combine_is_caught(monkeypatch):
    def bad(pm, pl, po, ns, off):
        O, L = np.zeros((len(ns),) + pm.shape[1:] + (po.shape[-1],)), np.zeros((len(ns),) + pm.shape[1:])
        for b in range(len(ns)):
            sl = slice(off[b], off[b] + ns[b])
            O[b] = po[sl].sum(0) / np.maximum(pl[sl].sum(0), 1e-300)[..., None]
            L[b] = np.log(np.maximum(pl[sl].sum(0), 1e-300)) + pm[sl].max(0)
        return O, L
    monkeypatch.setattr(A, "combine", bad)
    _fails(TA.test_split_emulation_equals_unsplit, 1, 3)


def test_split_range_off_by_one_is_caught(monkeypatch):
    def bad(L, n, i):
        nblk = -(-L // 16)
        return 16 * ((i * nblk) // n), min(L, 16 * (((i + 1) * nblk) // n) - 1)
    monkeypatch.setattr(P, "split_range", bad)
    _fails(TP.test_ranges_partition_and_are_nonempty)


def test_ignored_request_is_caught(monkeypatch):
    # the regression the pages describe: the stored default of one wins
    monkeypatch.setattr(P, "clamp_request", lambda L, n, mx: 1)
    _fails(TP.test_request_is_honoured_exactly)


# ---- the append oracle

import oracle.append as AP  # noqa: E402
import tests.test_oracle_append as TAP  # noqa: E402


def test_ties_away_from_zero_are_caught(monkeypatch):
    orig_vals = AP._POS_VALUES

    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        neg = np.signbit(x)
        ax = np.minimum(np.abs(np.nan_to_num(x)), AP.E4M3_MAX)
        hi = np.minimum(np.searchsorted(orig_vals, ax), len(orig_vals) - 1)
        lo = np.maximum(hi - 1, 0)
        pick_hi = (orig_vals[hi] - ax) <= (ax - orig_vals[lo])      # ties upward
        code = np.where(pick_hi, hi, lo).astype(np.uint8)
        code = np.where(np.isnan(x), np.uint8(0x7F), code)
        return (code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)
    monkeypatch.setattr(TAP, "e4m3_encode", bad)
    _fails(TAP.test_midpoints_go_to_the_even_code_and_off_midpoints_to_the_nearer)
    _fails(TAP.test_matches_torch_conversion_on_every_bf16_value)


def test_missing_saturation_is_caught(monkeypatch):
    orig = AP.e4m3_encode

    def bad(x):
        x = np.asarray(x, dtype=np.float64)
        out = orig(x)
        return np.where(np.abs(x) > AP.E4M3_MAX, np.uint8(0x7F) | (out & 0x80), out).astype(np.uint8)
    monkeypatch.setattr(TAP, "e4m3_encode", bad)
    _fails(TAP.test_saturation_and_nan)


def test_multiplying_by_a_rounded_reciprocal_is_caught(monkeypatch):
    def bad(codes, scale):
        x = C.decode_bf16(codes).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            y = x * (np.float32(1) / np.float32(scale))
        return AP.e4m3_encode(y)
    monkeypatch.setattr(TAP, "quantise_bf16", bad)
    _fails(TAP.test_quantise_divides_in_fp32, 7.0)


def test_wrong_slot_is_caught(monkeypatch):
    orig = AP.append_kv

    def bad(kc, vc, kn, vn, bt, pos, P, dt, k_scale=1.0, v_scale=1.0):
        return orig(kc, vc, kn, vn, bt, np.asarray(pos) + 1, P, dt, k_scale, v_scale)
    monkeypatch.setattr(TAP, "append_kv", bad)
    _fails(TAP.test_append_writes_exactly_the_target_rows, "bf16", False)


def test_query_scale_dropped_is_caught(monkeypatch):
    import tests.test_oracle_queries as TQ
    from oracle.append import quantise_bf16

    def bad(case, b, t, h):
        if case.q_scale is None:
            return C.decode_bf16(case.q[b, t, h])
        return C.decode_e4m3(quantise_bf16(case.q[b, t, h], case.q_scale))     # no x q_scale
    monkeypatch.setattr(A, "dequant_q", bad)
    monkeypatch.setattr(TQ, "dequant_q", bad)
    _fails(TQ.test_representable_queries_are_unchanged_and_attention_matches)
    _fails(TQ.test_queries_go_to_the_nearest_code)


def test_unquantised_queries_are_caught(monkeypatch):
    import tests.test_oracle_queries as TQ

    def bad(case, b, t, h):
        return C.decode_bf16(case.q[b, t, h])
    monkeypatch.setattr(A, "dequant_q", bad)
    monkeypatch.setattr(TQ, "dequant_q", bad)
    _fails(TQ.test_queries_go_to_the_nearest_code)
    _fails(TQ.test_queries_saturate_at_448_scales)


def test_dropped_merge_term_is_caught(monkeypatch):
    # the auto planner's estimate without the cost of the fp32 partials
    monkeypatch.setattr(P, "_merge_tokens", lambda ns, T, Hq, d_v, cus, tb, mla: 0)
    _fails(TP.test_auto_plan_worked_examples)


def test_fp32_row_bytes_for_mla_are_caught(monkeypatch):
    # the MLA merge priced at the grouped-query kernels' fp32 partial row
    orig = P._merge_tokens
    monkeypatch.setattr(P, "_merge_tokens",
                        lambda ns, T, Hq, d_v, cus, tb, mla: orig(ns, T, Hq, d_v, cus, tb, False))
    _fails(TP.test_auto_plan_worked_examples)

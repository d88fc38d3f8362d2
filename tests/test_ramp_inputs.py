"""The ramped-key inputs of the rescale parity tests really jump.

The partial kernels keep each row's O relative to a reference maximum and
rescale only when a tile's row maximum passes it by more than 8 in base 2
(a factor of 256).  These checks compute the base-2 scores of the ramped
inputs directly (q . k * scale * log2 e over the decoded codes) and confirm
that, inside the splits the GPU tests use, some row's later maximum exceeds
its maximum over the split's first 32 tokens by more than that margin.
"""
import math

import numpy as np

import oracle
from oracle import plan as oplan
from tests.test_gpu_parity import ramped_few_kv, ramped_mla, ramped_mla_e4m3


def _decode(codes):
    return (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _keys(case, hk):
    P = case.page_size
    L = int(case.seq_lens[0])
    pages = case.block_table[0, np.arange(L) // P]
    codes = case.k_cache[pages, hk, np.arange(L) % P, :]
    if case.kv_dtype == "e4m3":
        return oracle.decode_e4m3(codes) * case.k_scale                # [L, d_qk]
    return _decode(codes)


def _max_jump(case, split_ranges):
    """Largest (later max - max over the first 32 tokens) over rows and splits, base 2."""
    best = -math.inf
    for hk in range(case.Hkv):
        k = _keys(case, hk)
        heads = range(hk * case.g, (hk + 1) * case.g)
        q = _decode(case.q[0][:, list(heads), :]).reshape(-1, case.d_qk)   # [T*g, d]
        s = (q @ k.T) * case.scale / math.log(2)
        for (a, b) in split_ranges:
            if b - a <= 32:
                continue
            first = s[:, a:a + 32].max(axis=1)
            later = s[:, a + 32:b].max(axis=1)
            best = max(best, float((later - first).max()))
    return best


def _check(case):
    L = int(case.seq_lens[0])
    # one split, and the second and third of four (the splits holding the steps)
    assert _max_jump(case, [oplan.split_range(L, 1, 0)]) > 8
    assert _max_jump(case, [oplan.split_range(L, 4, 1)]) > 8
    assert _max_jump(case, [oplan.split_range(L, 4, 2)]) > 8


def test_mla_ramp_jumps_past_the_margin():
    _check(ramped_mla())


def test_few_kv_ramp_jumps_past_the_margin():
    _check(ramped_few_kv())


def test_mla_e4m3_ramp_jumps_past_the_margin():
    _check(ramped_mla_e4m3(False))

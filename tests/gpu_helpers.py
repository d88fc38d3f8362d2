"""Helpers of the GPU parity tests: run a synth case through the C ABI, compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import synth

# Tolerances (elementwise, |gpu - ref| <= ATOL + RTOL * |ref|): the bf16 /
# fp32-accumulate bound is max-abs 1e-2 and max-rel 2e-2; the FP8-KV bound is
# 3e-2 absolute against the oracle run on the same dequantised values.
ATOL_BF16, RTOL_BF16 = 1e-2, 2e-2
ATOL_FP8, RTOL_FP8 = 3e-2, 0.0


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def session_for(case, requested_splits=0, max_splits=64, layout="HND", q_pad_heads=0, debug=False,
                num_cus=0):
    import torch
    from split_kv_amd.session import DecodeSession
    t = synth.to_torch(case, "cuda", layout=layout, q_pad_heads=q_pad_heads)
    k = t["k_cache"]
    v = t["v_cache"]
    return DecodeSession(q=t["q"], k_cache=k, v_cache=v, block_table=t["block_table"],
                         seq_lens=case.seq_lens, scale=case.scale, k_scale=case.k_scale,
                         v_scale=case.v_scale, mla=case.mla, requested_splits=requested_splits,
                         max_splits=max_splits, out_fp32=case.out_fp32, debug=debug,
                         num_cus=num_cus, q_scale=case.q_scale), t


def to_np(x):
    import torch
    return x.detach().to(torch.float64).cpu().numpy()


def assert_close(got, ref, atol, rtol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    both_ninf = np.isneginf(got) & np.isneginf(ref)
    assert np.isfinite(got[~both_ninf]).all(), f"{what}: non-finite values in GPU output"
    g = np.where(both_ninf, 0.0, got)
    r = np.where(both_ninf, 0.0, ref)
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                             f"max abs err {err.max():.3e}; first bad {idx.tolist()} "
                             f"got {g[tuple(idx[0])]} ref {r[tuple(idx[0])]}")
    big = np.abs(r) > atol
    rel = float(np.max(err[big] / np.abs(r[big]))) if big.any() else 0.0
    return float(err.max()), rel


def tolerances(case):
    return (ATOL_FP8, RTOL_FP8) if case.kv_dtype == synth.KV_E4M3 else (ATOL_BF16, RTOL_BF16)

"""Helpers of the GPU parity tests: run a synth case through the C ABI, compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

import synth

# Tolerances: the bf16 / fp32-accumulate bound is max-abs 1e-2 and max-rel
# 2e-2; the FP8-KV bound is 3e-2 absolute against the oracle run on the same
# dequantised values.
ATOL_BF16, RTOL_BF16 = 1e-2, 2e-2
ATOL_FP8, RTOL_FP8 = 3e-2, 0.0
# The log-sum-exp is fp32 on both paths and never rounded to bf16: its own,
# much tighter absolute bound.
ATOL_LSE = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# Guard bands: every buffer the library writes (out, lse, workspace, tickets)
# sits inside a larger allocation whose GUARD bytes on either side hold a
# canary pattern; check_guards() asserts that no call wrote past its buffer
# (the failure behind the crash that "had been faking a split-KV problem":
# a read one slot past a small buffer).
GUARD = 4096
CANARY = 0x5A


def _guarded(torch, like):
    """A view shaped and typed like `like`, GUARD canary bytes on each side."""
    n = like.numel() * like.element_size()
    buf = torch.full((2 * GUARD + n,), CANARY, dtype=torch.uint8, device=like.device)
    view = buf[GUARD:GUARD + n].view(like.dtype).view(like.shape)
    view.copy_(like)
    return buf, n, view


def guard_buffers(sess):
    """Move the session's output-side buffers into guarded allocations."""
    import torch
    sess._guards = []
    for name in ("out", "lse", "workspace", "workspace_alt", "tickets", "debug"):
        t = getattr(sess, name, None)
        if t is None:
            continue
        buf, n, view = _guarded(torch, t)
        setattr(sess, name, view)
        sess._guards.append((name, buf, n))
    sess._build_args()


def check_guards(sess):
    import torch
    torch.cuda.synchronize()
    for name, buf, n in getattr(sess, "_guards", []):
        lo = buf[:GUARD].cpu().numpy()
        hi = buf[GUARD + n:].cpu().numpy()
        assert (lo == CANARY).all() and (hi == CANARY).all(), f"a kernel wrote outside `{name}`"


def session_for(case, requested_splits=0, max_splits=64, layout="HND", q_pad_heads=0, debug=False,
                num_cus=0, guard=True, q_pad_dim=0):
    import torch
    from split_kv_amd.session import DecodeSession
    t = synth.to_torch(case, "cuda", layout=layout, q_pad_heads=q_pad_heads, q_pad_dim=q_pad_dim)
    k = t["k_cache"]
    v = t["v_cache"]
    sess = DecodeSession(q=t["q"], k_cache=k, v_cache=v, block_table=t["block_table"],
                         seq_lens=case.seq_lens, scale=case.scale, k_scale=case.k_scale,
                         v_scale=case.v_scale, mla=case.mla, requested_splits=requested_splits,
                         max_splits=max_splits, out_fp32=case.out_fp32, debug=debug,
                         num_cus=num_cus, q_scale=case.q_scale)
    if guard:
        guard_buffers(sess)
    return sess, t


def to_np(x):
    import torch
    return x.detach().to(torch.float64).cpu().numpy()


def assert_close(got, ref, atol, rtol, what):
    """The parity bar, per element: |gpu - ref| <= max(atol, rtol * |ref|) --
    within max-abs atol, or, where rtol * |ref| exceeds it, within max-rel
    rtol.  Small outputs are judged absolutely: a relative figure there
    measures cancellation, not the kernel (the bf16 softmax weights of P V
    carry 2^-9 of sum |p v| / l each, so a ragged-batch output of 0.113 that
    is a small difference of large terms is off by 2.3% with 2.6e-3
    absolute).  Large outputs are judged relatively: bf16 itself spaces
    values 2^-6 apart in [2, 4).  Rows that see no key must be -inf on both
    sides.  Returns (max-abs, max-rel over |ref| > atol)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    both_ninf = np.isneginf(got) & np.isneginf(ref)
    assert np.isfinite(got[~both_ninf]).all(), f"{what}: non-finite values in GPU output"
    assert np.isfinite(ref[~both_ninf]).all(), f"{what}: the reference is -inf where the GPU output is finite"
    g = np.where(both_ninf, 0.0, got)
    r = np.where(both_ninf, 0.0, ref)
    err = np.abs(g - r)
    bad = err > np.maximum(atol, rtol * np.abs(r))
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


def pack_half_rows(o):
    """The MLA partial layout of o [..., 512]: a scale per 256-feature half
    (its largest |o| / 32767, fp32) and int16 codes, each the nearest integer
    to o / scale (0 where the half is all zero)."""
    h = o.reshape(o.shape[:-1] + (2, 256)).astype(np.float32)
    amax = np.abs(h).max(axis=-1)
    scales = (amax * np.float32(1.0 / 32767.0)).astype(np.float32)
    k = np.where(amax > 0, np.float32(32767.0) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    codes = np.clip(np.rint(h * k[..., None]), -32767, 32767).astype(np.int16)
    return scales, codes.reshape(o.shape)


def unpack_half_rows(scales, codes):
    """The values the MLA layout's codes stand for: code * scale of its half."""
    h = codes.reshape(codes.shape[:-1] + (2, 256)).astype(np.float64)
    return (h * scales[..., None].astype(np.float64)).reshape(codes.shape)

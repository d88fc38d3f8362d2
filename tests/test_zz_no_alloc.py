"""The allocation-free decode entry point (splitkv_decode_noalloc) through the C ABI.

It runs the same kernels as splitkv_decode with the partials in the library's
own device buffer, so its outputs must equal splitkv_decode's bit for bit, and
both must meet the oracle bound.  Two calls in a row, the second with a smaller
input, show that the shared buffer carries nothing from one call into the next.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_close, log, session_for, to_np, tolerances

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_both(case, n):
    import torch
    sess, _ = session_for(case, requested_splits=n)
    sess.decode()
    torch.cuda.synchronize()
    ref_out, ref_lse = sess.out.clone(), sess.lse.clone()
    sess.out.fill_(float("nan"))
    sess.lse.fill_(float("nan"))
    sess.workspace.fill_(float("nan"))          # the caller's workspace must not be read
    torch.cuda.synchronize()
    sess.decode_noalloc()
    torch.cuda.synchronize()
    assert torch.equal(sess.out, ref_out), "noalloc output differs from splitkv_decode"
    assert torch.equal(sess.lse, ref_lse), "noalloc lse differs from splitkv_decode"
    O, L = oracle.attend(case)
    atol, rtol = tolerances(case)
    e = assert_close(to_np(sess.out), O, atol, rtol, f"{case.name} noalloc out")
    assert_close(to_np(sess.lse), L, atol, rtol, f"{case.name} noalloc lse")
    return sess.total_slots, e


def test_noalloc_matches_decode_twice_second_smaller():
    _need_gpu()
    big = synth.fp8_batched(B=3, L=3001, seed=31)
    log("noalloc call 1: fp8 batched B=3 L=3001 n=8")
    s1, e1 = _run_both(big, 8)
    small = synth.few_kv_long(L=700, seed=5)
    log("noalloc call 2: few-kv L=700 n=4")
    s2, e2 = _run_both(small, 4)
    log(f"  slots {s1} then {s2}; max-abs {e1[0]:.2e}, {e2[0]:.2e}")


def test_noalloc_mla_then_smaller_gqa():
    _need_gpu()
    mla = synth.mla_decode(L=2048)
    log("noalloc call 1: mla L=2048 n=8")
    _run_both(mla, 8)
    small = synth.tiny_gqa()
    log("noalloc call 2: tiny gqa L=256 n=2")
    _run_both(small, 2)


def test_noalloc_refuses_plans_beyond_its_buffer():
    _need_gpu()
    import split_kv_amd as sk
    case = synth.mla_decode(L=65536)
    sess, _ = session_for(case, requested_splits=128, max_splits=256)
    need = sk.splitkv_workspace_bytes(sess.total_slots, case.T, case.Hq, case.d_v)
    assert need > sk.SPLITKV_NOALLOC_SCRATCH_BYTES
    with pytest.raises(sk.SplitKVError) as ei:
        sess.decode_noalloc()
    assert ei.value.status == sk.SPLITKV_ERR_WORKSPACE

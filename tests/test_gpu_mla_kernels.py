"""GPU parity of both MLA partial kernels on the same cases.

A step runs the 128-row kernel or, when every split range is short and the
64-row workgroups fit on the compute units at once, the short-range kernel
(the library decides from the plan's longest range).  Here each case runs
with each kernel forced (SPLITKV_MLA_KERNEL=short / long, read by the library
on every call) for the three cache/query kinds, against the oracle, with the
paged-addressing records bit-exact."""
import numpy as np
import pytest

import synth
from tests.gpu_helpers import log, session_for
from tests.test_gpu_parity import MLA_RPW, _check_debug, _check_full

pytestmark = pytest.mark.gpu

KINDS = {"bf16": dict(kv_dtype=synth.KV_BF16), "e4m3": dict(kv_dtype=synth.KV_E4M3),
         "e4m3-queries": dict(kv_dtype=synth.KV_E4M3, fp8_queries=True)}


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(params=["short", "long"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("SPLITKV_MLA_KERNEL", request.param)
    return request.param


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("L,n", [(2048, 16), (2048, 0), (2000, 3), (21, 2), (700, 0)])
def test_mla_kernels_agree_with_oracle(kernel, kind, L, n):
    _need_gpu()
    case = synth.mla_decode(L=L, seed=97 + L, **KINDS[kind])
    log(f"mla {kernel} kernel, {kind}, L={L} n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla {kernel} {kind} L={L} n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


@pytest.mark.parametrize("kind", list(KINDS))
def test_mla_kernels_short_sequences_and_partial_blocks(kernel, kind):
    # sequences shorter than the draft (rows with no visible key), and
    # T * Hq = 120 rows: the last 64- and 128-row blocks partly empty
    _need_gpu()
    extra = dict(KINDS[kind])
    fp8q = extra.pop("fp8_queries", False)
    case = synth.make_case("mla-kernels", B=3, T=3, Hq=40, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=[0, 2, 333], page_size=64, mla=True, std=0.5, seed=31,
                           fp8_queries=fp8q, **extra)
    log(f"mla {kernel} kernel, {kind}, seq_lens=[0,2,333] T=3 Hq=40")
    sess, _ = session_for(case, requested_splits=4, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla {kernel} {kind} short sequences")
    _check_debug(case, sess, 1, -(-120 // MLA_RPW))

"""The single-launch decode step and captured-graph steps, through the C ABI.

splitkv_decode_single_launch runs the grouped-query partial kernel with a
ticketed last-arriver merge instead of a second (combine) kernel.  Its output
must meet the oracle bound, agree with the two-kernel step, leave the ticket
counters at zero after every call, and write nothing outside its buffers.
It must do so on grids larger than one round of the GPU too (the ragged
batch's 1248 workgroups).  Decode steps captured in a HIP graph must give, on
every replay, the bits of the same step run eagerly.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (ATOL_LSE, assert_close, check_guards, log, session_for, to_np,
                               tolerances)

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = {
    "tiny-n2": (lambda: synth.tiny_gqa(), 2),
    "tiny-n4": (lambda: synth.tiny_gqa(), 4),
    "few-kv-L260-auto": (lambda: synth.few_kv_long(L=260), 0),
    "few-kv-L5900-n62": (lambda: synth.few_kv_long(L=5900), 62),
    "fp8-B3-n8": (lambda: synth.fp8_batched(B=3, L=3001, seed=31), 8),
    "ragged-auto": (lambda: synth.ragged(B=32, hi=4096), 0),
    "multitoken-T4-n3": (lambda: synth.make_case("gqa-multitoken", B=3, T=4, Hq=16, Hkv=2, d_qk=128,
                                                 d_v=128, seq_lens=[4, 37, 700], page_size=16,
                                                 seed=21), 3),
    "d64-e4m3-n5": (lambda: synth.make_case("d64", B=2, T=1, Hq=16, Hkv=4, d_qk=64, d_v=64,
                                            seq_lens=[999, 50], page_size=32, kv_dtype=synth.KV_E4M3,
                                            seed=64), 5),
    "zero-len-n4": (lambda: synth.make_case("zero-len", B=4, T=1, Hq=8, Hkv=2, d_qk=128, d_v=128,
                                            seq_lens=[0, 5, 300, 0], page_size=16, seed=3), 4),
}


@pytest.mark.parametrize("name", list(CASES))
def test_single_launch_matches_oracle_and_two_kernel_step(name):
    _need_gpu()
    import torch
    make, n = CASES[name]
    case = make()
    log(f"single launch {name}: n={n}")
    sess, _ = session_for(case, requested_splits=n)
    sess.decode()
    torch.cuda.synchronize()
    two_out, two_lse = sess.out.clone(), sess.lse.clone()
    O, L = oracle.attend(case)
    atol, rtol = tolerances(case)
    for call in range(2):                        # the tickets must be back at zero for the second
        sess.out.fill_(float("nan"))
        sess.lse.fill_(float("nan"))
        sess.decode_single_launch()
        torch.cuda.synchronize()
        e = assert_close(to_np(sess.out), O, atol, rtol, f"{name} call {call} out")
        assert_close(to_np(sess.lse), L, ATOL_LSE, 0.0, f"{name} call {call} lse")
        assert int(sess.tickets.abs().sum()) == 0, "tickets not left at zero"
        assert_close(to_np(sess.out), to_np(two_out), 2 * atol, 0.0, f"{name} vs two-kernel step")
        assert_close(to_np(sess.lse), to_np(two_lse), 2 * ATOL_LSE, 0.0, f"{name} lse vs two-kernel step")
        check_guards(sess)
        log(f"  call {call}: out max-abs {e[0]:.2e}; slots {sess.total_slots}")


@pytest.mark.parametrize("which", ["fp8-batched", "ragged-full"])
def test_single_launch_full_size_grids_match_two_kernel_step(which):
    # 256 workgroups (FP8 batch, one per CU) and 1248 (the ragged batch: more
    # than one round), at the auto plan: the single launch against the
    # two-kernel step, every row.
    _need_gpu()
    import torch
    case = synth.fp8_batched() if which == "fp8-batched" else synth.ragged()
    log(f"single launch vs two kernels, full size: {which}")
    sess, _ = session_for(case, requested_splits=0, max_splits=256)
    sess.decode()
    torch.cuda.synchronize()
    two_out, two_lse = sess.out.clone(), sess.lse.clone()
    atol, _ = tolerances(case)
    for call in range(2):
        sess.out.fill_(float("nan"))
        sess.lse.fill_(float("nan"))
        sess.decode_single_launch()
        torch.cuda.synchronize()
        assert_close(to_np(sess.out), to_np(two_out), 2 * atol, 0.0, f"{which} call {call} vs two-kernel")
        assert_close(to_np(sess.lse), to_np(two_lse), 2 * ATOL_LSE, 0.0, f"{which} call {call} lse")
        assert int(sess.tickets.abs().sum()) == 0, "counters not left at zero"
    check_guards(sess)


def test_single_launch_refuses_mla_and_missing_tickets():
    _need_gpu()
    import split_kv_amd as sk
    case = synth.mla_decode(L=300)
    sess, _ = session_for(case, requested_splits=2)
    with pytest.raises(sk.SplitKVError) as ei:
        sess.decode_single_launch()
    assert ei.value.status == sk.SPLITKV_ERR_UNSUPPORTED
    case = synth.few_kv_long(L=700, seed=5)
    sess, _ = session_for(case, requested_splits=4)
    sess.args.tickets = None
    with pytest.raises(sk.SplitKVError) as ei:
        sess.decode_single_launch()
    assert ei.value.status == sk.SPLITKV_ERR_INVALID_ARG


@pytest.mark.parametrize("mode", ["two-kernel", "single-launch", "mla"])
def test_captured_graph_steps_replay_bit_exact(mode):
    # Eight decode steps captured in one HIP graph (each on its own copy of
    # the page pool, as the bench runs them), replayed three times with eager
    # work and synchronisations in between: every replay must write the bits
    # of the eager step, which must meet the oracle bound.
    _need_gpu()
    import torch
    if mode == "mla":
        case = synth.mla_decode(L=2048)
    else:
        case = synth.few_kv_long(L=5900, seed=77)
    log(f"captured graph, {mode}")
    sess, t = session_for(case, requested_splits=0, max_splits=256)
    copies = []
    valid = case.block_table != synth.INT32_MAX
    for r in range(8):                           # the same pages, moved to other physical slots
        bt = case.block_table.copy()
        bt[valid] += r * case.num_pages
        copies.append(torch.from_numpy(bt).cuda())
    k = t["k_cache"].repeat(8, 1, 1, 1)
    v = t["v_cache"].repeat(8, 1, 1, 1) if t["v_cache"] is not None else None
    sess.k_cache, sess.v_cache = k, v
    sess.shape["num_pages"] = int(k.shape[0])
    sess._build_args()
    step = sess.decode_single_launch if mode == "single-launch" else sess.decode
    sess.set_block_table(copies[0])
    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = sess.out.clone(), sess.lse.clone()
    O, L = oracle.attend(case)
    atol, rtol = tolerances(case)
    assert_close(to_np(ref_out), O, atol, rtol, f"{mode} eager out")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for bt in copies:
            sess.set_block_table(bt)
            step()
    for rep in range(3):
        sess.out.fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sess.out, ref_out) and torch.equal(sess.lse, ref_lse), f"replay {rep} differs"
        if sess.tickets is not None:
            assert int(sess.tickets.abs().sum()) == 0
        sess.set_block_table(copies[rep % 8])      # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(sess.out, ref_out)
    check_guards(sess)
    del g

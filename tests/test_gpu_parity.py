"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every workload of the split-KV pages' hot path is covered: tiny GQA (fp32
out), few KV heads with long context swept over num_splits, batched GQA over
an e4m3 cache, MLA with six causal tokens, and a ragged batch planned
automatically.  Every size is compared element by element, the full sizes
(FP8 batch, MLA at L=65536 on the three paths, the ragged batch) over every
output row as well.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import plan as oplan
from tests.gpu_helpers import (ATOL_LSE, assert_close, check_guards, log, session_for, to_np,
                               tolerances, pack_half_rows, unpack_half_rows)

MLA_RPW = oplan.ROWS_PER_WG_MLA     # query rows of an MLA row block

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# The oracle's output for the full-size cases, computed once per case (the
# tests of one full-size case at several split counts share it; only those
# tests use the cache, and their cases are built unmodified from the
# generators).
_ORACLE = {}


def _oracle_attend(case, cache):
    if not cache:
        return oracle.attend(case)
    key = (case.name, case.seed, case.B, case.T, case.Hq, case.Hkv, case.d_qk, case.d_v, case.page_size,
           case.kv_dtype, case.q_scale, case.k_scale, case.v_scale, tuple(int(x) for x in case.seq_lens))
    if key not in _ORACLE:
        if len(_ORACLE) > 4:
            _ORACLE.clear()
        _ORACLE[key] = oracle.attend(case)
    return _ORACLE[key]


def _check_full(case, sess, tag, cache=False):
    import torch
    torch.cuda.synchronize()
    O, L = _oracle_attend(case, cache)
    atol, rtol = tolerances(case)
    e1 = assert_close(to_np(sess.out), O, atol, rtol, f"{tag} out")
    e2 = assert_close(to_np(sess.lse), L, ATOL_LSE, 0.0, f"{tag} lse")
    check_guards(sess)
    log(f"  {tag}: out max-abs {e1[0]:.2e} max-rel {e1[1]:.2e}; lse max-abs {e2[0]:.2e}")


def _check_debug(case, sess, Hkv, row_blocks):
    rec = sess.debug.cpu().numpy()
    ref = oplan.debug_records(case.seq_lens, case.block_table, case.page_size,
                              sess.num_splits_host, sess.slot_offset_host, Hkv, row_blocks)
    assert np.array_equal(rec, ref), "debug records differ from the oracle's integers"


# ---------------------------------------------------------------------------

def test_e4m3_widening_every_code_bit_exact():
    _need_gpu()
    import torch
    import split_kv_amd as sk
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(256, dtype=torch.int16, device="cuda")
    log("e4m3 -> bf16 all 256 codes")
    sk.splitkv_e4m3_to_bf16(codes.data_ptr(), out.data_ptr(), 256,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = oracle.decode_bf16(out.cpu().numpy().view(np.uint16))
    ref = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)


@pytest.mark.parametrize("n", [1, 2, 4])
@pytest.mark.parametrize("mode", ["decode", "partial+combine"])
def test_tiny_gqa_fp32_out(n, mode):
    _need_gpu()
    case = synth.tiny_gqa()
    log(f"tiny-gqa L=256 seed={case.seed} n={n} {mode}")
    sess, _ = session_for(case, requested_splits=n)
    assert sess.total_slots == n
    if mode == "decode":
        sess.decode()
    else:
        sess.partial()
        sess.combine()
    _check_full(case, sess, f"tiny n={n}")


@pytest.mark.parametrize("L", [260, 5900])
def test_few_kv_long_sweep(L):
    _need_gpu()
    import torch
    case = synth.few_kv_long(L=L)
    O, LSE = oracle.attend(case)
    outs = {}
    for n in [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 128, 256, 1000, 0]:
        # n = 0: the auto plan, the launch configuration bench.py times;
        # 256 is the largest split count, 1000 asks for more (clamped)
        log(f"few-kv-long L={L} seed={case.seed} n={n}")
        sess, _ = session_for(case, requested_splits=n, debug=True, max_splits=256)
        if n > 0:
            assert sess.total_slots == min(n, 256, -(-L // 16))
        sess.decode()
        torch.cuda.synchronize()
        e = assert_close(to_np(sess.out), O, 1e-2, 2e-2, f"L={L} n={n} out")
        assert_close(to_np(sess.lse), LSE, ATOL_LSE, 0.0, f"L={L} n={n} lse")
        check_guards(sess)
        _check_debug(case, sess, case.Hkv, 1)
        rec = sess.debug.cpu().numpy()
        assert (rec[..., 4] > rec[..., 3]).all(), "a requested split got an empty range"
        outs[n] = to_np(sess.out)
        log(f"  max-abs {e[0]:.2e}")
    # independent of the split count
    for n, o in outs.items():
        assert_close(o, outs[1], 2e-2, 4e-2, f"n={n} vs n=1")


def test_few_kv_partials_match_oracle_split_emulation():
    _need_gpu()
    import torch
    case = synth.few_kv_long(L=997, seed=77)
    sess, _ = session_for(case, requested_splits=7)
    log("few-kv partials L=997 n=7")
    sess.partial()
    torch.cuda.synchronize()
    pm, pl, po = oracle.split_partials(case, sess.num_splits_host, sess.slot_offset_host)
    gm, gl, go = (to_np(x) for x in sess.partials())
    assert_close(gm, pm, 1e-4, 1e-4, "part_m")
    assert_close(gl, pl, 1e-5 * max(1.0, float(np.abs(pl).max())), 1e-5, "part_l")
    check_guards(sess)
    # o carries the factor l (it is not normalised); the output bound applies
    # to each split's own softmax output o / l
    assert_close(go / gl[..., None], po / pl[..., None], 1e-2, 2e-2, "part_o / part_l")


@pytest.mark.parametrize("path", ["bf16", "e4m3", "e4m3-queries"])
def test_mla_partials_match_oracle_split_emulation(path):
    # The MLA kernels write o compactly (int16 codes, a scale per 256-feature
    # half); decoded, each split's own softmax output o / l must meet the
    # output bar against the oracle's fp64 split emulation, and m, l the
    # fp32-tight bounds.
    _need_gpu()
    import torch
    kv = synth.KV_BF16 if path == "bf16" else synth.KV_E4M3
    case = synth.mla_decode(L=1500, seed=91, kv_dtype=kv, fp8_queries=path == "e4m3-queries")
    sess, _ = session_for(case, requested_splits=5)
    log(f"mla partials {path} L=1500 n=5")
    sess.partial()
    torch.cuda.synchronize()
    pm, pl, po = oracle.split_partials(case, sess.num_splits_host, sess.slot_offset_host)
    gm, gl, go = (to_np(x) for x in sess.partials())
    # a score is an fp32 sum over 576 features (|s| up to ~20 here), so it is
    # off by up to ~1e-5 * |s|; m inherits that, and l = sum exp(s - m) the
    # same relative error, ~2e-4
    assert_close(gm, pm, 2e-4, 1e-5, "part_m")
    assert_close(gl, pl, 0.0, 2e-4, "part_l")
    check_guards(sess)
    atol, rtol = tolerances(case)
    assert_close(go / gl[..., None], po / pl[..., None], atol, rtol, "part_o / part_l")


def test_combine_alone_against_oracle_combine():
    _need_gpu()
    import torch
    import split_kv_amd as sk
    rng = np.random.default_rng(12)
    case = synth.few_kv_long(L=700, seed=5)
    sess, _ = session_for(case, requested_splits=9)
    sess.out_fp32 = True
    sess.out = torch.empty(sess.out.shape, dtype=torch.float32, device="cuda")
    sess._build_args()
    gm, gl, go = sess.partials()
    S, T, Hq, dv = go.shape
    m = rng.normal(0, 3, size=(S, T, Hq)).astype(np.float32)
    m[rng.random(m.shape) < 0.3] = -np.inf              # empty splits
    m[:, 0, 3] = -np.inf                                # a row that sees nothing
    l = np.where(np.isinf(m), 0, rng.uniform(0.5, 20, size=m.shape)).astype(np.float32)
    o = (rng.normal(size=(S, T, Hq, dv)) * l[..., None]).astype(np.float32)
    o[np.isinf(m)] = 0
    gm.copy_(torch.from_numpy(m))
    gl.copy_(torch.from_numpy(l))
    go.copy_(torch.from_numpy(o))
    o = o.astype(np.float64)
    log("combine alone, random partials with -inf rows")
    sess.combine()
    torch.cuda.synchronize()
    Oref, Lref = oracle.combine(m.astype(np.float64), l.astype(np.float64), o,
                                sess.num_splits_host, sess.slot_offset_host)
    assert_close(to_np(sess.out), Oref, 2e-5, 0.0, "combine out")
    assert_close(to_np(sess.lse), Lref, 2e-4, 0.0, "combine lse")
    check_guards(sess)
    assert (to_np(sess.out)[0, 0, 3] == 0).all() and np.isneginf(to_np(sess.lse)[0, 0, 3])


@pytest.mark.parametrize("hint", ["exact", "unknown", "low"])
@pytest.mark.parametrize("splits", [[1], [3], [9, 1, 21], [62], [130, 2]])
@pytest.mark.parametrize("d_v,T,Hq", [(64, 1, 8), (128, 1, 32), (256, 1, 16), (512, 6, 16)])
def test_combine_launch_shapes(d_v, T, Hq, splits, hint):
    # The merge sizes its launch (split groups per row, columns per
    # workgroup) from the plan's largest split count; a missing or too-small
    # hint must only cost time.  Random partials with empty splits, merged
    # through the C ABI, against the oracle's fp64 merge.
    _need_gpu()
    import torch
    import split_kv_amd as sk
    rng = np.random.default_rng(1000 + d_v + sum(splits))
    B, R = len(splits), T * Hq
    ns = np.array(splits, dtype=np.int32)
    off = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    S = int(off[-1])
    m = rng.normal(0, 3, size=(S, T, Hq)).astype(np.float32)
    m[rng.random(m.shape) < 0.25] = -np.inf
    l = np.where(np.isinf(m), 0, rng.uniform(0.5, 20, size=m.shape)).astype(np.float32)
    o = (rng.normal(size=(S, T, Hq, d_v)) * l[..., None]).astype(np.float32)
    o[np.isinf(m)] = 0
    nbytes = sk.splitkv_workspace_bytes(S, T, Hq, d_v)
    ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    ws[:S * R] = torch.from_numpy(m.reshape(-1)).cuda()
    ws[S * R:2 * S * R] = torch.from_numpy(l.reshape(-1)).cuda()
    if d_v == 512:
        # the MLA layout: int16 codes and a scale per 256-feature half; the
        # merge is checked on the values the codes stand for
        scales, codes = pack_half_rows(o)
        ws[2 * S * R:4 * S * R] = torch.from_numpy(scales.reshape(-1)).cuda()
        q0 = -(-(4 * S * R * 4) // 256) * 256 // 2
        ws.view(torch.int16)[q0:q0 + S * R * d_v] = torch.from_numpy(codes.reshape(-1)).cuda()
        o = unpack_half_rows(scales, codes)
    else:
        lo = -(-(2 * S * R * 4) // 256) * 256 // 4
        ws[lo:lo + S * R * d_v] = torch.from_numpy(o.reshape(-1)).cuda()
    o = o.astype(np.float64)
    out = torch.full((B, T, Hq, d_v), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    nsd, offd = torch.from_numpy(ns).cuda(), torch.from_numpy(off).cuda()
    lens = torch.full((B,), 16 * 256, dtype=torch.int32, device="cuda")     # not read by the merge
    a = sk.splitkv_args()
    a.num_splits, a.slot_offset, a.total_slots = nsd.data_ptr(), offd.data_ptr(), S
    a.seq_lens = lens.data_ptr()
    a.B, a.T, a.Hq, a.Hkv, a.d_qk, a.d_v = B, T, Hq, 1, d_v, d_v
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel() * 4
    a.out, a.out_dtype, a.lse = out.data_ptr(), sk.SPLITKV_OUT_F32, lse.data_ptr()
    a.max_seq_splits = {"exact": int(ns.max()), "unknown": 0, "low": 1}[hint]
    log(f"combine d_v={d_v} T={T} Hq={Hq} splits={splits} hint={hint}")
    sk.splitkv_combine(a, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    Oref, Lref = oracle.combine(m.astype(np.float64), l.astype(np.float64), o, ns, off)
    assert_close(to_np(out), Oref, 2e-5, 0.0, "combine out")
    assert_close(to_np(lse), Lref, 2e-4, 0.0, "combine lse")


def test_uniform_plan_promise_changes_nothing():
    # with every sequence split alike the merge takes its plan from
    # uniform_splits instead of reading it; both routes give the same bits
    _need_gpu()
    import torch
    case = synth.fp8_batched(B=3, L=997, seed=31)
    sess, _ = session_for(case, requested_splits=7)
    assert sess.args.uniform_splits == 7
    log("uniform plan: fp8 B=3 L=997 n=7")
    sess.decode()
    torch.cuda.synchronize()
    o1, l1 = sess.out.clone(), sess.lse.clone()
    sess.args.uniform_splits = 0
    sess.decode()
    torch.cuda.synchronize()
    assert torch.equal(o1, sess.out) and torch.equal(l1, sess.lse)
    _check_full(case, sess, "uniform plan")


def test_combine_of_one_split_is_identity():
    _need_gpu()
    import torch
    case = synth.few_kv_long(L=300, seed=8)
    sess, _ = session_for(case, requested_splits=1)
    sess.out_fp32 = True
    sess.out = torch.empty(sess.out.shape, dtype=torch.float32, device="cuda")
    sess._build_args()
    log("combine(n=1) identity")
    sess.partial()
    sess.combine()
    torch.cuda.synchronize()
    gm, gl, go = (to_np(x) for x in sess.partials())
    want = go[0] / gl[0][..., None]
    got = to_np(sess.out)[0]
    assert np.allclose(got, want, rtol=3e-7, atol=1e-30)
    assert np.allclose(to_np(sess.lse)[0], gm[0] + np.log(gl[0]), rtol=1e-6)


@pytest.mark.parametrize("n", [1, 2, 8, 0])
def test_fp8_small_full_compare(n):
    _need_gpu()
    case = synth.fp8_batched(B=3, L=3001, seed=31)
    log(f"fp8 B=3 L=3001 n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"fp8 small n={n}")
    _check_debug(case, sess, case.Hkv, 1)


def test_fp8_clamped_scale():
    _need_gpu()
    case = synth.fp8_batched(B=2, L=1500, seed=32, fp8_scale=1 / 128)
    log("fp8 clamp variant scale=1/128")
    sess, _ = session_for(case, requested_splits=4)
    sess.decode()
    _check_full(case, sess, "fp8 clamp")


@pytest.mark.parametrize("n", [1, 4, 8])
def test_mla_small_full_compare(n):
    _need_gpu()
    case = synth.mla_decode(L=2048)
    log(f"mla L=2048 n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


def test_mla_tiles_cut_by_ranges_and_pages():
    # L = 2000, n = 3: splits [0, 656), [656, 1328), [1328, 2000) end inside a
    # 32-token tile, and the third starts 48 tokens into a 64-token page, so
    # each of its tiles has its two halves in different pages
    _need_gpu()
    case = synth.mla_decode(L=2000, seed=13)
    log("mla L=2000 n=3 (partial tiles, tiles across pages)")
    sess, _ = session_for(case, requested_splits=3, debug=True)
    assert [tuple(r[2:]) for r in sess.slot_info_host] == [(0, 656), (656, 1328), (1328, 2000)]
    sess.decode()
    _check_full(case, sess, "mla L=2000 n=3")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


def test_mla_short_causal_edge():
    # L = 21: the last split holds keys only the later draft tokens see
    _need_gpu()
    case = synth.mla_decode(L=21, seed=9)
    log("mla L=21 n=2 (empty causal rows)")
    sess, _ = session_for(case, requested_splits=2)
    sess.decode()
    _check_full(case, sess, "mla L=21")


@pytest.mark.parametrize("n", [0, 1, 16])
def test_ragged_small_full_compare(n):
    _need_gpu()
    case = synth.ragged(B=32, hi=4096)
    log(f"ragged B=32 hi=4096 seed={case.seed} n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"ragged n={n}")
    _check_debug(case, sess, case.Hkv, 1)


@pytest.mark.parametrize("d,kv", [(128, synth.KV_BF16), (256, synth.KV_BF16), (128, synth.KV_E4M3)])
@pytest.mark.parametrize("n", [1, 3, 0])
def test_gqa_multi_token_causal(d, kv, n):
    # T = 4 query tokens per sequence (speculative decode on a grouped-query
    # cache): g*T = 32 rows, two row blocks; L = T leaves the first token a
    # single visible key
    _need_gpu()
    case = synth.make_case("gqa-multitoken", B=3, T=4, Hq=16, Hkv=2, d_qk=d, d_v=d,
                           seq_lens=[4, 37, 700], page_size=16, kv_dtype=kv, seed=21)
    log(f"gqa T=4 d={d} kv={kv} n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"gqa T=4 d={d} n={n}")
    _check_debug(case, sess, case.Hkv, 2)


def test_layouts_and_noncontiguous_query():
    _need_gpu()
    case = synth.ragged(B=8, hi=2000, seed=41)
    log("ragged NHD layout, padded q")
    sess, _ = session_for(case, requested_splits=3, layout="NHD", q_pad_heads=5)
    assert not sess.q.is_contiguous()
    sess.decode()
    _check_full(case, sess, "NHD + strided q")


def test_page_permutation_and_repeat_bit_identical():
    _need_gpu()
    import torch
    case = synth.few_kv_long(L=5900, seed=55)
    sess, t = session_for(case, requested_splits=16)
    sess.decode()
    torch.cuda.synchronize()
    out1, lse1 = sess.out.clone(), sess.lse.clone()
    sess.decode()
    torch.cuda.synchronize()
    assert torch.equal(out1, sess.out) and torch.equal(lse1, sess.lse), "repeat run differs"
    # move every page to another physical slot
    rng = np.random.default_rng(99)
    perm = rng.permutation(case.num_pages)
    case2 = synth.few_kv_long(L=5900, seed=55)
    case2.k_cache = np.empty_like(case.k_cache)
    case2.v_cache = np.empty_like(case.v_cache)
    case2.k_cache[perm] = case.k_cache
    case2.v_cache[perm] = case.v_cache
    bt = case.block_table.copy()
    valid = bt != synth.INT32_MAX
    bt[valid] = perm[bt[valid]]
    case2.block_table = bt
    log("page permutation invariance L=5900 n=16")
    sess2, _ = session_for(case2, requested_splits=16)
    sess2.decode()
    torch.cuda.synchronize()
    assert torch.equal(out1, sess2.out) and torch.equal(lse1, sess2.lse)


# ---- full-size workloads, every row -----------------------------------------

def test_fp8_full_size():
    _need_gpu()
    case = synth.fp8_batched()
    log(f"fp8 full B=8 L=32000 auto plan, every row")
    sess, _ = session_for(case, requested_splits=0)
    log(f"  plan: splits {sess.num_splits_host.tolist()}")
    sess.decode()
    _check_full(case, sess, "fp8 full", cache=True)


@pytest.mark.parametrize("n", [1, 4, 8, 0])
def test_mla_full_size(n):
    _need_gpu()
    case = synth.mla_decode(L=65536)
    log(f"mla full L=65536 n={n}, every row")
    sess, _ = session_for(case, requested_splits=n, max_splits=256)
    sess.decode()
    _check_full(case, sess, f"mla full n={n}", cache=True)


def test_ragged_full_size():
    _need_gpu()
    case = synth.ragged()
    log(f"ragged full B=32 seed={case.seed}, sum L={int(case.seq_lens.sum())}, every row")
    sess, _ = session_for(case, requested_splits=0, debug=True)
    log(f"  plan total slots {sess.total_slots}")
    sess.decode()
    _check_debug(case, sess, case.Hkv, 1)
    _check_full(case, sess, "ragged full", cache=True)


# ---------------------------------------------------------------------------
# Running-max jumps inside a split.  The kernels keep O relative to a reference
# maximum per row and rescale O and l only when a tile's row maximum passes it
# by more than 8 in base 2; keys scaled up part-way through the sequence make
# that happen inside splits (tests/test_ramp_inputs.py checks the jump on the
# CPU).

def ramped_mla():
    case = synth.mla_decode(L=2048, seed=21)
    return synth.ramp_keys(case, [(700, 30.0), (1300, 100.0)], d0=512)


def ramped_mla_e4m3(fp8_queries):
    # the cache scale leaves room for the x100 rope features (2.65 is about
    # the largest |x| of the N(0, 0.5) draw)
    case = synth.make_case("mla-fp8-ramp", B=1, T=6, Hq=128, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=[2048], page_size=64, mla=True, std=0.5, seed=23,
                           kv_dtype=synth.KV_E4M3, fp8_scale=100 * 2.65 / 448,
                           fp8_queries=fp8_queries)
    return synth.ramp_keys(case, [(700, 30.0), (1300, 100.0)], d0=512)


def ramped_few_kv():
    case = synth.few_kv_long(L=2000, seed=22)
    return synth.ramp_keys(case, [(700, 4.0), (1300, 16.0)])


@pytest.mark.parametrize("n", [1, 4])
def test_mla_rescale_inside_split(n):
    _need_gpu()
    case = ramped_mla()
    log(f"mla L=2048 keys ramped x30 at 700, x100 at 1300, n={n}")
    sess, _ = session_for(case, requested_splits=n)
    sess.decode()
    _check_full(case, sess, f"mla ramp n={n}")


@pytest.mark.parametrize("fp8_queries", [False, True])
@pytest.mark.parametrize("n", [1, 4])
def test_mla_e4m3_rescale_inside_split(n, fp8_queries):
    _need_gpu()
    case = ramped_mla_e4m3(fp8_queries)
    log(f"mla e4m3 cache, {'e4m3' if fp8_queries else 'bf16'} queries, L=2048 rope keys ramped "
        f"x30 at 700, x100 at 1300, n={n}")
    sess, _ = session_for(case, requested_splits=n)
    sess.decode()
    _check_full(case, sess, f"mla e4m3 ramp n={n} q8={fp8_queries}")


@pytest.mark.parametrize("n", [1, 4])
def test_gqa_rescale_inside_split(n):
    _need_gpu()
    case = ramped_few_kv()
    log(f"few-kv L=2000 keys ramped x4 at 700, x16 at 1300, n={n}")
    sess, _ = session_for(case, requested_splits=n)
    sess.decode()
    _check_full(case, sess, f"gqa ramp n={n}")


# ---------------------------------------------------------------------------
# Empty sequences: L = 0 (no cached token at all; its one page holds only
# poison) and, for six draft tokens, L < T (the first tokens see no key).
# Such rows give out = 0 and lse = -inf.

@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_E4M3])
@pytest.mark.parametrize("n", [0, 1, 4])
def test_gqa_zero_length_sequences(kv_dtype, n):
    _need_gpu()
    case = synth.make_case("zero-len", B=4, T=1, Hq=8, Hkv=2, d_qk=128, d_v=128,
                           seq_lens=[0, 5, 300, 0], page_size=16, kv_dtype=kv_dtype, seed=3)
    log(f"gqa {kv_dtype} seq_lens=[0,5,300,0] n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"zero-len {kv_dtype} n={n}")
    _check_debug(case, sess, case.Hkv, 1)


@pytest.mark.parametrize("n", [1, 4])
def test_mla_sequences_shorter_than_the_draft(n):
    _need_gpu()
    case = synth.make_case("mla-short", B=3, T=6, Hq=128, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=[0, 3, 100], page_size=64, mla=True, std=0.5, seed=4)
    log(f"mla seq_lens=[0,3,100] T=6 n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla short n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


# ---------------------------------------------------------------------------
# MLA over an e4m3 latent cache (bf16 queries, one per-tensor scale shared by
# keys and values): the codes are widened exactly, so the bar is the FP8 one
# against the oracle on the same dequantised values.

@pytest.mark.parametrize("n", [1, 4, 8])
def test_mla_fp8_small_full_compare(n):
    _need_gpu()
    case = synth.mla_decode(L=2048, kv_dtype=synth.KV_E4M3)
    log(f"mla e4m3 L=2048 n={n} k_scale={case.k_scale}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla e4m3 n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


def test_mla_fp8_tiles_cut_by_ranges_and_pages():
    _need_gpu()
    case = synth.mla_decode(L=2000, seed=13, kv_dtype=synth.KV_E4M3)
    log("mla e4m3 L=2000 n=3 (partial tiles, tiles across pages)")
    sess, _ = session_for(case, requested_splits=3, debug=True)
    sess.decode()
    _check_full(case, sess, "mla e4m3 L=2000 n=3")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


@pytest.mark.parametrize("n", [1, 4])
def test_mla_fp8_sequences_shorter_than_the_draft(n):
    _need_gpu()
    case = synth.make_case("mla-fp8-short", B=3, T=6, Hq=128, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=[0, 3, 100], page_size=64, mla=True, std=0.5, seed=4,
                           kv_dtype=synth.KV_E4M3)
    log(f"mla e4m3 seq_lens=[0,3,100] n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla e4m3 short n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


def test_mla_fp8_full_size():
    _need_gpu()
    case = synth.mla_decode(L=65536, kv_dtype=synth.KV_E4M3)
    log("mla e4m3 L=65536 auto plan, every row")
    sess, _ = session_for(case, requested_splits=0, max_splits=256)
    sess.decode()
    _check_full(case, sess, "mla e4m3 L=65536", cache=True)


# ---------------------------------------------------------------------------
# MLA with e4m3 queries over the e4m3 latent cache (the FP8 matrix path): the
# oracle quantises the queries with the same per-tensor encoding and attends
# exactly over the dequantised values (the FP8 bar, 3e-2).

@pytest.mark.parametrize("n", [1, 4, 8])
def test_mla_fp8q_small_full_compare(n):
    _need_gpu()
    case = synth.mla_decode(L=2048, kv_dtype=synth.KV_E4M3, fp8_queries=True)
    log(f"mla e4m3 queries L=2048 n={n} q_scale={case.q_scale} k_scale={case.k_scale}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla fp8q n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


def test_mla_fp8q_tiles_cut_by_ranges_and_pages():
    _need_gpu()
    case = synth.mla_decode(L=2000, seed=13, kv_dtype=synth.KV_E4M3, fp8_queries=True)
    log("mla e4m3 queries L=2000 n=3 (partial sub-tiles and windows, sub-tiles across pages)")
    sess, _ = session_for(case, requested_splits=3, debug=True)
    sess.decode()
    _check_full(case, sess, "mla fp8q L=2000 n=3")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


@pytest.mark.parametrize("n", [1, 4])
def test_mla_fp8q_sequences_shorter_than_the_draft(n):
    _need_gpu()
    case = synth.make_case("mla-fp8q-short", B=3, T=6, Hq=128, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=[0, 3, 100], page_size=64, mla=True, std=0.5, seed=4,
                           kv_dtype=synth.KV_E4M3, fp8_queries=True)
    log(f"mla e4m3 queries seq_lens=[0,3,100] n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla fp8q short n={n}")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


@pytest.mark.parametrize("T,Hq,L,n", [(1, 128, 3000, 4), (2, 16, 777, 3), (3, 40, 1500, 0)])
def test_mla_fp8q_other_shapes(T, Hq, L, n):
    _need_gpu()
    case = synth.mla_decode(L=L, seed=60 + T, T=T, Hq=Hq, kv_dtype=synth.KV_E4M3, fp8_queries=True)
    log(f"mla e4m3 queries T={T} Hq={Hq} L={L} n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla fp8q T={T} Hq={Hq}")
    _check_debug(case, sess, 1, -(-(T * Hq) // MLA_RPW))


def test_mla_fp8q_saturating_scale_strided_query_nhd_cache():
    # q_scale an eighth of amax|q| / 448: the largest query values saturate at
    # +-448 codes (the oracle applies the same clamp); the query is a strided
    # view (padded head dimension) and the latent cache is stored NHD
    import dataclasses
    _need_gpu()
    case = synth.mla_decode(L=1000, seed=71, kv_dtype=synth.KV_E4M3, fp8_queries=True)
    case = dataclasses.replace(case, q_scale=float(np.float32(case.q_scale / 8)))
    qv = np.abs(oracle.decode_bf16(case.q)) / case.q_scale
    log(f"mla e4m3 queries, q_scale={case.q_scale}: {int((qv > 448).sum())} query values saturate")
    assert (qv > 448).sum() > 100
    sess, _ = session_for(case, requested_splits=4, layout="NHD", q_pad_heads=3, debug=True)
    sess.decode()
    _check_full(case, sess, "mla fp8q saturating q_scale, NHD, strided q")
    _check_debug(case, sess, 1, -(-768 // MLA_RPW))


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_E4M3])
@pytest.mark.parametrize("pad", ["heads", "dim"])
def test_mla_query_row_layouts(kv_dtype, pad):
    # The query rows (t, h) of a sequence are read either as evenly spaced
    # rows (a padded row: stride 600 elements, 600 * Hq per token) or, when
    # the token stride is not Hq row strides (padded heads), one row at a time;
    # 3 x 40 rows leave a partial last block of 128.
    _need_gpu()
    case = synth.mla_decode(L=1500, seed=83, T=3, Hq=40, kv_dtype=kv_dtype)
    log(f"mla {kv_dtype} query padded along {pad}")
    sess, t = session_for(case, requested_splits=5, q_pad_heads=3 if pad == "heads" else 0,
                          q_pad_dim=24 if pad == "dim" else 0, debug=True)
    q = t["q"]
    assert q.stride(2) == (600 if pad == "dim" else 576)
    assert (q.stride(1) == 40 * q.stride(2)) == (pad == "dim")
    sess.decode()
    _check_full(case, sess, f"mla {kv_dtype} query padded along {pad}")
    _check_debug(case, sess, 1, -(-(3 * 40) // MLA_RPW))


@pytest.mark.parametrize("path", ["gqa-bf16", "gqa-e4m3", "mla-bf16", "mla-e4m3", "mla-e4m3-queries"])
def test_rows_without_visible_keys_beside_visible_ones(path):
    # The lazy rescale moves the rows of a 16-row block whose maximum jumped
    # and must leave the others untouched, including rows that have seen no
    # key yet (it once computed their factor as exp2(-inf + inf) = NaN).
    # Grouped-query: T=4 x 4 heads per block; L=305 in 19 splits leaves a
    # last split [288, 305) whose second group (another wave) holds token
    # 304, seen only by the last draft token, so the other rows are empty in
    # that wave but not in the workgroup.  MLA: T=3 x 40 heads puts draft
    # tokens 0 and 1 in one block; with L=2 and one split, token 0's rows see
    # nothing while token 1's see a key, and single-split rows are written
    # straight to the output.
    _need_gpu()
    kv = synth.KV_BF16 if path.endswith("bf16") else synth.KV_E4M3
    if path.startswith("gqa"):
        case = synth.make_case("mixed-visibility", B=1, T=4, Hq=16, Hkv=4, d_qk=128, d_v=128,
                               seq_lens=[305], page_size=16, kv_dtype=kv, seed=33)
        n, blocks, hkv = 19, 1, 4
    else:
        case = synth.make_case("mixed-visibility-mla", B=2, T=3, Hq=40, Hkv=1, d_qk=576, d_v=512,
                               seq_lens=[2, 300], page_size=64, mla=True, std=0.5, seed=34, kv_dtype=kv,
                               fp8_queries=path.endswith("queries"))
        n, blocks, hkv = 1, -(-(3 * 40) // MLA_RPW), 1
    log(f"{path}: rows with and without visible keys in one block, n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"{path} mixed visibility")
    _check_debug(case, sess, hkv, blocks)


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_E4M3])
@pytest.mark.parametrize("seed", range(8))
def test_gqa_random_shapes(seed, kv):
    # seeded draws of batch, query tokens, head grouping, head dim, lengths,
    # page size (any multiple of 16), cache layout and split request
    _need_gpu()
    rng = np.random.default_rng(800 + seed)
    B = int(rng.integers(1, 5))
    T = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    d = int(rng.choice([128, 256]))
    lens = [int(x) for x in rng.integers(0, 3000, size=B)]
    P = int(rng.choice([16, 32, 48, 64, 256]))
    layout = str(rng.choice(["HND", "NHD"]))
    n = int(rng.choice([0, 1, 3, 8, 40]))
    case = synth.make_case(f"gqa-rand{seed}", B=B, T=T, Hq=g * Hkv, Hkv=Hkv, d_qk=d, d_v=d,
                           seq_lens=lens, page_size=P, kv_dtype=kv, seed=810 + seed)
    log(f"gqa {kv} random seed={seed}: B={B} T={T} Hq={g * Hkv} Hkv={Hkv} d={d} L={lens} P={P} "
        f"{layout} n={n}")
    sess, _ = session_for(case, requested_splits=n, layout=layout, debug=True)
    sess.decode()
    _check_full(case, sess, f"gqa {kv} random seed={seed}")
    _check_debug(case, sess, Hkv, -(-(T * g) // 16))


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_E4M3])
@pytest.mark.parametrize("seed", range(4))
def test_gqa_head_dim_64_random_shapes(seed, kv):
    # head dimension 64: the value loads cover half of a 128-feature lane
    # row, and the merge runs on 16 float4 columns per row
    _need_gpu()
    rng = np.random.default_rng(700 + seed)
    B = int(rng.integers(1, 5))
    T = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8, 16]))
    lens = [int(x) for x in rng.integers(0, 3000, size=B)]
    P = int(rng.choice([16, 64, 128]))
    n = int(rng.choice([0, 1, 4, 30]))
    layout = str(rng.choice(["HND", "NHD"]))
    case = synth.make_case(f"gqa-d64-rand{seed}", B=B, T=T, Hq=g * Hkv, Hkv=Hkv, d_qk=64, d_v=64,
                           seq_lens=lens, page_size=P, kv_dtype=kv, seed=710 + seed)
    log(f"gqa d=64 {kv} seed={seed}: B={B} T={T} Hq={g * Hkv} Hkv={Hkv} L={lens} P={P} {layout} n={n}")
    sess, _ = session_for(case, requested_splits=n, layout=layout, debug=True)
    sess.decode()
    _check_full(case, sess, f"gqa d=64 {kv} seed={seed}")
    _check_debug(case, sess, Hkv, -(-(T * g) // 16))


@pytest.mark.parametrize("mode", ["bf16", "e4m3", "e4m3-queries"])
@pytest.mark.parametrize("seed", range(6))
def test_mla_random_shapes(seed, mode):
    # seeded draws of batch, draft length, head count, lengths (tiles, windows
    # and sub-tiles cut anywhere), page size and split request, for each MLA path
    _need_gpu()
    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 7))
    Hq = int(rng.choice([16, 40, 64, 128]))
    lens = [int(x) for x in rng.integers(0, 2600, size=B)]
    n = int(rng.choice([0, 1, 2, 5, 9]))
    case = synth.make_case(f"mla-rand{seed}", B=B, T=T, Hq=Hq, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=lens, page_size=int(rng.choice([16, 64, 128])), mla=True,
                           std=0.5, seed=910 + seed,
                           kv_dtype=synth.KV_BF16 if mode == "bf16" else synth.KV_E4M3,
                           fp8_queries=mode == "e4m3-queries")
    log(f"mla {mode} random seed={seed}: B={B} T={T} Hq={Hq} L={lens} P={case.page_size} n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla {mode} random seed={seed}")
    _check_debug(case, sess, 1, -(-(T * Hq) // MLA_RPW))


def test_mla_fp8q_full_size():
    _need_gpu()
    case = synth.mla_decode(L=65536, kv_dtype=synth.KV_E4M3, fp8_queries=True)
    log("mla e4m3 queries L=65536 auto plan, every row")
    sess, _ = session_for(case, requested_splits=0, max_splits=256)
    sess.decode()
    _check_full(case, sess, "mla fp8q L=65536", cache=True)


# ---------------------------------------------------------------------------
# MLA at other decode shapes: one token (no causal mask within the draft),
# and head counts whose T*Hq rows leave the last 128-row block partly empty.

@pytest.mark.parametrize("T,Hq,L,n", [(1, 128, 3000, 4), (2, 16, 777, 3), (3, 40, 1500, 0)])
@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_E4M3])
def test_mla_other_shapes(T, Hq, L, n, kv_dtype):
    _need_gpu()
    case = synth.mla_decode(L=L, seed=50 + T, T=T, Hq=Hq, kv_dtype=kv_dtype)
    log(f"mla {kv_dtype} T={T} Hq={Hq} L={L} n={n}")
    sess, _ = session_for(case, requested_splits=n, debug=True)
    sess.decode()
    _check_full(case, sess, f"mla {kv_dtype} T={T} Hq={Hq}")
    _check_debug(case, sess, 1, -(-(T * Hq) // MLA_RPW))

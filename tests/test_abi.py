"""CPU checks of the C ABI: the library loads, exports every declared symbol,
its host planner matches the oracle's independent planner bit for bit, and
bad arguments come back as status codes (no device is touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import split_kv_amd as sk
from oracle import plan as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        return sk.load()
    except RuntimeError as e:
        pytest.fail(f"library not built: {e}")


def test_exports_every_declared_symbol():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "splitkv.h")).read()
    declared = set(re.findall(r"\b(splitkv_[a-z0-9_]+)\s*\(", header))
    assert declared, "no declarations parsed"
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in splitkv.h but not exported"
    assert declared == set(sk.EXPORTED)


def test_struct_layouts_match():
    lib = _lib()
    assert lib.splitkv_args_size() == ctypes.sizeof(sk.splitkv_args)
    assert lib.splitkv_plan_args_size() == ctypes.sizeof(sk.splitkv_plan_args)
    assert lib.splitkv_append_args_size() == ctypes.sizeof(sk.splitkv_append_args)


def test_constants_agree_with_oracle():
    assert sk.SPLITKV_GRANULE == oplan.GRANULE
    assert sk.SPLITKV_AUTO_SPLIT_MIN_BYTES == oplan.AUTO_SPLIT_MIN_BYTES
    assert sk.SPLITKV_AUTO_LAT_NUM == oplan.AUTO_LAT_NUM
    assert sk.SPLITKV_AUTO_LAT_DEN == oplan.AUTO_LAT_DEN
    assert sk.SPLITKV_AUTO_BALANCE == oplan.AUTO_BALANCE
    assert sk.SPLITKV_AUTO_WG_OVERHEAD_BYTES == oplan.AUTO_WG_OVERHEAD_BYTES
    assert sk.SPLITKV_MAX_SPLITS_LIMIT == oplan.MAX_SPLITS_LIMIT
    assert sk.SPLITKV_ROWS_PER_WG_GQA == oplan.ROWS_PER_WG_GQA
    assert sk.SPLITKV_ROWS_PER_WG_MLA == oplan.ROWS_PER_WG_MLA
    header = open(os.path.join(ROOT, "include", "splitkv.h")).read()
    for name in ("GRANULE", "AUTO_SPLIT_MIN_BYTES", "AUTO_LAT_NUM", "AUTO_LAT_DEN", "AUTO_BALANCE",
                 "AUTO_WG_OVERHEAD_BYTES", "MAX_SPLITS_LIMIT", "ROWS_PER_WG_GQA", "ROWS_PER_WG_MLA"):
        m = re.search(rf"#define SPLITKV_{name} (\d+)", header)
        assert int(m.group(1)) == getattr(sk, f"SPLITKV_{name}")


def test_split_range_matches_oracle():
    _lib()
    for L in list(range(0, 700)) + [5900, 32000, 65536, 131072]:
        nblk = max(1, -(-L // 16))
        for n in (1, 2, 3, 5, 7, 16, 33, 64, 255):
            if n > nblk:
                continue
            for i in range(n):
                assert sk.splitkv_split_range(L, n, i) == oplan.split_range(L, n, i)


def _plan(lens, T, Hq, Hkv, kernel, req, mx, cus, d_qk=128, d_v=128, kv=sk.SPLITKV_KV_BF16):
    pa = sk.splitkv_plan_args(B=len(lens), T=T, Hq=Hq, Hkv=Hkv, kernel=kernel, requested_splits=req,
                              max_splits=mx, num_cus=cus, d_qk=d_qk, d_v=d_v, kv_dtype=kv)
    return sk.splitkv_plan(pa, lens)


def _oplan(lens, T, Hq, Hkv, kernel, req, mx, cus, d_qk=128, d_v=128, kv=sk.SPLITKV_KV_BF16):
    rpw = oplan.ROWS_PER_WG_MLA if kernel == sk.SPLITKV_KERNEL_MLA else oplan.ROWS_PER_WG_GQA
    return oplan.make_plan(lens, T=T, Hq=Hq, Hkv=Hkv, requested=req, max_splits=mx, num_cus=cus,
                           rows_per_wg=rpw, d_qk=d_qk, d_v=d_v,
                           elem=1 if kv == sk.SPLITKV_KV_E4M3 else 2)


# (d_qk, d_v, kv dtype) per kernel: the configurations the kernels are built for
HEADS = {sk.SPLITKV_KERNEL_GQA: [(64, 64, sk.SPLITKV_KV_BF16), (128, 128, sk.SPLITKV_KV_BF16),
                                 (256, 256, sk.SPLITKV_KV_BF16), (64, 64, sk.SPLITKV_KV_E4M3),
                                 (128, 128, sk.SPLITKV_KV_E4M3), (256, 256, sk.SPLITKV_KV_E4M3)],
         sk.SPLITKV_KERNEL_MLA: [(576, 512, sk.SPLITKV_KV_BF16), (576, 512, sk.SPLITKV_KV_E4M3)]}


@pytest.mark.parametrize("kernel", [sk.SPLITKV_KERNEL_GQA, sk.SPLITKV_KERNEL_MLA])
def test_planner_bit_exact_against_oracle(kernel):
    _lib()
    shapes = [(1, 16, 2), (1, 32, 4), (6, 128, 1), (1, 32, 8), (2, 8, 2)]
    for L in list(range(0, 4097, 37)) + [5900, 32000, 65536, 131072]:
        for (T, Hq, Hkv) in shapes:
            for n in (0, 1, 2, 3, 8, 17, 64):
                for mx in (1, 8, 64, 256):
                    for cus in (1, 80, 256):
                        for hd in HEADS[kernel]:
                            got = _plan([L], T, Hq, Hkv, kernel, n, mx, cus, *hd)
                            ref = _oplan([L], T, Hq, Hkv, kernel, n, mx, cus, *hd)
                            for a, b in zip(got, ref):
                                assert np.array_equal(a, b), (L, T, Hq, Hkv, n, mx, cus, hd)
    # batches: ragged ones as the ragged workload draws them, and uniform ones
    import synth
    batches = [synth.log_uniform_lengths(np.random.default_rng(seed), 32) for seed in range(20)]
    batches += [[32000] * 8, [5900] * 3, [1, 2, 15, 16, 17, 255, 131072], [300] * 64, [0, 0, 7]]
    for lens in batches:
        for (T, Hq, Hkv) in [(1, 32, 8), (1, 32, 4), (6, 128, 1)]:
            for n in (0, 1, 4, 16, 64):
                for mx in (64, 256):
                    for hd in HEADS[kernel]:
                        got = _plan(lens, T, Hq, Hkv, kernel, n, mx, 256, *hd)
                        ref = _oplan(lens, T, Hq, Hkv, kernel, n, mx, 256, *hd)
                        for a, b in zip(got, ref):
                            assert np.array_equal(a, b), (lens, T, Hq, Hkv, n, mx, hd)


def test_requested_count_is_honoured():
    _lib()
    for n in range(1, 65):
        ns, off, seq = _plan([5900], 1, 16, 2, sk.SPLITKV_KERNEL_GQA, n, 64, 256)
        assert ns[0] == n and off[-1] == n


def test_plan_errors():
    _lib()
    with pytest.raises(sk.SplitKVError):
        _plan([10], 1, 16, 3, 0, 1, 64, 256)            # Hq % Hkv != 0
    with pytest.raises(sk.SplitKVError):
        _plan([10], 1, 16, 2, 0, 1, 300, 256)           # max_splits above the limit
    with pytest.raises(sk.SplitKVError):
        _plan([-1], 1, 16, 2, 0, 1, 64, 256)            # negative length
    with pytest.raises(sk.SplitKVError):
        _plan([10], 1, 16, 2, 7, 1, 64, 256)            # unknown kernel
    with pytest.raises(sk.SplitKVError):
        _plan([10], 1, 16, 2, 0, 0, 64, 256, d_qk=0)    # head dimension missing
    with pytest.raises(sk.SplitKVError):
        _plan([10], 1, 16, 2, 0, 0, 64, 256, kv=5)      # unknown KV dtype


def test_workspace_bytes():
    _lib()
    S, T, Hq, dv = 13, 2, 16, 256
    rows = S * T * Hq
    ml = -(-(2 * rows * 4) // 256) * 256
    assert sk.splitkv_workspace_bytes(S, T, Hq, dv) == ml + rows * dv * 4


def test_validate_block_table():
    _lib()
    bt = np.array([[3, 1, 2**31 - 1], [0, 2, 4]], dtype=np.int32)
    sk.splitkv_validate_block_table(bt, [20, 40], 16, 5)
    with pytest.raises(sk.SplitKVError):
        sk.splitkv_validate_block_table(bt, [40, 40], 16, 5)    # reads the padding entry
    with pytest.raises(sk.SplitKVError):
        sk.splitkv_validate_block_table(bt, [20, 40], 16, 4)    # page 4 out of range


def _args(**over):
    a = sk.splitkv_args()
    base = dict(q=0x1000, q_stride_b=16 * 128, q_stride_t=16 * 128, q_stride_h=128,
                k_cache=0x2000, v_cache=0x3000, k_stride_page=2 * 16 * 128, k_stride_head=16 * 128,
                k_stride_tok=128, v_stride_page=2 * 16 * 128, v_stride_head=16 * 128,
                v_stride_tok=128, block_table=0x4000, bt_stride=4, seq_lens=0x5000,
                num_splits=0x5100, slot_offset=0x5200, slot_info=0x5300, total_slots=1, B=1, T=1,
                Hq=16, Hkv=2, d_qk=128, d_v=128, page_size=16, num_pages=4, kv_dtype=0,
                scale=0.1, k_scale=1.0, v_scale=1.0, workspace=0x6000, workspace_bytes=1 << 20,
                out=0x7000, out_dtype=0, lse=0x8000, debug=None)
    base.update(over)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(q=None), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(Hkv=3), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(d_qk=96, d_v=96), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(d_qk=64, d_v=128), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(page_size=24), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(q=0x1008), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(k_stride_tok=100), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(workspace_bytes=16), sk.SPLITKV_ERR_WORKSPACE),
    (dict(kv_dtype=1), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(total_slots=0), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(scale=0.0), sk.SPLITKV_ERR_INVALID_ARG),
])
def test_decode_argument_errors_without_device(over, code):
    lib = _lib()
    a = _args(**over)
    st = lib.splitkv_decode_partial(ctypes.byref(a), None)
    assert st == code, (st, sk.splitkv_last_error())
    assert sk.splitkv_last_error()


def test_uniform_splits_must_match_the_slot_count():
    lib = _lib()
    a = _args(uniform_splits=3)             # B = 1 but total_slots = 1
    assert lib.splitkv_combine(ctypes.byref(a), None) == sk.SPLITKV_ERR_INVALID_ARG
    assert "uniform_splits" in sk.splitkv_last_error()
    a = _args(uniform_splits=-1)
    assert lib.splitkv_combine(ctypes.byref(a), None) == sk.SPLITKV_ERR_INVALID_ARG


@pytest.mark.parametrize("m", [-1, 257])
def test_max_seq_splits_hint_range(m):
    lib = _lib()
    a = _args(max_seq_splits=m)
    assert lib.splitkv_combine(ctypes.byref(a), None) == sk.SPLITKV_ERR_INVALID_ARG
    assert "max_seq_splits" in sk.splitkv_last_error()


def test_mla_shape_errors_without_device():
    lib = _lib()
    a = _args(Hkv=1, d_qk=576, d_v=256, Hq=128, T=6)
    assert lib.splitkv_mla_decode_partial(ctypes.byref(a), None) == sk.SPLITKV_ERR_UNSUPPORTED
    a = _args(kv_dtype=1)
    assert lib.splitkv_decode(ctypes.byref(a), 5, None) == sk.SPLITKV_ERR_INVALID_ARG


@pytest.mark.parametrize("over,code", [
    (dict(q_dtype=7), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(q_dtype=1, q_scale=0.0), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(q_dtype=1, q_scale=float("inf")), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(q_dtype=1, q_scale=0.01, kv_dtype=0), sk.SPLITKV_ERR_UNSUPPORTED),
])
def test_e4m3_query_errors_without_device(over, code):
    # an MLA-shaped call over an e4m3 cache; the workspace is also too small,
    # so no case here can get past validation
    lib = _lib()
    base = dict(Hkv=1, Hq=128, T=6, d_qk=576, d_v=512, kv_dtype=1, q_stride_b=6 * 128 * 576,
                q_stride_t=128 * 576, q_stride_h=576, k_stride_page=16 * 576, k_stride_head=16 * 576,
                k_stride_tok=576, workspace_bytes=16)
    base.update(over)
    a = _args(**base)
    assert lib.splitkv_mla_decode_partial(ctypes.byref(a), None) == code, sk.splitkv_last_error()
    assert "q_" in sk.splitkv_last_error() or "e4m3 queries" in sk.splitkv_last_error()
    # the grouped-query kernels take no e4m3 queries
    a = _args(q_dtype=1, q_scale=0.01, workspace_bytes=16)
    assert lib.splitkv_decode_partial(ctypes.byref(a), None) == sk.SPLITKV_ERR_UNSUPPORTED
    assert "e4m3 queries" in sk.splitkv_last_error()


def _append_args(**over):
    a = sk.splitkv_append_args()
    base = dict(k_new=0x1000, v_new=0x1800, k_new_stride_b=2 * 128, k_new_stride_t=2 * 128,
                k_new_stride_h=128, v_new_stride_b=2 * 128, v_new_stride_t=2 * 128,
                v_new_stride_h=128, k_cache=0x2000, v_cache=0x3000, k_stride_page=2 * 16 * 128,
                k_stride_head=16 * 128, k_stride_tok=128, v_stride_page=2 * 16 * 128,
                v_stride_head=16 * 128, v_stride_tok=128, block_table=0x4000, bt_stride=4,
                positions=0x5000, B=1, T=1, Hkv=2, d_k=128, d_v=128, page_size=16, num_pages=4,
                kv_dtype=1, k_scale=0.5, v_scale=0.5)
    base.update(over)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(k_new=None), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(v_new=None), sk.SPLITKV_ERR_INVALID_ARG),          # v_cache given without v_new
    (dict(positions=None), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(T=0), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(num_pages=0), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(d_k=100), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(k_scale=0.0), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(v_scale=float("inf")), sk.SPLITKV_ERR_INVALID_ARG),
    (dict(k_new=0x1008), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(k_stride_tok=100), sk.SPLITKV_ERR_UNSUPPORTED),
    (dict(kv_dtype=0, k_stride_tok=4), sk.SPLITKV_ERR_UNSUPPORTED),   # 8 bytes: not 16-aligned for bf16
    (dict(block_table=0x4002), sk.SPLITKV_ERR_INVALID_ARG),
])
def test_append_argument_errors_without_device(over, code):
    lib = _lib()
    a = _append_args(**over)
    st = lib.splitkv_append_kv(ctypes.byref(a), None)
    assert st == code, (st, sk.splitkv_last_error())
    assert sk.splitkv_last_error()


def test_version_string():
    _lib()
    assert sk.splitkv_version()


def test_noalloc_refuses_an_oversized_plan_without_a_device():
    # 256 MLA slots of 768 rows need ~404 MB of partials, more than the
    # library's 64 MiB buffer: refused on the host, before any device call
    lib = _lib()
    a = sk.splitkv_args()
    a.B, a.T, a.Hq, a.Hkv, a.d_qk, a.d_v, a.total_slots = 1, 6, 128, 1, 576, 512, 256
    assert sk.splitkv_workspace_bytes(256, 6, 128, 512) > sk.SPLITKV_NOALLOC_SCRATCH_BYTES
    st = lib.splitkv_decode_noalloc(ctypes.byref(a), sk.SPLITKV_KERNEL_MLA, None)
    assert st == sk.SPLITKV_ERR_WORKSPACE
    assert "library buffer" in sk.splitkv_last_error()


def test_calibration_argument_errors_without_device():
    # the probes check their arguments before touching a device
    lib = sk.load()
    ok_sink = ctypes.c_void_p(256)
    assert lib.splitkv_calib_mfma(1, 1, None, None) == sk.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_calib_mfma(0, 1, ok_sink, None) == sk.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_calib_mfma(1, 0, ok_sink, None) == sk.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_calib_mfma(1, 1, ctypes.c_void_p(258), None) == sk.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_calib_lds_read(1, 1, 2, ok_sink, None) == sk.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_calib_lds_read(1, (1 << 24) + 1, 0, ok_sink, None) == sk.SPLITKV_ERR_INVALID_ARG
    assert "splitkv_calib_lds_read" in sk.splitkv_last_error()


def test_mla_kernel_choice_query(monkeypatch):
    # no hint: the 128-row kernel; the environment switch forces either;
    # a null args is the 128-row kernel too
    lib = sk.load()
    assert lib.splitkv_mla_short_range(None) == 0
    a = sk.splitkv_args()
    a.B, a.T, a.Hq, a.Hkv, a.total_slots, a.max_range_tokens = 1, 6, 128, 1, 18, 0
    monkeypatch.delenv("SPLITKV_MLA_KERNEL", raising=False)
    assert not sk.splitkv_mla_short_range(a)
    monkeypatch.setenv("SPLITKV_MLA_KERNEL", "short")
    assert sk.splitkv_mla_short_range(a)
    monkeypatch.setenv("SPLITKV_MLA_KERNEL", "long")
    a.max_range_tokens = 114
    assert not sk.splitkv_mla_short_range(a)

"""GPU parity of the KV append step (splitkv_append_kv through the C ABI).

The cache written by the kernel must equal the oracle's byte for byte: the
new rows in their slots (bf16 codes unchanged, or e4m3 codes of x / scale),
every other byte untouched -- including the poisoned page tails and spare
pages of the synthetic caches, and the rows of tokens the call must skip.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev_cache(arr, layout):
    """[pages][H][P][D] codes -> device tensor holding them in `layout`, and its element strides."""
    import torch
    host = torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr)
    if layout == "NHD":
        t = host.permute(0, 2, 1, 3).contiguous().cuda()        # stored [page][slot][head][d]
        st = (t.stride(0), t.stride(2), t.stride(1))             # page, head, token
    else:
        t = host.contiguous().cuda()
        st = (t.stride(0), t.stride(1), t.stride(2))
    return t, st


def _host_cache(t, layout, dtype):
    a = t.cpu().numpy()
    if layout == "NHD":
        a = a.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(a).view(dtype)


def _run(case, k_new, v_new, positions, layout="HND", k_scale=None, v_scale=None, block_table=None):
    import torch
    import split_kv_amd as sk
    fp8 = case.kv_dtype == synth.KV_E4M3
    cdt = np.uint8 if fp8 else np.uint16
    ks = float(case.k_scale if k_scale is None else k_scale)
    vs = float(case.v_scale if v_scale is None else v_scale)
    bt = case.block_table if block_table is None else block_table
    kc, kst = _dev_cache(case.k_cache, layout)
    vc, vst = (None, (0, 0, 0)) if case.v_cache is None else _dev_cache(case.v_cache, layout)
    kn = torch.from_numpy(k_new.view(np.int16)).cuda()
    vn = None if v_new is None else torch.from_numpy(v_new.view(np.int16)).cuda()
    btd = torch.from_numpy(np.ascontiguousarray(bt)).cuda()
    pos = torch.from_numpy(np.asarray(positions, dtype=np.int32)).cuda()
    a = sk.splitkv_append_args()
    a.k_new, a.v_new = kn.data_ptr(), (vn.data_ptr() if vn is not None else None)
    a.k_new_stride_b, a.k_new_stride_t, a.k_new_stride_h = kn.stride(0), kn.stride(1), kn.stride(2)
    if vn is not None:
        a.v_new_stride_b, a.v_new_stride_t, a.v_new_stride_h = vn.stride(0), vn.stride(1), vn.stride(2)
    a.k_cache, a.v_cache = kc.data_ptr(), (vc.data_ptr() if vc is not None else None)
    a.k_stride_page, a.k_stride_head, a.k_stride_tok = kst
    a.v_stride_page, a.v_stride_head, a.v_stride_tok = vst
    a.block_table, a.bt_stride, a.positions = btd.data_ptr(), btd.shape[1], pos.data_ptr()
    B, T, Hkv, dk = k_new.shape
    a.B, a.T, a.Hkv, a.d_k = B, T, Hkv, dk
    a.d_v = v_new.shape[3] if v_new is not None else (512 if case.mla else dk)
    a.page_size, a.num_pages = case.page_size, case.k_cache.shape[0]
    a.kv_dtype = sk.SPLITKV_KV_E4M3 if fp8 else sk.SPLITKV_KV_BF16
    a.k_scale, a.v_scale = ks, vs
    sk.splitkv_append_kv(a, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got_k = _host_cache(kc, layout, cdt)
    got_v = None if vc is None else _host_cache(vc, layout, cdt)
    ref_k, ref_v = oracle.append_kv(case.k_cache, case.v_cache, k_new, v_new, bt, positions,
                                    case.page_size, "e4m3" if fp8 else "bf16", ks, vs)
    return got_k, got_v, ref_k, ref_v


def _check(got_k, got_v, ref_k, ref_v, tag):
    # bit-exact, except that a NaN input may become either e4m3 NaN code
    # (0x7F or 0xFF: the format has two and the sign of a NaN means nothing)
    for name, g, r in (("k", got_k, ref_k), ("v", got_v, ref_v)):
        if r is None:
            assert g is None
            continue
        bad = g != r
        if r.dtype == np.uint8:
            nan_ref = (r & 0x7F) == 0x7F
            bad &= ~(nan_ref & ((g & 0x7F) == 0x7F))
            if nan_ref.any():
                log(f"  {tag} {name}: NaN inputs gave codes {sorted(set(np.unique(g[nan_ref]).tolist()))}")
        assert not bad.any(), (f"{tag} {name}: {int(bad.sum())} codes differ, first at "
                               f"{np.argwhere(bad)[:3].tolist()}: got {g[bad][:3]} want {r[bad][:3]}")
    log(f"  {tag}: caches bit-exact")


def _new_rows(rng, B, T, Hkv, d, std=1.0):
    return synth.to_bf16_codes(rng.standard_normal((B, T, Hkv, d), dtype=np.float32) * np.float32(std))


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_E4M3])
@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("T", [1, 3])
def test_append_gqa(kv_dtype, layout, T):
    _need_gpu()
    rng = np.random.default_rng(41)
    case = synth.make_case("append", B=5, T=1, Hq=16, Hkv=4, d_qk=128, d_v=128,
                           seq_lens=[40, 16, 300, 1, 64], page_size=16, kv_dtype=kv_dtype, seed=17)
    # positions at a page start, a page end, mid-page, zero, the sequence end
    positions = np.array([32, 15, 150, 0, 64 - T], dtype=np.int32)
    kn, vn = _new_rows(rng, 5, T, 4, 128, 3.0), _new_rows(rng, 5, T, 4, 128, 3.0)
    log(f"append gqa {kv_dtype} {layout} T={T} positions={positions.tolist()}")
    _check(*_run(case, kn, vn, positions, layout), f"gqa {kv_dtype} {layout} T={T}")


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_E4M3])
def test_append_latent_mla(kv_dtype):
    _need_gpu()
    rng = np.random.default_rng(42)
    case = synth.make_case("append-mla", B=2, T=1, Hq=128, Hkv=1, d_qk=576, d_v=512,
                           seq_lens=[200, 70], page_size=64, mla=True, kv_dtype=kv_dtype, std=0.5,
                           seed=18)
    positions = np.array([63, 64], dtype=np.int32)
    kn = _new_rows(rng, 2, 6, 1, 576, 0.5)
    log(f"append mla {kv_dtype} T=6 positions={positions.tolist()}")
    _check(*_run(case, kn, None, positions), f"mla {kv_dtype}")


@pytest.mark.parametrize("scale", [1.0, 1 / 64, 7.0, 37.0])
def test_append_quantises_every_bf16_code(scale):
    # one row per 128 bf16 codes: all 65536 codes pass through the conversion
    # (at scale 7, 60 of them round differently if x / scale were computed as
    # x times a rounded reciprocal)
    _need_gpu()
    case = synth.make_case("append-all", B=1, T=1, Hq=1, Hkv=1, d_qk=128, d_v=128,
                           seq_lens=[512], page_size=16, kv_dtype=synth.KV_E4M3, seed=19)
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1, 512, 1, 128)
    vn = codes[:, ::-1].copy()
    log(f"append every bf16 code, scale={scale}")
    _check(*_run(case, codes, vn, np.array([0], dtype=np.int32), k_scale=scale, v_scale=scale),
           f"all codes scale={scale}")


def test_append_skips_tokens_outside_the_table_and_cache():
    _need_gpu()
    rng = np.random.default_rng(43)
    case = synth.make_case("append-skip", B=4, T=1, Hq=8, Hkv=2, d_qk=128, d_v=128,
                           seq_lens=[40, 40, 40, 40], page_size=16, kv_dtype=synth.KV_E4M3, seed=20)
    bt = case.block_table.copy()                 # 3 columns per row
    bt[1, 2] = case.k_cache.shape[0] + 5         # past the cache
    bt[2, 2] = -3                                # negative page
    # sequence 0 at -2: tokens -2, -1 skipped, 0 written; 1 and 2 write into
    # their bad third column (skipped) after one good token; 3 runs past the
    # row's three columns (48 tokens)
    positions = np.array([-2, 31, 31, 46], dtype=np.int32)
    kn, vn = _new_rows(rng, 4, 3, 2, 128), _new_rows(rng, 4, 3, 2, 128)
    log("append with skipped tokens")
    got_k, got_v, ref_k, ref_v = _run(case, kn, vn, positions, block_table=bt)
    _check(got_k, got_v, ref_k, ref_v, "skips")
    changed = int((ref_k != case.k_cache).any(axis=(1, 3)).sum())
    assert changed == 5, changed                 # (0:0) (1:31) (2:31) (3:46) (3:47)

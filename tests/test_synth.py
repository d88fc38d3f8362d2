"""The input generators honour their poison and layout conventions."""
import numpy as np

import synth
from oracle.codes import decode_bf16, decode_e4m3


def test_poison_and_padding_conventions():
    c = synth.make_case("t", B=3, T=1, Hq=4, Hkv=2, d_qk=8, d_v=8, seq_lens=[5, 16, 33],
                        page_size=16, seed=1)
    used = set()
    for b, L in enumerate(c.seq_lens):
        n = -(-int(L) // 16)
        used.update(c.block_table[b, :n].tolist())
        assert (c.block_table[b, n:] == synth.INT32_MAX).all()
        last = c.block_table[b, n - 1]
        tail = int(L) - (n - 1) * 16
        assert np.isnan(decode_bf16(c.k_cache[last, :, tail:])).all()
        assert np.isfinite(decode_bf16(c.k_cache[last, :, :tail])).all()
    spare = [p for p in range(c.num_pages) if p not in used]
    assert spare and np.isnan(decode_bf16(c.v_cache[spare])).all()


def test_fp8_scale_and_clamp():
    c = synth.fp8_batched(B=1, L=64, seed=3)
    v = decode_e4m3(c.k_cache)
    assert np.nanmax(np.abs(v)) == 448.0                 # amax maps to the top code
    c2 = synth.fp8_batched(B=1, L=64, seed=3, fp8_scale=1 / 128)
    v2 = decode_e4m3(c2.k_cache)
    assert (np.abs(v2[np.isfinite(v2)]) == 448.0).sum() > 0   # the clamp fired


def test_workload_shapes():
    c = synth.tiny_gqa()
    assert (c.B, c.Hq, c.Hkv, c.d_qk, c.page_size, c.num_pages) == (1, 8, 2, 128, 256, 1)
    assert c.out_fp32
    c = synth.few_kv_long(L=260)
    assert (c.Hq, c.Hkv, c.d_qk, c.page_size) == (16, 2, 256, 16) and c.kv_bytes() == 260 * 2 * 512 * 2
    c = synth.mla_decode(L=128)
    assert c.mla and c.v_cache is None and c.k_cache.shape[1:] == (1, 64, 576) and c.causal
    c = synth.ragged(B=8, hi=4096)
    assert c.seq_lens.tolist()[:7] == [1, 2, 15, 16, 17, 255, 4096]

"""Pins of the fp64 attention oracle against things other than itself.

* brute force: a scalar loop with math.fsum on tiny inputs;
* a library special case: torch's scaled_dot_product_attention in fp64;
* closed forms: K = 0, V = const, L = 1, two keys (golden fixture);
* index probes: a one-hot key under a random page permutation, and a key just
  past a causal limit;
* the split/combine emulation equals the unsplit result, and the pages'
  empty-split statement (golden fixture).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from oracle import plan as P
from oracle.codes import decode_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_rows(q, K, V, sigma, limits):
    R, n = len(q), len(K)
    O, LSE = [], []
    for r in range(R):
        vis = [j for j in range(n) if j <= limits[r]]
        if not vis:
            O.append([0.0] * len(V[0]))
            LSE.append(-math.inf)
            continue
        s = {j: sigma * math.fsum(q[r][d] * K[j][d] for d in range(len(q[r]))) for j in vis}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in vis}
        l = math.fsum(w.values())
        O.append([math.fsum(w[j] * V[j][d] for j in vis) / l for d in range(len(V[0]))])
        LSE.append(m + math.log(l))
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("seed", range(6))
def test_attend_rows_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, n, d, dv = 5, int(rng.integers(1, 40)), int(rng.integers(1, 8)), int(rng.integers(1, 6))
    q = rng.standard_normal((R, d))
    K = rng.standard_normal((n, d)) * 2
    V = rng.standard_normal((n, dv))
    limits = rng.integers(-1, n + 2, size=R)
    sigma = 0.7
    O, L = A.attend_rows(q, K, V, sigma, limits)
    Ob, Lb = brute_rows(q.tolist(), K.tolist(), V.tolist(), sigma, limits.tolist())
    assert np.allclose(O, Ob, rtol=1e-13, atol=1e-13)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    assert np.allclose(L[fin], Lb[fin], rtol=1e-13, atol=1e-13)


def _case_tiny_paged(seed, B=2, T=1, Hq=8, Hkv=2, D=16, Ls=(37, 64), P=16, kv="bf16"):
    # an explicit FP8 scale of 0.5 leaves room (+-224) for the probe key below
    return synth.make_case("t", B=B, T=T, Hq=Hq, Hkv=Hkv, d_qk=D, d_v=D, seq_lens=list(Ls),
                           page_size=P, kv_dtype=kv, seed=seed,
                           fp8_scale=0.5 if kv == "e4m3" else None)


def test_attend_vs_torch_sdpa_fp64():
    # T = 1: every key is visible, so the result is plain SDPA with the KV heads
    # repeated g times (grouped-query attention) -- a library routine, run in fp64
    c = _case_tiny_paged(3, B=1, Ls=(50,), Hq=8, Hkv=2, D=32)
    O, LSE = A.attend(c)
    L = int(c.seq_lens[0])
    Ks, Vs = [], []
    for hk in range(c.Hkv):
        K, V = A.dequant_kv(c, 0, hk)
        Ks.append(K)
        Vs.append(V)
    K = torch.tensor(np.stack(Ks))            # [Hkv, L, D]
    V = torch.tensor(np.stack(Vs))
    K = K.repeat_interleave(c.g, dim=0)       # [Hq, L, D]
    V = V.repeat_interleave(c.g, dim=0)
    q = torch.tensor(decode_bf16(c.q[0, 0]))[:, None, :]   # [Hq, 1, D]
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=c.scale)[:, 0]
    assert np.allclose(O[0, 0], ref.numpy(), rtol=1e-12, atol=1e-12)
    s = c.scale * torch.einsum("hd,hld->hl", q[:, 0], K)
    assert np.allclose(LSE[0, 0], torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_attend_causal_vs_torch_sdpa_fp64():
    # T = 4 causal tokens at the end of the cache: SDPA with an explicit mask
    c = synth.make_case("t", B=1, T=4, Hq=4, Hkv=1, d_qk=24, d_v=24, seq_lens=[30],
                        page_size=16, seed=11)
    O, LSE = A.attend(c)
    K, V = A.dequant_kv(c, 0, 0)
    L = 30
    mask = torch.zeros(4, L, dtype=torch.bool)
    for t in range(4):
        mask[t, :L - 4 + t + 1] = True
    for h in range(4):
        q = torch.tensor(decode_bf16(c.q[0, :, h]))       # [T, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], torch.tensor(K)[None], torch.tensor(V)[None], attn_mask=mask[None], scale=c.scale)[0]
        assert np.allclose(O[0, :, h], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_closed_form_zero_keys_mean_of_values():
    rng = np.random.default_rng(0)
    V = rng.standard_normal((23, 5))
    O, L = A.attend_rows(rng.standard_normal((2, 4)), np.zeros((23, 4)), V, 0.3, [22, 9])
    assert np.allclose(O[0], V.mean(axis=0), rtol=1e-14, atol=1e-14)
    assert np.allclose(O[1], V[:10].mean(axis=0), rtol=1e-14, atol=1e-14)
    assert np.allclose(L, [math.log(23), math.log(10)], rtol=1e-15)


def test_closed_form_constant_values_and_single_key():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((40, 6)) * 3
    O, _ = A.attend_rows(rng.standard_normal((3, 6)), K, np.full((40, 2), 2.5), 0.9, [39, 39, 0])
    assert np.allclose(O, 2.5, rtol=1e-14)
    q = rng.standard_normal((1, 6))
    O, L = A.attend_rows(q, K[:1], np.array([[7.0, -1.0]]), 0.9, [0])
    assert np.allclose(O, [[7.0, -1.0]]) and np.isclose(L[0], 0.9 * float(q[0] @ K[0]), rtol=1e-14)


def test_golden_two_key():
    g = json.load(open(os.path.join(GOLDEN, "two_key.json")))
    O, L = A.attend_rows(np.array([g["q"]]), np.array(g["k"]), np.array(g["v"]), g["sigma"], [1])
    assert np.allclose(O[0], g["O"], rtol=1e-14, atol=1e-14)
    assert np.isclose(L[0], g["LSE"], rtol=1e-14)


def test_golden_empty_splits_contribute_zero():
    g = json.load(open(os.path.join(GOLDEN, "empty_split.json")))
    m = np.array([float(x) for x in g["m"]])[:, None, None]
    l = np.array(g["l"])[:, None, None]
    o = np.array(g["o"], dtype=np.float64)[:, None, None, :]
    O, L = A.combine(m, l, o, [4], [0, 4])
    assert np.allclose(O[0, 0, 0], g["O"], rtol=1e-15) and np.isclose(L[0, 0, 0], g["LSE"])
    # and the single-split combine is the identity o/l, m + ln l
    O1, L1 = A.combine(m[:1], l[:1], o[:1], [1], [0, 1])
    assert np.allclose(O1, O) and np.allclose(L1, L)


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
def test_one_hot_probe_through_page_permutation(kv):
    # make logical key j* of head hk point along q so that it dominates; the output
    # must then be that token's value: pins page lookup, slot, and head grouping
    c = _case_tiny_paged(7, B=2, Hq=8, Hkv=2, D=16, Ls=(37, 70), kv=kv)
    b, hk, jstar = 1, 1, 41
    page = c.block_table[b][jstar // c.page_size]
    slot = jstar % c.page_size
    h = hk * c.g + 2
    qh = decode_bf16(c.q[b, 0, h])
    if kv == "bf16":
        c.k_cache[page, hk, slot] = synth.to_bf16_codes((qh * 40).astype(np.float32))
    else:
        c.k_cache[page, hk, slot] = synth.to_e4m3_codes((qh * 40 / c.k_scale).astype(np.float32))
    O, _ = A.attend(c)
    _, V = A.dequant_kv(c, b, hk)
    assert np.allclose(O[b, 0, h], V[jstar], atol=1e-6)
    # a query head of the other KV head must not see it
    h2 = 0 * c.g + 2
    assert not np.allclose(O[b, 0, h2], V[jstar], atol=1e-2)


def test_causal_probe_future_key_gets_zero_weight():
    c = synth.make_case("t", B=1, T=3, Hq=2, Hkv=1, d_qk=16, d_v=16, seq_lens=[40],
                        page_size=16, seed=9)
    O0, L0 = A.attend(c)
    # poison the key/value just past token t=0's limit (position 40-3+0+1 = 38):
    j = 38
    page, slot = c.block_table[0][j // 16], j % 16
    c.k_cache[page, 0, slot] = synth.to_bf16_codes(np.full(16, 50.0, dtype=np.float32))
    c.v_cache[page, 0, slot] = synth.to_bf16_codes(np.full(16, 1e4, dtype=np.float32))
    O1, L1 = A.attend(c)
    assert np.array_equal(O0[0, 0], O1[0, 0]) and np.array_equal(L0[0, 0], L1[0, 0])
    assert not np.allclose(O0[0, 1], O1[0, 1])        # token 1 does see position 38


@pytest.mark.parametrize("T,n", [(1, 1), (1, 3), (1, 7), (4, 5), (6, 4)])
def test_split_emulation_equals_unsplit(T, n):
    c = synth.make_case("t", B=3, T=T, Hq=8, Hkv=2, d_qk=16, d_v=12, seq_lens=[19, 100, 6],
                        page_size=16, seed=21 + n)
    if T > 1:
        c.seq_lens[2] = max(int(c.seq_lens[2]), T)
    ns, off, _ = P.make_plan(c.seq_lens, T=T, Hq=8, Hkv=2, requested=n, max_splits=64,
                             num_cus=4, rows_per_wg=16)
    pm, pl, po = A.split_partials(c, ns, off)
    O, L = A.combine(pm, pl, po, ns, off)
    Oref, Lref = A.attend(c)
    assert np.allclose(O, Oref, rtol=1e-12, atol=1e-12)
    assert np.allclose(L, Lref, rtol=1e-12, atol=1e-12)


def test_split_emulation_has_empty_causal_rows():
    # the last split of a short causal sequence holds keys only the later tokens see
    c = synth.make_case("t", B=1, T=6, Hq=2, Hkv=1, d_qk=8, d_v=8, seq_lens=[20],
                        page_size=16, seed=2)
    ns, off, _ = P.make_plan(c.seq_lens, T=6, Hq=2, Hkv=1, requested=2, max_splits=64,
                             num_cus=4, rows_per_wg=16)
    pm, pl, po = A.split_partials(c, ns, off)
    # split 1 covers [16, 20): token t sees j <= 14 + t, so t = 0, 1 see nothing there
    assert np.isneginf(pm[1, 0]).all() and np.isneginf(pm[1, 1]).all()
    assert np.isfinite(pm[1, 2]).all()
    O, L = A.combine(pm, pl, po, ns, off)
    Oref, Lref = A.attend(c)
    assert np.allclose(O, Oref, rtol=1e-12, atol=1e-12)


def test_select_matches_full():
    c = _case_tiny_paged(4, B=2, Hq=8, Hkv=2, D=16, Ls=(37, 70))
    O, L = A.attend(c)
    sel = [(1, 0, 5), (0, 0, 0), (1, 0, 2)]
    Os, Ls = A.attend(c, select=sel)
    for i, (b, t, h) in enumerate(sel):
        assert np.array_equal(Os[i], O[b, t, h]) and Ls[i] == L[b, t, h]

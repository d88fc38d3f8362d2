"""Pins of the oracle planner: the range contract checked by brute force.

The page-borne requirement is that the runtime split count decides the
ranges, so a request of n <= nblk splits yields exactly n non-empty ranges
("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48% Slower", sections "The
actual bug is one missing constructor argument" and "Why passing num_splits
manually does not help").
"""
import numpy as np
import pytest

from oracle import plan as P


def test_ranges_partition_and_are_nonempty():
    for L in list(range(0, 600)) + [4095, 4096, 5900, 32000, 65536, 131072]:
        nblk = -(-L // 16)
        for n in range(1, 65):
            if L > 0 and n > nblk:
                continue
            if L == 0 and n > 1:
                continue
            covered = []
            prev_e = 0
            for i in range(n):
                s, e = P.split_range(L, n, i)
                assert s == prev_e, (L, n, i)
                if L > 0:
                    assert e > s, (L, n, i)          # honoured: no empty split
                assert s % 16 == 0
                covered.extend(range(s, e))
                prev_e = e
            assert prev_e == L
            assert covered == list(range(L))


def test_range_sizes_balanced():
    # sizes differ by at most one granule (brute-force check of the floor formula)
    for L in (260, 5900, 32000, 65536):
        nblk = -(-L // 16)
        for n in (1, 2, 3, 7, 16, 64):
            sizes = [P.split_range(L, n, i)[1] - P.split_range(L, n, i)[0] for i in range(n)]
            full = sizes[:-1]
            if full:
                assert max(full) - min(full) <= 16


def test_request_is_honoured_exactly():
    for L in (17, 260, 5900):
        nblk = -(-L // 16)
        for n in range(1, 65):
            ns, off, info = P.make_plan([L], T=1, Hq=16, Hkv=2, requested=n, max_splits=64,
                                        num_cus=256, rows_per_wg=16)
            assert ns[0] == min(n, nblk)
            assert off.tolist() == [0, ns[0]]
            assert [r[1] & 0xffff for r in info] == list(range(ns[0]))
            assert all(r[3] > r[2] for r in info)


def test_clamps():
    assert P.clamp_request(0, 8, 64) == 1
    assert P.clamp_request(1, 8, 64) == 1
    assert P.clamp_request(16, 8, 64) == 1
    assert P.clamp_request(17, 8, 64) == 2
    assert P.clamp_request(100000, 300, 64) == 64
    assert P.split_range(0, 1, 0) == (0, 0)


def test_auto_plan_never_exceeds_target():
    # the floor keeps sum_b n_b * units <= target workgroups
    import numpy as np
    rng = np.random.default_rng(3)
    for _ in range(200):
        B = int(rng.integers(1, 40))
        lens = rng.integers(0, 200000, size=B).tolist()
        for (T, Hq, Hkv, rpw) in [(1, 32, 8, 16), (6, 128, 1, 64), (1, 16, 2, 16)]:
            ns, off, _ = P.make_plan(lens, T=T, Hq=Hq, Hkv=Hkv, requested=0, max_splits=256,
                                     num_cus=256, rows_per_wg=rpw)
            units = Hkv * -(-(Hq // Hkv) * T // rpw)
            per_cu = P.AUTO_WG_PER_CU_MLA if rpw == 64 else P.AUTO_WG_PER_CU
            over = [n for n, Lb in zip(ns, lens) if n > 1]
            assert sum(over) * units <= per_cu * 256 or not over


def test_auto_plan_targets_two_wg_per_cu():
    # 8 x 32000 tokens, 4 KV heads, g=8 rows -> 32 units per split; 512 target WGs
    ns, off, seq = P.make_plan([32000] * 8, T=1, Hq=32, Hkv=4, requested=0, max_splits=256,
                               num_cus=256, rows_per_wg=16)
    assert ns.tolist() == [16] * 8                # chunk = ceil(8*32000*4/512) = 2000
    # minimum chunk: short sequences get one split
    ns, _, _ = P.make_plan([90, 300, 600], T=1, Hq=8, Hkv=2, requested=0, max_splits=64,
                           num_cus=256, rows_per_wg=16)
    assert ns.tolist() == [1, 3, 6]               # chunk = AUTO_MIN_TOKENS = 96, floor
    # slot_info holds (b, n << 16 | i, start, end)
    ns, off, info = P.make_plan([40, 5000], T=1, Hq=8, Hkv=2, requested=3, max_splits=64,
                                num_cus=256, rows_per_wg=16)
    assert ns.tolist() == [3, 3] and off.tolist() == [0, 3, 6]
    assert [(r[0], r[1] >> 16, r[1] & 0xffff) for r in info] == \
        [(0, 3, 0), (0, 3, 1), (0, 3, 2), (1, 3, 0), (1, 3, 1), (1, 3, 2)]
    assert [tuple(r[2:]) for r in info] == [(0, 16), (16, 32), (32, 40),
                                            (0, 1664), (1664, 3328), (3328, 5000)]


def test_debug_records_brute_force():
    rng = np.random.default_rng(5)
    Ls = [1, 15, 16, 17, 300]
    Pg = 16
    pages = [-(-L // Pg) for L in Ls]
    bt = np.full((len(Ls), max(pages)), 2**31 - 1, dtype=np.int32)
    perm = rng.permutation(sum(pages))
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    ns, off, _ = P.make_plan(Ls, T=1, Hq=4, Hkv=1, requested=4, max_splits=64, num_cus=8,
                             rows_per_wg=16)
    rec = P.debug_records(Ls, bt, Pg, ns, off, Hkv=1, row_blocks=1)
    for b, L in enumerate(Ls):
        for i in range(ns[b]):
            r = rec[off[b] + i, 0, 0]
            s, e = int(r[3]), int(r[4])
            toks = list(range(s, e))
            phys = sorted(set(int(bt[b][j // Pg]) for j in toks))
            x = 0
            for p in phys:
                x ^= p
            assert r[0] == b and r[1] == i and r[5] == len(phys) and r[6] == x
            assert r[7] == sum(phys) % 2**31

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


def _auto(lens, *, T=1, Hq=16, Hkv=2, d=(256, 256), elem=2, cus=256, rpw=16, mx=256):
    return P.make_plan(lens, T=T, Hq=Hq, Hkv=Hkv, requested=0, max_splits=mx, num_cus=cus,
                       rows_per_wg=rpw, d_qk=d[0], d_v=d[1], elem=elem)[0].tolist()


def test_auto_plan_invariants():
    rng = np.random.default_rng(3)
    for _ in range(150):
        B = int(rng.integers(1, 40))
        lens = rng.integers(0, 200000, size=B).tolist()
        for (T, Hq, Hkv, rpw, d, elem) in [(1, 32, 8, 16, (128, 128), 2), (6, 128, 1, 128, (576, 512), 2),
                                           (1, 16, 2, 16, (256, 256), 2), (1, 32, 4, 16, (128, 128), 1)]:
            ns = _auto(lens, T=T, Hq=Hq, Hkv=Hkv, d=d, elem=elem, rpw=rpw)
            tb = (d[0] * 2 if rpw == P.ROWS_PER_WG_MLA else (d[0] + d[1]) * elem)
            c_lat = max(16, int(np.floor(np.sqrt(1.5 * max(lens)))) - 1)
            for n, Lb in zip(ns, lens):
                assert 1 <= n <= max(1, min(256, -(-Lb // 16)))
                if Lb < c_lat:
                    assert n == 1                         # shorter than the latency floor
            if max(lens) * tb < P.AUTO_SPLIT_MIN_BYTES:
                assert ns == [1] * B


def test_auto_plan_worked_examples():
    # Below the byte threshold nothing is split: D=128 bf16 reads tb = 512 B per
    # token, and 383 * 512 = 196096 < 196608 <= 384 * 512.
    assert _auto([383], Hq=8, d=(128, 128)) == [1]
    # L=384 (units 2, overhead 64): c_lat = max(16, isqrt(576)) = 24, W = 768.
    # One round and balanced: c = 24, 16 splits of 1-2 granules -> 64 + 32 =
    # 96, plus the merge: 2 * 16 * 8 rows * 130 * 4 B = 133120 B over 256 units
    # of 512 B tokens -> 2, score 98.  Fewer splits (c = 32): 12 splits of two
    # granules -> 96 + 1 (99840 B) = 97, the lowest.  Half (c = 48): 8 splits
    # of three granules -> 112 + 1.
    assert _auto([384], Hq=8, d=(128, 128)) == [12]
    assert _auto([256], Hq=8, d=(128, 128)) == [1]          # the tiny decode shape
    # Few-KV-head decode at L=5900, D=256 bf16 (tb = 1024, overhead 32 tokens):
    # c_lat = isqrt(8850) = 94 (94^2 = 8836); W = 11800 -> c1 = 94.
    # one round: floor(5900/94) = 62 splits, ranges of 5 or 6 granules -> the
    # longest workgroup costs 96 + 32 = 128, plus the merge of 62 partials of
    # 16 rows x 258 fp32 written and read, 2047488 B over 256 x 1024 -> 8:
    # 136; balanced: 63 splits, also at most 6 granules -> 128 + 8 = 136 (a
    # tie keeps one round); 4/3 (c = 126): 46 splits of up to 9 granules ->
    # 176 + 6; half (c = 188): 31 splits -> 224 + 4.
    assert _auto([5900]) == [62]
    # Eight e4m3 sequences of 32000, Hq=32, Hkv=4, D=128 (tb = 256, overhead
    # 128): units = 4, W = 1024000, c_lat = isqrt(48000) = 219.  One round:
    # c = 4000 -> 8 splits, 256 workgroups of 4000 tokens -> 4128 + merge 33.
    # Balanced: c = 1000 -> 32 splits, 1024 workgroups of ~1000 tokens on 256
    # units -> four each, ~4512 + 130.  4/3 and half: 5 and 4 splits, single
    # workgroups of 6400 and 8000 tokens.  One round wins.
    assert _auto([32000] * 8, Hq=32, Hkv=4, d=(128, 128), elem=1) == [8] * 8
    # MLA decode at L=65536 (T=6, 128 heads -> 768 rows, units = 6 row blocks
    # of 128, tb = 1152; an MLA partial row is 2 x 512 bytes of codes and 16
    # of m, l and two scales): c_lat = isqrt(98304) = 313, W = 393216; one
    # round: c = 1536 -> 42 splits, 252 workgroups of up to 1568 tokens ->
    # 1597 + merge 228 (42 slots x 768 rows x 1040 B written and read, over
    # 256 x 1152 B) = 1825; 4/3: c = 2048 -> 32 splits of 2048 -> 2077 + 174;
    # half: 21 splits -> 3165 + 114; balanced: c = 384 -> 171 splits, 1026
    # workgroups, about four per unit -> 2001 + 927.  One round wins.
    assert _auto([65536], T=6, Hq=128, Hkv=1, d=(576, 512), rpw=128) == [42]
    # The same at L=2048, where the merge decides: c_lat = c = 55.  One round:
    # 37 splits -> 93 + 201 = 294; balanced: 38 splits -> 93 + 206; 4/3, c =
    # 74: 27 splits -> 109 + 147 = 256; half, c = 110: 18 splits of 112 or 128
    # tokens -> 157 + 98 = 255, the lowest.  An e4m3 cache counts the same
    # tb: a token costs the matrix work.
    assert _auto([2048], T=6, Hq=128, Hkv=1, d=(576, 512), rpw=128) == [18]
    assert _auto([2048], T=6, Hq=128, Hkv=1, d=(576, 512), rpw=128, elem=1) == [18]
    # At L=4096 the compact partial row decides between two candidates:
    # c_lat = 78, c = 96.  One round: 42 splits -> 141 + 228 = 369; 4/3, c =
    # 128: 32 splits of 128 tokens -> 157 + 174 (51118080 B) = 331, the
    # lowest; half: 21 splits of 192 -> 237 + 114 = 351; balanced: 53 splits
    # -> 218 + 288.  Priced at the fp32 row of the grouped-query kernels (514
    # x 4 B) the merges would double (4/3: 157 + 343 = 500; half: 237 + 225 =
    # 462) and half would win with 21.
    assert _auto([4096], T=6, Hq=128, Hkv=1, d=(576, 512), rpw=128) == [32]
    # Unequal lengths on 4 units (Hq = Hkv = 1 -> units = 1; D=128 bf16, overhead
    # 64): lens 4096, 3000, 200, 200, W = 7496, c_lat = 78.  One round: c = 1874
    # -> [2, 1, 1, 1]; the 3000-token workgroup alone costs 3064.  Balanced:
    # c = ceil(7496/16) = 469 -> [9, 7, 1, 1], 18 workgroups costing 8648 in
    # total, none above 528, so list scheduling ends by 8648/4 + 528 < 3064,
    # and its merge (16 partials of 130 fp32, 16640 B over 4 x 512) adds 9.
    # 4/3 and half leave every sequence whole: 4160.
    assert _auto([4096, 3000, 200, 200], Hq=1, Hkv=1, d=(128, 128), cus=4) == [9, 7, 1, 1]
    # max_splits caps the count; nblk caps short sequences
    assert _auto([5900], mx=16) == [16]
    assert _auto([0, 0]) == [1, 1]


def test_plan_records():
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

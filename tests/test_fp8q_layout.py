"""Host-side checks of the e4m3-query MLA kernel's sub-tile layout (CPU only).

The kernel stores chunk c (16 bytes) of sub-tile token t at position
c ^ swz8(t), swz8(t) = ((t >> 2) & 1) | ((((t >> 3) ^ (t >> 4)) & 1) << 1),
and fills a 32 x 576-byte sub-tile with 18 wave-level loads (lane j of load i
fills position 64 i + j).  These checks restate those formulas from the
kernel's description and confirm the properties its comments claim: the
fill is a permutation of the sub-tile, every row stays inside its 36
chunks, and under the LDS bank model measured on gfx950 (16-byte reads
served 32 lanes at a time from 128 four-byte banks, transposing 8-byte reads
32 lanes at a time from 64) both operand reads are conflict-free.
"""
import itertools

ROW = 576
CHUNKS = 36


def swz8(t):
    return ((t >> 2) & 1) | ((((t >> 3) ^ (t >> 4)) & 1) << 1)


def test_fill_is_a_permutation_of_the_sub_tile():
    seen = set()
    for i in range(18):
        for j in range(64):
            q = 64 * i + j
            tok, pos = divmod(q, CHUNKS)
            chunk = pos ^ swz8(tok)
            assert 0 <= chunk < CHUNKS
            seen.add((tok, chunk))
            # loads 0-8 hold tokens 0-15, loads 9-17 tokens 16-31 (one page half each)
            assert (tok < 16) == (i < 9)
    assert len(seen) == 32 * CHUNKS


def test_score_operand_reads_are_conflict_free():
    # 16x16x128 step: lane (token n16 + 16 g, qg) reads chunk 8 ks + qg (and 8 ks + 4 + qg)
    for g, ks, second, half in itertools.product(range(2), range(4), range(2), range(2)):
        banks = []
        for qg in (2 * half, 2 * half + 1):           # 32 lanes: qg pair x 16 tokens
            for n16 in range(16):
                t = 16 * g + n16
                c = 8 * ks + 4 * second + qg
                addr = t * ROW + 16 * (c ^ swz8(t))
                banks += [(addr // 4 + w) % 128 for w in range(4)]
        assert len(set(banks)) == 128


def test_transposing_value_reads_are_conflict_free():
    # lane x of group qg reads 8 bytes of token 16 (j >> 2) + 4 qg + (j & 3), j = x >> 1,
    # half x & 1 of chunk c
    for c, half in itertools.product(range(32), range(2)):
        banks = []
        for qg in (2 * half, 2 * half + 1):
            for x in range(16):
                j = x >> 1
                t = 16 * (j >> 2) + 4 * qg + (j & 3)
                addr = t * ROW + 16 * (c ^ swz8(t)) + 8 * (x & 1)
                banks += [(addr // 4 + w) % 64 for w in range(2)]
        assert len(set(banks)) == 64


def test_rope_operand_reads_are_conflict_free():
    # 16x16x32 step of wave half hf: lane (token n16 + 16 g, qg) reads 8 bytes,
    # half qg & 1 of chunk 32 + 2 hf + (qg >> 1) (8-byte reads: the 64-bank model)
    for g, hf, half in itertools.product(range(2), range(2), range(2)):
        banks = []
        for qg in (2 * half, 2 * half + 1):
            for n16 in range(16):
                t = 16 * g + n16
                c = 32 + 2 * hf + (qg >> 1)
                addr = t * ROW + 16 * (c ^ swz8(t)) + 8 * (qg & 1)
                banks += [(addr // 4 + w) % 64 for w in range(2)]
        assert len(set(banks)) == 64, (g, hf, half, len(set(banks)))

"""Host-side checks of the MLA partial kernel's LDS layouts (CPU only).

The formulas below restate the kernel's description of its tiles:

* bf16 tile (32 tokens x 1152 bytes): 16-byte chunk c of token t at position
  c ^ swz_bf16(t), swz_bf16(t) = ((t >> 2) ^ ((t & 2) << 1)) & 7;
* e4m3 tile (32 tokens x 576 bytes): chunk c of token t at position
  4 (c >> 2) + ((c & 3) ^ swz_e4m3(t)), swz_e4m3(t) = ((t >> 3) & 1) << 1 | ((t >> 4) & 1);
* a tile is filled by wave-level loads of 1 KiB, lane j of load i filling
  position 64 i + j (token (64 i + j) // chunks, position (64 i + j) % chunks);
* a wave's 32 query rows are staged in a bf16 tile's layout by 36 such loads.

The checks confirm what the kernel's comments claim: each fill is a
permutation of its tile, a tile's first half of loads holds tokens 0-15 (one
page), and under the LDS bank model measured on gfx950 (16-byte reads served
32 lanes at a time from 128 four-byte banks, transposing 8-byte reads 32 lanes
at a time from 64) every operand read is conflict-free.
"""
import itertools

BF16_ROW, BF16_CHUNKS = 1152, 72
E4M3_ROW, E4M3_CHUNKS = 576, 36


def swz_bf16(t):
    return ((t >> 2) ^ ((t & 2) << 1)) & 7


def swz_e4m3(t):
    return (((t >> 3) & 1) << 1) | ((t >> 4) & 1)


def pos_bf16(t, c):
    return c ^ swz_bf16(t)


def pos_e4m3(t, c):
    return 4 * (c >> 2) + ((c & 3) ^ swz_e4m3(t))


def addr_bf16(t, c):
    return t * BF16_ROW + 16 * pos_bf16(t, c)


def addr_e4m3(t, c):
    return t * E4M3_ROW + 16 * pos_e4m3(t, c)


def banks16(addrs):
    """Banks a pass of 32 lanes of 16-byte reads touches (128-bank model)."""
    out = []
    for a in addrs:
        out += [(a // 4 + w) % 128 for w in range(4)]
    return out


def banks8(addrs):
    """Banks a pass of 32 lanes of 8-byte reads touches (64-bank model)."""
    out = []
    for a in addrs:
        out += [(a // 4 + w) % 64 for w in range(2)]
    return out


def _fill(chunks, loads, pos):
    seen = set()
    for i in range(loads):
        for j in range(64):
            tok, p = divmod(64 * i + j, chunks)
            # the chunk held at position p (the position map is its own inverse)
            c = next(c for c in range(chunks) if pos(tok, c) == p)
            assert 0 <= c < chunks
            seen.add((tok, c))
            if loads in (18, 36) and chunks * 32 == 64 * loads:
                assert (tok < 16) == (i < loads // 2)
    return seen


def test_tile_fills_are_permutations_with_page_halves():
    assert len(_fill(BF16_CHUNKS, 36, pos_bf16)) == 32 * BF16_CHUNKS
    assert len(_fill(E4M3_CHUNKS, 18, pos_e4m3)) == 32 * E4M3_CHUNKS


def test_position_maps_are_involutions_inside_the_row():
    for t in range(32):
        assert sorted(pos_bf16(t, c) for c in range(BF16_CHUNKS)) == list(range(BF16_CHUNKS))
        assert sorted(pos_e4m3(t, c) for c in range(E4M3_CHUNKS)) == list(range(E4M3_CHUNKS))
        assert all(pos_bf16(t, pos_bf16(t, c)) == c for c in range(BF16_CHUNKS))
        assert all(pos_e4m3(t, pos_e4m3(t, c)) == c for c in range(E4M3_CHUNKS))


def test_bf16_key_and_query_reads_are_conflict_free():
    # a pass is the 32 lanes of one h (lane = r32 + 32 h); kind 0 reads chunk
    # 2 i + h, kind 1 chunks 4 (i >> 1) + 2 h + (i & 1) (query staging too)
    for i, h in itertools.product(range(36), range(2)):
        for c in (2 * i + h, 4 * (i >> 1) + 2 * h + (i & 1)):
            if c < BF16_CHUNKS:
                assert len(set(banks16([addr_bf16(r, c) for r in range(32)]))) == 128, (i, h, c)


def test_e4m3_key_reads_are_conflict_free():
    # bf16 queries: read m takes chunk 2 m + h; e4m3 queries: product p takes
    # chunks 4 p + 2 h + c, c = 0, 1
    for m, h in itertools.product(range(18), range(2)):
        assert len(set(banks16([addr_e4m3(r, 2 * m + h) for r in range(32)]))) == 128
    for p, h, c in itertools.product(range(9), range(2), range(2)):
        assert len(set(banks16([addr_e4m3(r, 4 * p + 2 * h + c) for r in range(32)]))) == 128


def test_bf16_transposing_value_reads_are_conflict_free():
    # read r of 16-token step kb, value block blk: lane (x, g1, h) reads 8
    # bytes of token 16 kb + 8 r + 4 h + x / 4, chunk 4 blk + 2 g1 + (x & 3) / 2,
    # half x & 1; a pass is the 32 lanes of one h
    for kb, r, blk, h in itertools.product(range(2), range(2), range(16), range(2)):
        addrs = []
        for g1, x in itertools.product(range(2), range(16)):
            tv = 16 * kb + 8 * r + 4 * h + x // 4
            c = 4 * blk + 2 * g1 + (x & 3) // 2
            addrs.append(addr_bf16(tv, c) + 8 * (x & 1))
        assert len(set(banks8(addrs))) == 64, (kb, r, blk, h)


def test_e4m3_transposing_value_reads_are_conflict_free():
    # lane x = 2 j + sh of group (g1, h) reads 8 codes of token
    # 16 kb + 8 (j / 4) + 4 h + j % 4, chunk 2 blk + g1, half sh
    for kb, blk, h in itertools.product(range(2), range(16), range(2)):
        addrs = []
        for g1, x in itertools.product(range(2), range(16)):
            j, sh = x >> 1, x & 1
            tv = 16 * kb + 8 * (j // 4) + 4 * h + j % 4
            addrs.append(addr_e4m3(tv, 2 * blk + g1) + 8 * sh)
        assert len(set(banks8(addrs))) == 64, (kb, blk, h)


def test_value_read_offsets_match_the_kernels_closed_forms():
    # the kernel folds the transposing reads' addresses into per-lane offsets
    # vofs plus a constant; recompute both ways for every lane
    for lane, kb, blk in itertools.product(range(64), range(2), range(16)):
        x, g1, h = lane & 15, (lane >> 4) & 1, lane >> 5
        # bf16, read r
        for r in range(2):
            tv = 16 * kb + 8 * r + 4 * h + x // 4
            direct = addr_bf16(tv, 4 * blk + 2 * g1 + (x & 3) // 2) + 8 * (x & 1)
            i = (blk & 1) ^ kb
            vofs = ((4 * h + (x >> 2)) * BF16_ROW + 64 * (i ^ (x >> 3)) +
                    16 * ((2 * g1 + ((x & 3) >> 1)) ^ (2 * r + h)) + 8 * (x & 1))
            folded = 16 * kb * BF16_ROW + 8 * r * BF16_ROW + 128 * (blk >> 1) + vofs
            assert direct == folded, (lane, kb, blk, r)
        # e4m3
        j, sh = x >> 1, x & 1
        tv = 16 * kb + 8 * (j >> 2) + 4 * h + (j & 3)
        direct = addr_e4m3(tv, 2 * blk + g1) + 8 * sh
        vofs = tv * E4M3_ROW + 32 * ((blk & 1) ^ (j >> 2)) + 16 * (g1 ^ kb) + 8 * sh
        assert direct == 64 * (blk >> 1) + vofs, (lane, kb, blk)

"""Split planner and range contract, written independently -- oracle (test only).

The pages fix the behaviour, not the formula:

* the KV range of each sequence is divided into ``num_splits`` ranges that
  are spread over many compute units ("vLLM 0.30.0 FA4 SplitKV Bug: H100
  Decode Can Be 48% Slower", section "What SplitKV is trying to do");
* the count the caller passes at run time must be the one that decides the
  ranges -- the regression read a stored default of one, so every split past
  the first got an empty range (section "The actual bug is one missing
  constructor argument"; section "Why passing num_splits manually does not
  help");
* a good count depends on the machine and on the cost of the merge: eight
  splits won in isolation but lost in the server ("Shipped: 484.5 tok/s on
  one GB300 ...", section "Why 8 splits lost").

The integer contract below is the reading this project fixes (the pages print
none).  The HIP library implements the same contract in its own C++ code; the
two are compared bit for bit.

* Granule G = 16 tokens; nblk(L) = ceil(L / G).
* A request n > 0 is honoured exactly whenever n <= min(max_splits, nblk):
  n_eff = clamp(n, 1, min(max_splits, max(nblk, 1))).
* Auto mode (n == 0): R = AUTO_WG_PER_CU * num_cus target workgroups
  (AUTO_WG_PER_CU_MLA for the MLA kernel, whose workgroup fills a CU),
  units = Hkv * ceil(g*T / rows_per_wg) workgroups per split of a sequence,
  chunk = max(AUTO_MIN_TOKENS, ceil(sum_b L_b * units / R)),
  n_b = clamp(floor(L_b / chunk), 1, min(max_splits, max(nblk_b, 1))) -- floor,
  so the total never exceeds R workgroups (a second partial round of
  workgroups would double the step time).
* Split i of n covers [G*floor(i*nblk/n), min(L, G*floor((i+1)*nblk/n))).
  Because n <= nblk every range holds at least one token, the ranges are
  disjoint and contiguous and their union is [0, L).  L == 0 gives one empty
  range [0, 0).
"""
import numpy as np

# Constants of the contract (the library publishes its own copies; a test
# checks that the two agree).
GRANULE = 16
AUTO_MIN_TOKENS = 96
AUTO_WG_PER_CU = 2
AUTO_WG_PER_CU_MLA = 1
MAX_SPLITS_LIMIT = 256
ROWS_PER_WG_GQA = 16
ROWS_PER_WG_MLA = 64


def _ceil_div(a, b):
    return -(-a // b)


def num_blocks(L: int) -> int:
    return _ceil_div(int(L), GRANULE)


def split_range(L: int, n: int, i: int):
    """Token range [s, e) of split i out of n for a sequence of L tokens."""
    nblk = num_blocks(L)
    s = GRANULE * ((i * nblk) // n)
    e = min(int(L), GRANULE * (((i + 1) * nblk) // n))
    return s, e


def clamp_request(L: int, n: int, max_splits: int) -> int:
    cap = min(max_splits, max(num_blocks(L), 1))
    return max(1, min(int(n), cap))


def make_plan(seq_lens, *, T: int, Hq: int, Hkv: int, requested: int, max_splits: int,
              num_cus: int, rows_per_wg: int):
    """Return (num_splits[B], slot_offset[B+1], slot_info[S, 4]) as int32 arrays.

    ``slot_info[s]`` is the work record of slot ``s`` (split ``i`` of sequence
    ``b``): ``(b, (n_b << 16) | i, start, end)`` with [start, end) its range.
    """
    L = [int(x) for x in seq_lens]
    B = len(L)
    if requested > 0:
        ns = [clamp_request(Lb, requested, max_splits) for Lb in L]
    else:
        g = Hq // Hkv
        units = Hkv * _ceil_div(g * T, rows_per_wg)
        work = sum(L) * units
        per_cu = AUTO_WG_PER_CU_MLA if rows_per_wg == ROWS_PER_WG_MLA else AUTO_WG_PER_CU
        target = per_cu * num_cus
        chunk = max(AUTO_MIN_TOKENS, _ceil_div(work, target))
        ns = [clamp_request(Lb, Lb // chunk, max_splits) for Lb in L]
    off = [0]
    for n in ns:
        off.append(off[-1] + n)
    info = []
    for b, n in enumerate(ns):
        for i in range(n):
            s, e = split_range(L[b], n, i)
            info.append((b, (n << 16) | i, s, e))
    return (np.array(ns, dtype=np.int32), np.array(off, dtype=np.int32),
            np.array(info, dtype=np.int32).reshape(-1, 4))


def debug_records(seq_lens, block_table, page_size, num_splits, slot_offset, Hkv, row_blocks):
    """Integer record each partial workgroup exports, as the oracle expects it.

    Shape [S, Hkv, row_blocks, 8]: (b, i, hk, s, e, groups, xor_phys, sum_phys)
    where the last three run over the 16-token groups of [s, e): ``groups`` is
    their count, ``xor_phys`` the XOR of the physical page each group reads
    (block_table[b][16*k // P]) and ``sum_phys`` their sum modulo 2^31.
    """
    S = int(slot_offset[-1])
    rec = np.zeros((S, Hkv, row_blocks, 8), dtype=np.int64)
    for b in range(len(seq_lens)):
        Lb = int(seq_lens[b])
        n = int(num_splits[b])
        for i in range(n):
            s, e = split_range(Lb, n, i)
            groups = 0
            x = 0
            acc = 0
            for k in range(s // GRANULE, _ceil_div(e, GRANULE)):
                phys = int(block_table[b][(k * GRANULE) // page_size])
                groups += 1
                x ^= phys
                acc = (acc + phys) % (2**31)
            slot = int(slot_offset[b]) + i
            for hk in range(Hkv):
                for rb in range(row_blocks):
                    rec[slot, hk, rb] = (b, i, hk, s, e, groups, x, acc)
    return rec.astype(np.int32)

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
* Auto mode (n == 0) weighs more splits against the merge they add and the
  start-up latency of every extra workgroup.  Per token a workgroup streams
  tb = (d_qk + d_v) * elem bytes; MLA counts tb = d_qk * 2 whatever the cache
  dtype (V is part of the same row, and its cost per token is the matrix
  work on bf16 operands, the same for an e4m3 cache); a split of a sequence is
  units = Hkv * ceil(g*T / rows_per_wg)
  workgroups; cap_b = min(max_splits, max(nblk_b, 1)); L_max = max_b L_b.
  - If L_max * tb < AUTO_SPLIT_MIN_BYTES, every n_b = 1 (nothing to merge).
  - Latency floor c_lat = max(G, isqrt(L_max * AUTO_LAT_NUM // AUTO_LAT_DEN))
    tokens per split; W = units * sum_b L_b.
  - Candidate "one round": c1 = max(c_lat, ceil(W / num_cus)),
    n_b = clamp(floor(L_b / c1), 1, cap_b).
  - Candidate "balanced": c = max(c_lat, ceil(W / (AUTO_BALANCE * num_cus))),
    n_b = clamp(ceil(L_b / c), 1, cap_b).
  - Candidates "fewer splits": one round with c = ceil(4 * c1 / 3) and with
    c = 2 * c1 (floor as in one round).
  - Each candidate is scored by greedy list scheduling plus its merge: its
    workgroups, in launch order (slots in order, the units of a slot one
    after another), each go to whichever of num_cus compute units is free
    first, costing ceil(AUTO_WG_OVERHEAD_BYTES / tb) + (end - start) tokens;
    to the latest finish is added ceil(Pb / (num_cus * tb)) tokens, Pb =
    2 * sum over sequences with n_b > 1 of n_b * T * Hq * row_bytes, the
    partials written and read back by the merge, spread over every compute
    unit; row_bytes = (d_v + 2) * 4 (fp32 m, l, o), or 2 * d_v + 16 for MLA
    (int16 codes of o; m, l and two scales in fp32).  The lowest score wins; on a tie the earlier candidate in
    the order one round, balanced, 4/3, 2.
* Split i of n covers [G*floor(i*nblk/n), min(L, G*floor((i+1)*nblk/n))).
  Because n <= nblk every range holds at least one token, the ranges are
  disjoint and contiguous and their union is [0, L).  L == 0 gives one empty
  range [0, 0).
"""
import heapq
import math

import numpy as np

# Constants of the contract (the library publishes its own copies; a test
# checks that the two agree).
GRANULE = 16
AUTO_SPLIT_MIN_BYTES = 196608
AUTO_LAT_NUM = 3
AUTO_LAT_DEN = 2
AUTO_BALANCE = 4
AUTO_WG_OVERHEAD_BYTES = 32768
MAX_SPLITS_LIMIT = 256
ROWS_PER_WG_GQA = 16
ROWS_PER_WG_MLA = 128


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


def _latest_finish(L, ns, units, num_cus, overhead):
    """Greedy list scheduling of the plan's workgroups (in launch order) on num_cus units."""
    free = [0] * num_cus
    latest = 0
    for Lb, n in zip(L, ns):
        for i in range(n):
            s, e = split_range(Lb, n, i)
            for _ in range(units):
                t = heapq.heappop(free) + overhead + (e - s)
                latest = max(latest, t)
                heapq.heappush(free, t)
    return latest


def _merge_tokens(ns, T, Hq, d_v, num_cus, tb, mla):
    """The partials a plan writes and the merge reads back, in tokens of
    streaming spread over every compute unit (single-split sequences have none)."""
    row_bytes = 2 * d_v + 16 if mla else (d_v + 2) * 4
    pb = 2 * sum(n for n in ns if n > 1) * T * Hq * row_bytes
    return _ceil_div(pb, num_cus * tb)


def _auto_counts(L, *, T, Hq, Hkv, max_splits, num_cus, rows_per_wg, d_qk, d_v, elem):
    mla = rows_per_wg == ROWS_PER_WG_MLA
    tb = d_qk * 2 if mla else (d_qk + d_v) * elem
    units = Hkv * _ceil_div((Hq // Hkv) * T, rows_per_wg)
    lmax = max(L)
    if lmax * tb < AUTO_SPLIT_MIN_BYTES:
        return [1] * len(L)
    c_lat = max(GRANULE, math.isqrt(lmax * AUTO_LAT_NUM // AUTO_LAT_DEN))
    W = units * sum(L)
    c1 = max(c_lat, _ceil_div(W, num_cus))
    cb = max(c_lat, _ceil_div(W, AUTO_BALANCE * num_cus))
    one = [clamp_request(Lb, Lb // c1, max_splits) for Lb in L]
    bal = [clamp_request(Lb, _ceil_div(Lb, cb), max_splits) for Lb in L]
    c43 = _ceil_div(4 * c1, 3)
    few = [clamp_request(Lb, Lb // c43, max_splits) for Lb in L]
    half = [clamp_request(Lb, Lb // (2 * c1), max_splits) for Lb in L]
    ov = _ceil_div(AUTO_WG_OVERHEAD_BYTES, tb)
    best, best_score = None, None
    for ns in (one, bal, few, half):
        score = _latest_finish(L, ns, units, num_cus, ov) + _merge_tokens(ns, T, Hq, d_v, num_cus, tb, mla)
        if best_score is None or score < best_score:
            best, best_score = ns, score
    return best


def make_plan(seq_lens, *, T: int, Hq: int, Hkv: int, requested: int, max_splits: int,
              num_cus: int, rows_per_wg: int, d_qk: int = 0, d_v: int = 0, elem: int = 2):
    """Return (num_splits[B], slot_offset[B+1], slot_info[S, 4]) as int32 arrays.

    ``slot_info[s]`` is the work record of slot ``s`` (split ``i`` of sequence
    ``b``): ``(b, (n_b << 16) | i, start, end)`` with [start, end) its range.
    Auto mode (``requested == 0``) needs the head dimensions and the KV element
    size in bytes (``elem``: 2 for bf16, 1 for e4m3).
    """
    L = [int(x) for x in seq_lens]
    if requested > 0:
        ns = [clamp_request(Lb, requested, max_splits) for Lb in L]
    else:
        if d_qk < 1 or d_v < 1:
            raise ValueError("auto mode needs d_qk and d_v")
        ns = _auto_counts(L, T=T, Hq=Hq, Hkv=Hkv, max_splits=max_splits, num_cus=num_cus,
                          rows_per_wg=rows_per_wg, d_qk=d_qk, d_v=d_v, elem=elem)
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

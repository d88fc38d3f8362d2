"""Plain fp64 softmax decode attention over a paged cache -- oracle (test only).

Definitions (the pages give the method, this file writes out the result it
must reach):

* Dequantise: logical token j of sequence b lives at page
  ``block_table[b][j // P]``, slot ``j % P``; its key and value are the decoded
  codes times the per-tensor scale (``k_scale``, ``v_scale``; both 1 for
  bf16).  For MLA a single latent row of width d_qk serves as the key and its
  first d_v columns as the value ("Shipped: 484.5 tok/s on one GB300 ...",
  table "What shipped": split-KV MLA decode).
* Head grouping: query head h reads KV head floor(h / g), g = Hq / Hkv (the
  grouped-query shape of "vLLM 0.30.0 FA4 SplitKV Bug ...", section "What
  SplitKV is trying to do"; consecutive grouping is this project's reading).
* Positions: query token t of a sequence with L cached tokens (its own T
  tokens included) sits at position L - T + t and sees keys j <= L - T + t.
  For T = 1 that is every cached key; for the six speculative tokens of the
  MLA workload it is causal within the six.
* Scores s_j = sigma * q . k_j; m = max_j s_j; w_j = exp(s_j - m);
  l = sum_j w_j; O = sum_j w_j v_j / l; LSE = m + ln l.  A row that sees no
  key gives O = 0 and LSE = -inf.

The split-KV method reaches exactly this result up to rounding order: each
split computes a partial (m_i, l_i, o_i) over its own range and a combine
merges them, with empty splits contributing zero weight ("vLLM 0.30.0 FA4
SplitKV Bug ...", sections "What SplitKV is trying to do" and "Why the result
is still correct").  ``split_partials`` and ``combine`` emulate that in fp64;
the merge is the standard log-sum-exp rescaling (the pages say "combine ...
correctly" without a formula): M = max_i m_i, w_i = exp(m_i - M) (zero for an
empty split), O = sum_i w_i o_i / sum_i w_i l_i, LSE = M + ln(sum_i w_i l_i).
"""
import numpy as np

from .append import quantise_bf16
from .codes import decode_bf16, decode_e4m3
from .plan import split_range


def _decode(codes, kv_dtype):
    return decode_bf16(codes) if kv_dtype == "bf16" else decode_e4m3(codes)


def dequant_kv(case, b: int, hk: int, upto: int = None):
    """Gather and decode keys and values of sequence b, KV head hk, tokens [0, upto).

    Returns (K [n, d_qk], V [n, d_v]) in fp64, in logical token order.
    """
    L = int(case.seq_lens[b]) if upto is None else int(upto)
    P = case.page_size
    j = np.arange(L)
    pages = case.block_table[b][j // P].astype(np.int64)
    slots = j % P
    if case.mla:
        rows = case.k_cache[pages, 0, slots, :]
        K = _decode(rows, case.kv_dtype) * case.k_scale
        V = _decode(rows[:, :case.d_v], case.kv_dtype) * case.v_scale
    else:
        K = _decode(case.k_cache[pages, hk, slots, :], case.kv_dtype) * case.k_scale
        V = _decode(case.v_cache[pages, hk, slots, :], case.kv_dtype) * case.v_scale
    return K, V


def dequant_q(case, b: int, t: int, h: int) -> np.ndarray:
    """Query row (b, t, h) as the kernel must read it, in fp64.

    bf16 queries: the decoded codes.  e4m3 queries (case.q_scale set): each
    value is quantised to the e4m3 code of q / q_scale and read back as code
    x q_scale, the same per-tensor encoding as an FP8 cache ("Xqa decode
    kernels", timeline: FP8-Q, used only where the cache is FP8).
    """
    codes = case.q[b, t, h]
    qs = getattr(case, "q_scale", None)
    if qs is None:
        return decode_bf16(codes)
    return decode_e4m3(quantise_bf16(codes, qs)) * float(qs)


def attend_rows(q, K, V, sigma, limits):
    """Softmax attention of query rows q [R, d] over keys K [n, d] / values V [n, dv].

    Row r sees keys j <= limits[r].  Returns (O [R, dv], LSE [R]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    R = q.shape[0]
    dv = V.shape[1]
    O = np.zeros((R, dv))
    LSE = np.full(R, -np.inf)
    if K.shape[0] == 0:
        return O, LSE
    s = float(sigma) * (q @ K.T)                       # [R, n]
    j = np.arange(K.shape[0])
    visible = j[None, :] <= np.asarray(limits)[:, None]
    s = np.where(visible, s, -np.inf)
    for r in range(R):
        if not visible[r].any():
            continue
        m = np.max(s[r])
        w = np.exp(s[r] - m)
        l = np.sum(w)
        O[r] = (w @ V) / l
        LSE[r] = m + np.log(l)
    return O, LSE


def _rows_of_group(case, hk):
    """Query rows (t, h) that read KV head hk, in (t, h) order."""
    g = case.g
    return [(t, h) for t in range(case.T) for h in range(hk * g, (hk + 1) * g)]


def attend(case, select=None):
    """Exact attention output.

    Without ``select`` returns (O [B, T, Hq, d_v], LSE [B, T, Hq]).  With
    ``select`` (a list of (b, t, h)) returns (O [len, d_v], LSE [len]) for
    just those rows.
    """
    B, T = case.B, case.T
    g = case.g
    if select is None:
        want = {(b, hk): _rows_of_group(case, hk) for b in range(B) for hk in range(case.Hkv)}
        O = np.zeros((B, T, case.Hq, case.d_v))
        LSE = np.full((B, T, case.Hq), -np.inf)
    else:
        want = {}
        for (b, t, h) in select:
            want.setdefault((b, h // g), []).append((t, h))
        outO = np.zeros((len(select), case.d_v))
        outL = np.full(len(select), -np.inf)
        index = {tuple(x): i for i, x in enumerate(select)}
    for (b, hk), rows in want.items():
        L = int(case.seq_lens[b])
        K, V = dequant_kv(case, b, hk)
        qhat = np.stack([dequant_q(case, b, t, h) for (t, h) in rows])
        limits = [L - T + t for (t, h) in rows]
        o, lse = attend_rows(qhat, K, V, case.scale, limits)
        for r, (t, h) in enumerate(rows):
            if select is None:
                O[b, t, h] = o[r]
                LSE[b, t, h] = lse[r]
            else:
                outO[index[(b, t, h)]] = o[r]
                outL[index[(b, t, h)]] = lse[r]
    if select is None:
        return O, LSE
    return outO, outL


def _partial_rows(q, K, V, sigma, lo, hi, limits):
    """Unnormalised partial (m, l, o) of rows q over key range [lo, hi)."""
    R = q.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, V.shape[1]))
    if hi <= lo:
        return m, l, o
    s = float(sigma) * (q @ K[lo:hi].T)
    j = np.arange(lo, hi)
    for r in range(R):
        vis = j <= limits[r]
        if not vis.any():
            continue
        mr = np.max(s[r][vis])
        w = np.where(vis, np.exp(np.where(vis, s[r], mr) - mr), 0.0)
        m[r] = mr
        l[r] = np.sum(w)
        o[r] = w @ V[lo:hi]
    return m, l, o


def split_partials(case, num_splits, slot_offset):
    """fp64 partials of every split: (part_m [S,T,Hq], part_l [S,T,Hq], part_o [S,T,Hq,d_v]).

    m is in natural-log units (max of sigma*q.k over the split's visible keys),
    l = sum exp(s - m), o = sum exp(s - m) * v (not normalised).  A row with no
    visible key in the split gives (-inf, 0, 0).
    """
    S = int(slot_offset[-1])
    T, Hq = case.T, case.Hq
    pm = np.full((S, T, Hq), -np.inf)
    pl = np.zeros((S, T, Hq))
    po = np.zeros((S, T, Hq, case.d_v))
    for b in range(case.B):
        L = int(case.seq_lens[b])
        n = int(num_splits[b])
        for hk in range(case.Hkv):
            rows = _rows_of_group(case, hk)
            K, V = dequant_kv(case, b, hk)
            qhat = np.stack([dequant_q(case, b, t, h) for (t, h) in rows])
            limits = [L - T + t for (t, h) in rows]
            for i in range(n):
                s, e = split_range(L, n, i)
                m, l, o = _partial_rows(qhat, K, V, case.scale, s, e, limits)
                slot = int(slot_offset[b]) + i
                for r, (t, h) in enumerate(rows):
                    pm[slot, t, h] = m[r]
                    pl[slot, t, h] = l[r]
                    po[slot, t, h] = o[r]
    return pm, pl, po


def combine(part_m, part_l, part_o, num_splits, slot_offset):
    """Log-sum-exp merge of the partials of each sequence -> (O [B,T,Hq,d_v], LSE [B,T,Hq])."""
    B = len(num_splits)
    _, T, Hq = part_m.shape
    dv = part_o.shape[-1]
    O = np.zeros((B, T, Hq, dv))
    LSE = np.full((B, T, Hq), -np.inf)
    for b in range(B):
        sl = slice(int(slot_offset[b]), int(slot_offset[b]) + int(num_splits[b]))
        m = part_m[sl]                               # [n, T, Hq]
        l = part_l[sl]
        o = part_o[sl]
        M = np.max(m, axis=0)                        # [T, Hq]
        finite = np.isfinite(M)
        Msafe = np.where(finite, M, 0.0)
        w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - Msafe), 0.0)
        lam = np.sum(w * l, axis=0)
        num = np.sum(w[..., None] * o, axis=0)
        ok = finite & (lam > 0)
        O[b] = np.where(ok[..., None], num / np.where(ok, lam, 1.0)[..., None], 0.0)
        LSE[b] = np.where(ok, Msafe + np.log(np.where(ok, lam, 1.0)), -np.inf)
    return O, LSE

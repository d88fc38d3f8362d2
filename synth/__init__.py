"""Seeded synthetic decode-attention workloads.

This module only draws inputs: random queries, a paged KV cache stored as raw
bf16 / e4m3 codes, block tables and sequence lengths.  It holds none of the
attention arithmetic (no dequantisation, no softmax, no split planning), so
both the HIP path and the fp64 oracle can consume the same arrays without
sharing any of the method's code.

The shapes follow the workloads the split-KV pages discuss:

* few KV heads with a long KV history in single-token decode ("vLLM 0.30.0
  FA4 SplitKV Bug: H100 Decode Can Be 48% Slower", sections "What SplitKV is
  trying to do" and "Gemma 4 exposes the failure clearly");
* MLA decode of one request at six speculative tokens ("Shipped: 484.5 tok/s
  on one GB300 ...", table "What shipped");
* bf16 queries over an FP8 KV cache in a paged, HND-layout cache ("Xqa
  decode kernels", sections "Purpose" and "Test Plan").

Cache layout (logical, "HND"): ``cache[page][kv_head][slot][d]``.  A sequence
``b`` owns logical token ``j`` at ``cache[block_table[b][j // P]][hk][j % P]``.

Poison conventions, so that a read of memory the method must not touch shows
up in the output:

* slots at or past ``L_b`` in the last page of a sequence hold NaN codes;
* pages that no block table references hold NaN codes;
* block-table entries past ``ceil(L_b / P)`` hold ``INT32_MAX``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

INT32_MAX = 2**31 - 1
BF16_NAN = 0x7FC0        # quiet NaN in bfloat16
E4M3_NAN = 0x7F          # NaN in the OCP e4m3fn encoding (no infinities)
E4M3_MAX = 448.0

KV_BF16 = "bf16"
KV_E4M3 = "e4m3"


@dataclasses.dataclass
class Case:
    """One decode-attention problem, as raw codes plus metadata."""
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    page_size: int
    kv_dtype: str                 # "bf16" or "e4m3"
    mla: bool                     # one latent cache, V = K[..., :d_v]
    causal: bool
    scale: float                  # softmax scale sigma, an fp32 value
    k_scale: float                # per-tensor dequant scale (1.0 for bf16)
    v_scale: float
    out_fp32: bool                # output dtype: fp32 if True, else bf16
    seq_lens: np.ndarray          # [B] int32
    block_table: np.ndarray       # [B, max_pages] int32
    q: np.ndarray                 # [B, T, Hq, d_qk] uint16 (bf16 codes)
    k_cache: np.ndarray           # [num_pages, Hkv, P, d_qk] uint16 or uint8 codes
    v_cache: Optional[np.ndarray]  # [num_pages, Hkv, P, d_v] codes, None for MLA
    seed: int
    q_scale: Optional[float] = None  # e4m3 queries: per-tensor scale (None: bf16 queries)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode step must read (each cached token once)."""
        tok = int(np.sum(self.seq_lens.astype(np.int64)))
        elem = 1 if self.kv_dtype == KV_E4M3 else 2
        if self.mla:
            return tok * self.d_qk * elem
        return tok * self.Hkv * (self.d_qk + self.d_v) * elem


# --------------------------------------------------------------------------
# rounding of fp32 draws to storage codes (input preparation only)
# --------------------------------------------------------------------------

def _torch():
    import torch  # local import: the generators are usable without a GPU
    return torch


def to_bf16_codes(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even) and return raw codes."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Clamp to +-448 and round to OCP e4m3fn (RNE); return raw codes.

    torch's CPU conversion does not saturate (500 becomes NaN), so the clamp
    comes first.
    """
    torch = _torch()
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


# --------------------------------------------------------------------------
# page pools and block tables
# --------------------------------------------------------------------------

def _page_pool(rng, seq_lens, page_size, spare_frac=0.03, contiguous=False):
    """Assign physical pages to sequences.

    Returns (block_table, num_pages).  With ``contiguous`` every sequence owns
    consecutive pages in order; otherwise the pool is a seeded permutation with
    a few spare pages that no sequence references.
    """
    pages_per = [max(1, -(-int(L) // page_size)) for L in seq_lens]
    used = sum(pages_per)
    spare = 0 if contiguous else max(1, int(math.ceil(used * spare_frac)))
    num_pages = used + spare
    perm = np.arange(num_pages) if contiguous else rng.permutation(num_pages)
    max_pages = max(pages_per)
    bt = np.full((len(seq_lens), max_pages), INT32_MAX, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, num_pages


def _fill_cache(rng, num_pages, H, P, D, std, dtype, bt, seq_lens, scale_out, chunk_pages=4096):
    """Draw a paged cache; page tails and unreferenced pages hold NaN codes."""
    if dtype == KV_BF16:
        cache = np.empty((num_pages, H, P, D), dtype=np.uint16)
    else:
        cache = np.empty((num_pages, H, P, D), dtype=np.uint8)
    amax = 0.0
    draws = []
    # first pass: draw in chunks (fp32), remember amax for the FP8 scale
    for p0 in range(0, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        x = rng.standard_normal((p1 - p0, H, P, D), dtype=np.float32) * np.float32(std)
        if dtype == KV_BF16:
            cache[p0:p1] = to_bf16_codes(x)
        else:
            amax = max(amax, float(np.max(np.abs(x))))
            draws.append((p0, p1, x))
    if dtype == KV_E4M3:
        s = scale_out if scale_out is not None else amax / E4M3_MAX
        inv = np.float32(1.0) / np.float32(s)
        for p0, p1, x in draws:
            cache[p0:p1] = to_e4m3_codes(x * inv)
        scale = float(np.float32(s))
    else:
        scale = 1.0
    nan = BF16_NAN if dtype == KV_BF16 else E4M3_NAN
    referenced = np.zeros(num_pages, dtype=bool)
    for b, L in enumerate(seq_lens):
        n = max(1, -(-int(L) // P))
        pages = bt[b, :n]
        referenced[pages] = True
        tail = int(L) - (n - 1) * P          # valid slots in the last page
        cache[pages[-1], :, tail:, :] = nan
    cache[~referenced] = nan
    return cache, scale


# --------------------------------------------------------------------------
# the workloads
# --------------------------------------------------------------------------

def log_uniform_lengths(rng, B, lo=1, hi=131072, forced=(1, 2, 15, 16, 17, 255, 131072)):
    """Ragged lengths: floor(exp(u)), u ~ U[ln lo, ln hi], with forced edge entries first."""
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    L = np.floor(np.exp(u)).astype(np.int64)
    L = np.clip(L, lo, hi)
    for i, v in enumerate(forced[:B]):
        L[i] = v
    return L.astype(np.int32)


def make_case(name: str, *, B: int, T: int, Hq: int, Hkv: int, d_qk: int, d_v: int,
              seq_lens, page_size: int, kv_dtype: str = KV_BF16, mla: bool = False,
              std: float = 1.0, q_std: Optional[float] = None, scale: Optional[float] = None,
              out_fp32: bool = False, seed: int = 0, contiguous: bool = False,
              fp8_scale: Optional[float] = None, fp8_queries: bool = False) -> Case:
    """Generic generator; every workload below is one call of it.

    fp8_queries: the caller asks for e4m3 queries with the per-tensor scale
    amax|q| / 448 (the recipe of the e4m3 caches); q itself stays bf16."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    scale = float(np.float32(scale))
    q_std = std if q_std is None else q_std
    bt, num_pages = _page_pool(rng, seq_lens, page_size, contiguous=contiguous)
    qx = rng.standard_normal((B, T, Hq, d_qk), dtype=np.float32) * np.float32(q_std)
    q = to_bf16_codes(qx)
    if mla:
        k_cache, k_scale = _fill_cache(rng, num_pages, 1, page_size, d_qk, std, kv_dtype, bt,
                                       seq_lens, fp8_scale)
        v_cache, v_scale = None, k_scale
    else:
        k_cache, k_scale = _fill_cache(rng, num_pages, Hkv, page_size, d_qk, std, kv_dtype, bt,
                                       seq_lens, fp8_scale)
        v_cache, v_scale = _fill_cache(rng, num_pages, Hkv, page_size, d_v, std, kv_dtype, bt,
                                       seq_lens, fp8_scale)
    q_scale = None
    if fp8_queries:
        qv = (q.astype(np.uint32) << 16).view(np.float32)
        q_scale = float(np.float32(float(np.max(np.abs(qv))) / E4M3_MAX))
    return Case(name=name, B=B, T=T, Hq=Hq, Hkv=Hkv, d_qk=d_qk, d_v=d_v, page_size=page_size,
                kv_dtype=kv_dtype, mla=mla, causal=T > 1, scale=scale, k_scale=k_scale,
                v_scale=v_scale, out_fp32=out_fp32, seq_lens=seq_lens, block_table=bt, q=q,
                k_cache=k_cache, v_cache=v_cache, seed=seed, q_scale=q_scale)


def tiny_gqa(L: int = 256, seed: int = 1001) -> Case:
    """Tiny GQA decode: B=1, T=1, Hq=8, Hkv=2, D=128, contiguous bf16, fp32 output."""
    P = max(16, -(-L // 16) * 16)          # one page holds the whole sequence
    return make_case("tiny-gqa", B=1, T=1, Hq=8, Hkv=2, d_qk=128, d_v=128, seq_lens=[L],
                     page_size=P, out_fp32=True, seed=seed, contiguous=True)


def few_kv_long(L: int = 5900, seed: int = 1002) -> Case:
    """Few-KV-head long-context decode: B=1, T=1, Hq=16, Hkv=2, D=256, page 16, bf16."""
    return make_case("few-kv-long", B=1, T=1, Hq=16, Hkv=2, d_qk=256, d_v=256, seq_lens=[L],
                     page_size=16, seed=seed)


def fp8_batched(B: int = 8, L: int = 32000, seed: int = 1003, fp8_scale=None) -> Case:
    """Batched GQA with an e4m3 KV cache: Hq=32, Hkv=4, D=128, page 16, bf16 queries."""
    return make_case("fp8-batched", B=B, T=1, Hq=32, Hkv=4, d_qk=128, d_v=128,
                     seq_lens=[L] * B, page_size=16, kv_dtype=KV_E4M3, seed=seed,
                     fp8_scale=fp8_scale)


def mla_decode(L: int = 2048, seed: int = 1004, T: int = 6, Hq: int = 128,
               kv_dtype: str = KV_BF16, fp8_queries: bool = False) -> Case:
    """MLA decode: 6 causal query tokens, 128 heads, one 576-wide latent head (V = first 512).

    kv_dtype e4m3 stores the latent cache as FP8 codes with one per-tensor
    scale (keys and values share it, being the same rows); fp8_queries (e4m3
    cache only) adds a query scale for e4m3 queries."""
    name = "mla" if kv_dtype == KV_BF16 else ("mla-fp8q" if fp8_queries else "mla-fp8")
    return make_case(name, B=1, T=T, Hq=Hq, Hkv=1, d_qk=576, d_v=512, seq_lens=[L], page_size=64,
                     mla=True, std=0.5, seed=seed, kv_dtype=kv_dtype, fp8_queries=fp8_queries)


def ragged(B: int = 32, seed: int = 1005, hi: int = 131072, seq_lens=None) -> Case:
    """Ragged batch: Hq=32, Hkv=8, D=128, bf16, log-uniform lengths in [1, hi], page 16."""
    rng = np.random.default_rng(seed + 7919)
    if seq_lens is None:
        forced = tuple(min(v, hi) for v in (1, 2, 15, 16, 17, 255, 131072))
        seq_lens = log_uniform_lengths(rng, B, hi=hi, forced=forced)
    return make_case("ragged", B=B, T=1, Hq=32, Hkv=8, d_qk=128, d_v=128, seq_lens=seq_lens,
                     page_size=16, seed=seed)


def ramp_keys(case: Case, steps, d0: int = 0, d1: Optional[int] = None) -> Case:
    """Scale key features [d0, d1) of later tokens, in place.

    ``steps`` is a list of (first_token, factor): logical token j of every
    sequence gets the factor of the last step with first_token <= j (1 before
    the first step).  Scaled values are re-rounded to bf16.  Scores then grow
    along the sequence, so a running softmax maximum jumps inside a split;
    with [d0, d1) inside the rope features of an MLA cache, the values (its
    first d_v features) stay as drawn.  An e4m3 cache keeps its scale: the
    scaled codes are re-rounded to e4m3 (clamped to +-448), so the case must
    have been drawn with a scale that leaves room for the factors.
    """
    d1 = case.d_qk if d1 is None else d1
    P = case.page_size
    steps = sorted(steps)
    for b, L in enumerate(case.seq_lens):
        for j in range(int(L)):
            f = 1.0
            for j0, fac in steps:
                if j >= j0:
                    f = fac
            if f == 1.0:
                continue
            page = case.block_table[b, j // P]
            codes = case.k_cache[page, :, j % P, d0:d1]
            if case.kv_dtype == KV_BF16:
                vals = (codes.astype(np.uint32) << 16).view(np.float32) * np.float32(f)
                case.k_cache[page, :, j % P, d0:d1] = to_bf16_codes(vals)
            else:
                torch = _torch()
                vals = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy()
                case.k_cache[page, :, j % P, d0:d1] = to_e4m3_codes(vals * np.float32(f))
    return case


# --------------------------------------------------------------------------
# bf16 code helpers for the GPU side's upload (bit views only, no rounding)
# --------------------------------------------------------------------------

def random_queries(rng, shape, std=1.0) -> np.ndarray:
    return to_bf16_codes(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


# --------------------------------------------------------------------------
# device upload (array conversion only)
# --------------------------------------------------------------------------

def to_torch(case: Case, device, layout: str = "HND", q_pad_heads: int = 0, q_pad_dim: int = 0):
    """Copy a case's arrays to ``device`` as torch tensors.

    layout "HND" keeps [page][head][slot][d] contiguous; "NHD" stores
    [page][slot][head][d] and returns the [page][head][slot][d] strided view.
    ``q_pad_heads`` > 0 embeds q in a wider head dimension so that the query
    tensor the kernels see is not contiguous; ``q_pad_dim`` > 0 pads each
    query row instead (rows evenly spaced, wider than the row).
    """
    torch = _torch()

    def cache(arr):
        if arr is None:
            return None
        dt = torch.int16 if arr.dtype == np.uint16 else torch.uint8
        host = torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr)
        if layout == "NHD":
            t = host.permute(0, 2, 1, 3).contiguous().to(device)
            t = t.permute(0, 2, 1, 3)
        else:
            t = host.to(device)
        assert t.dtype == dt
        return t.view(torch.bfloat16) if dt == torch.int16 else t

    q = torch.from_numpy(case.q.view(np.int16))
    if q_pad_heads or q_pad_dim:
        B, T, Hq, D = q.shape
        big = torch.zeros((B, T, Hq + q_pad_heads, D + q_pad_dim), dtype=torch.int16)
        big[:, :, :Hq, :D] = q
        qd = big.to(device)[:, :, :Hq, :D]
    else:
        qd = q.to(device)
    return dict(q=qd.view(torch.bfloat16), k_cache=cache(case.k_cache), v_cache=cache(case.v_cache),
                block_table=torch.from_numpy(case.block_table).to(device))

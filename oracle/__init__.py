"""fp64 CPU oracle for split-KV decode attention -- TEST INFRASTRUCTURE ONLY.

This package is the correctness reference the HIP path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (``split_kv_amd``) never does and
shares no code, header, table or constant with it.  The only thing both sides
consume is the seeded input arrays drawn by ``synth``.

What it computes follows the split-KV pages:

* plain softmax attention of a few query tokens over a long paged KV cache
  (``attention.attend``) -- the result the method must reach exactly, up to
  rounding order ("vLLM 0.30.0 FA4 SplitKV Bug: H100 Decode Can Be 48%
  Slower", section "Why the result is still correct");
* the split of the KV range into ``num_splits`` ranges, each giving a partial
  result, merged by a combine step (same page, section "What SplitKV is trying
  to do"), in fp64 (``attention.split_partials`` / ``attention.combine``);
* the split planner and its integer range contract (``plan``), which must
  honour the runtime split count (same page, section "The actual bug is one
  missing constructor argument");
* exact decoders for bf16 and OCP e4m3fn codes (``codes``), for the FP8 KV
  cache read with bf16 queries ("Xqa decode kernels", section "Purpose");
* the step before decode: the new tokens' key/value rows written into their
  pages, quantised to e4m3 for an FP8 cache (``append``).

Every function is pinned by ``-m "not gpu"`` tests against brute force, closed
forms, library special cases and exhaustive code tables; none is "parity
unpinned".
"""
from . import codes, plan, attention, append  # noqa: F401
from .codes import decode_bf16, decode_e4m3  # noqa: F401
from .plan import split_range, make_plan, debug_records  # noqa: F401
from .attention import (dequant_kv, attend, split_partials, combine,  # noqa: F401
                        attend_rows)
from .append import e4m3_encode, quantise_bf16, append_kv  # noqa: F401

"""DecodeSession: plan + caller-owned buffers around the C ABI, for torch users.

This is marshalling only.  It runs ``splitkv_plan`` on the host, copies the
plan arrays to the device, allocates the workspace, output and log-sum-exp
tensors with torch (the library itself never allocates), fills a
``splitkv_args`` block from tensor addresses and strides, and calls the
library's entry points on torch's current stream.  No arithmetic of the
method happens here.
"""
from __future__ import annotations

import numpy as np

from . import (SPLITKV_KERNEL_GQA, SPLITKV_KERNEL_MLA, SPLITKV_KV_BF16, SPLITKV_KV_E4M3,
               SPLITKV_MAX_SPLITS_LIMIT, SPLITKV_OUT_BF16, SPLITKV_OUT_F32, SPLITKV_Q_BF16, SPLITKV_Q_E4M3,
               SPLITKV_ROWS_PER_WG_GQA, SPLITKV_ROWS_PER_WG_MLA,
               splitkv_args, splitkv_combine, splitkv_decode, splitkv_decode_noalloc,
               splitkv_decode_partial, splitkv_decode_single_launch,
               splitkv_decode_partial_fp8, splitkv_mla_decode_partial, splitkv_plan,
               splitkv_plan_args, splitkv_workspace_bytes)


def _torch():
    import torch
    return torch


class DecodeSession:
    """One decode-attention problem on the current HIP device.

    q:           bf16 tensor [B, T, Hq, d_qk] (last dim contiguous, 16-byte aligned rows)
    k_cache:     [num_pages, Hkv, P, d_qk] view (bf16, or uint8 / float8_e4m3fn codes);
                 any strides with the feature dim contiguous
    v_cache:     same with d_v (None for MLA, where V = K[..., :d_v])
    block_table: int32 [B, max_pages] on the device
    seq_lens:    host sequence lengths (numpy or list)
    q_scale:     MLA over an e4m3 cache only: if given, the kernel quantises q to
                 e4m3 codes of q / q_scale and runs on the FP8 matrix path
    alternate_workspaces: keep two workspaces and let decode steps take them in
                 turn (a step that writes the partials the previous step's merge
                 has just read ran 30.2 instead of 25.0 us on the six-token MLA
                 shape at L=2048; the library keeps no state between calls, so the
                 alternation is the caller's)
    """

    def __init__(self, *, q, k_cache, v_cache, block_table, seq_lens, scale: float,
                 k_scale: float = 1.0, v_scale: float = 1.0, mla: bool = False,
                 requested_splits: int = 0, max_splits: int = SPLITKV_MAX_SPLITS_LIMIT, num_cus: int = 0,
                 out_fp32: bool = False, with_lse: bool = True, debug: bool = False,
                 q_scale: float | None = None, alternate_workspaces: bool = True):
        torch = _torch()
        self.torch = torch
        dev = q.device
        self.mla = bool(mla)
        B, T, Hq, d_qk = q.shape
        num_pages, Hkv, P, _ = k_cache.shape
        d_v = 512 if mla else v_cache.shape[-1]
        fp8 = k_cache.dtype in (torch.uint8, torch.float8_e4m3fn)
        self.kv_dtype = SPLITKV_KV_E4M3 if fp8 else SPLITKV_KV_BF16
        self.kernel = SPLITKV_KERNEL_MLA if mla else SPLITKV_KERNEL_GQA
        self.shape = dict(B=B, T=T, Hq=Hq, Hkv=Hkv, d_qk=d_qk, d_v=d_v, P=P, num_pages=num_pages)
        self.q, self.k_cache, self.v_cache = q, k_cache, v_cache
        self.block_table = block_table
        self.seq_lens_host = np.ascontiguousarray(seq_lens, dtype=np.int32)
        self.seq_lens = torch.as_tensor(self.seq_lens_host, device=dev)
        self.scale, self.k_scale, self.v_scale = float(scale), float(k_scale), float(v_scale)
        self.q_dtype = SPLITKV_Q_BF16 if q_scale is None else SPLITKV_Q_E4M3
        self.q_scale = 1.0 if q_scale is None else float(q_scale)
        self.out_fp32 = out_fp32
        self.out = torch.empty((B, T, Hq, d_v), dtype=torch.float32 if out_fp32 else torch.bfloat16,
                               device=dev)
        self.lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev) if with_lse else None
        self.want_debug = debug
        self.num_cus = num_cus
        self.max_splits = max_splits
        self.alternate_workspaces = alternate_workspaces
        self._phase = 0
        self.replan(requested_splits)

    # -- plan ---------------------------------------------------------------
    def replan(self, requested_splits: int):
        torch = self.torch
        s = self.shape
        pa = splitkv_plan_args(B=s["B"], T=s["T"], Hq=s["Hq"], Hkv=s["Hkv"], kernel=self.kernel,
                               requested_splits=requested_splits, max_splits=self.max_splits,
                               num_cus=self.num_cus, d_qk=s["d_qk"], d_v=s["d_v"],
                               kv_dtype=self.kv_dtype)
        ns, off, info = splitkv_plan(pa, self.seq_lens_host)
        self.requested_splits = requested_splits
        self.num_splits_host, self.slot_offset_host, self.slot_info_host = ns, off, info
        dev = self.q.device
        self.num_splits = torch.as_tensor(ns, device=dev)
        self.slot_offset = torch.as_tensor(off, device=dev)
        self.slot_info = torch.as_tensor(info, device=dev)
        self.total_slots = int(off[-1])
        nbytes = splitkv_workspace_bytes(self.total_slots, s["T"], s["Hq"], s["d_v"])
        self.workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=dev)
        self.workspace_alt = (torch.empty_like(self.workspace)
                              if self.alternate_workspaces and self.total_slots > s["B"] else None)
        # arrival counters of the single-launch step (zero; each call leaves them zero)
        if not self.mla:
            rb = -(-((s["Hq"] // s["Hkv"]) * s["T"]) // SPLITKV_ROWS_PER_WG_GQA)
            self.tickets = torch.zeros((s["B"], s["Hkv"], rb), dtype=torch.int32, device=dev)
        else:
            self.tickets = None
        if self.want_debug:
            rows = s["T"] * s["Hq"] if self.mla else (s["Hq"] // s["Hkv"]) * s["T"]
            rpw = SPLITKV_ROWS_PER_WG_MLA if self.mla else SPLITKV_ROWS_PER_WG_GQA
            self.row_blocks = -(-rows // rpw)
            self.debug = torch.full((self.total_slots, s["Hkv"], self.row_blocks, 8), -1,
                                    dtype=torch.int32, device=dev)
        else:
            self.debug = None
        self._build_args()

    def _build_args(self):
        s = self.shape
        q, k, v = self.q, self.k_cache, self.v_cache
        a = splitkv_args()
        a.q = q.data_ptr()
        a.q_stride_b, a.q_stride_t, a.q_stride_h = q.stride(0), q.stride(1), q.stride(2)
        a.k_cache = k.data_ptr()
        a.k_stride_page, a.k_stride_head, a.k_stride_tok = k.stride(0), k.stride(1), k.stride(2)
        if v is not None:
            a.v_cache = v.data_ptr()
            a.v_stride_page, a.v_stride_head, a.v_stride_tok = v.stride(0), v.stride(1), v.stride(2)
        a.block_table = self.block_table.data_ptr()
        a.bt_stride = self.block_table.stride(0)
        a.seq_lens = self.seq_lens.data_ptr()
        a.num_splits = self.num_splits.data_ptr()
        a.slot_offset = self.slot_offset.data_ptr()
        a.slot_info = self.slot_info.data_ptr()
        a.total_slots = self.total_slots
        a.B, a.T, a.Hq, a.Hkv = s["B"], s["T"], s["Hq"], s["Hkv"]
        a.d_qk, a.d_v, a.page_size, a.num_pages = s["d_qk"], s["d_v"], s["P"], s["num_pages"]
        a.kv_dtype = self.kv_dtype
        a.scale, a.k_scale, a.v_scale = self.scale, self.k_scale, self.v_scale
        a.q_dtype, a.q_scale = self.q_dtype, self.q_scale
        a.workspace = self.workspace.data_ptr()
        a.workspace_bytes = self.workspace.numel() * 4
        a.out = self.out.data_ptr()
        a.out_dtype = SPLITKV_OUT_F32 if self.out_fp32 else SPLITKV_OUT_BF16
        a.lse = self.lse.data_ptr() if self.lse is not None else None
        a.debug = self.debug.data_ptr() if self.debug is not None else None
        ns = self.num_splits_host
        a.uniform_splits = int(ns[0]) if len(ns) and (ns == ns[0]).all() else 0
        a.max_seq_splits = int(ns.max()) if len(ns) else 0
        info = self.slot_info_host
        a.max_range_tokens = max(1, int((info[:, 3] - info[:, 2]).max())) if len(info) else 0
        a.tickets = self.tickets.data_ptr() if self.tickets is not None else None
        self.args = a

    def set_block_table(self, block_table):
        """Point later steps at another block table of the same shape (no re-plan)."""
        self.block_table = block_table
        self.args.block_table = block_table.data_ptr()
        self.args.bt_stride = block_table.stride(0)

    # -- steps ----------------------------------------------------------------
    def _stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def _step(self, fn):
        """Run one decode step on the next workspace of the alternation."""
        if self.workspace_alt is not None:
            ws = self.workspace_alt if self._phase else self.workspace
            self._phase ^= 1
            self.args.workspace = ws.data_ptr()
        try:
            fn(self.args, self.kernel, self._stream())
        finally:
            self.args.workspace = self.workspace.data_ptr()
        return self.out, self.lse

    def decode(self):
        """The whole decode step: partial kernel, then the combine where needed."""
        return self._step(splitkv_decode)

    def decode_single_launch(self):
        """The whole grouped-query decode step in one kernel (ticketed last-arriver merge)."""
        return self._step(splitkv_decode_single_launch)

    def decode_noalloc(self):
        """The whole decode step with the partials in the library's own buffer."""
        splitkv_decode_noalloc(self.args, self.kernel, self._stream())
        return self.out, self.lse

    def partial(self):
        """Partial kernel only: writes (m, l, o) of every slot into the workspace."""
        if self.mla:
            splitkv_mla_decode_partial(self.args, self._stream())
        elif self.kv_dtype == SPLITKV_KV_E4M3:
            splitkv_decode_partial_fp8(self.args, self._stream())
        else:
            splitkv_decode_partial(self.args, self._stream())

    def combine(self):
        splitkv_combine(self.args, self._stream())
        return self.out, self.lse

    def partials(self):
        """(part_m [S,T,Hq], part_l [S,T,Hq], part_o [S,T,Hq,d_v]) of the workspace:
        views, except the MLA layout's o, which is decoded from its int16 codes
        and half-row scales into a new fp32 tensor."""
        s = self.shape
        S, T, Hq, dv = self.total_slots, s["T"], s["Hq"], s["d_v"]
        rows = S * T * Hq
        w = self.workspace
        pm, pl = w[:rows].view(S, T, Hq), w[rows:2 * rows].view(S, T, Hq)
        if dv == 512:
            scales = w[2 * rows:4 * rows].view(S, T, Hq, 2)
            q0 = -(-(4 * rows * 4) // 256) * 256 // 2          # int16 offset of the codes
            codes = w.view(self.torch.int16)[q0:q0 + rows * dv].view(S, T, Hq, 2, dv // 2)
            return pm, pl, (codes.float() * scales[..., None]).reshape(S, T, Hq, dv)
        ml = -(-(2 * rows * 4) // 256) * 256 // 4
        return pm, pl, w[ml:ml + rows * dv].view(S, T, Hq, dv)

"""Python binding of libsplitkv.so, the gfx950 split-KV decode-attention library.

Argument marshalling only: every function here has the name of the C entry
point it calls (see ``include/splitkv.h``) and does no arithmetic of the
method.  Device buffers are plain integers (device addresses, e.g. a torch
tensor's ``data_ptr()``); streams are ``hipStream_t`` values as integers
(e.g. ``torch.cuda.current_stream().cuda_stream``).

The library must be built (``python -m split_kv_amd.build``); importing
works without it, but the first call raises ``RuntimeError`` -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsplitkv.so")

SPLITKV_OK = 0
SPLITKV_ERR_INVALID_ARG = -1
SPLITKV_ERR_UNSUPPORTED = -2
SPLITKV_ERR_WORKSPACE = -3
SPLITKV_ERR_LAUNCH = -4
SPLITKV_ERR_DEVICE = -5

SPLITKV_GRANULE = 16
SPLITKV_AUTO_SPLIT_MIN_BYTES = 196608
SPLITKV_AUTO_LAT_NUM = 3
SPLITKV_AUTO_LAT_DEN = 2
SPLITKV_AUTO_BALANCE = 4
SPLITKV_AUTO_WG_OVERHEAD_BYTES = 32768
SPLITKV_MAX_SPLITS_LIMIT = 256
SPLITKV_ROWS_PER_WG_GQA = 16
SPLITKV_ROWS_PER_WG_MLA = 128
SPLITKV_DEBUG_INTS = 8
SPLITKV_NOALLOC_SCRATCH_BYTES = 64 << 20
SPLITKV_SINGLE_LAUNCH_MAX_WORKGROUPS = 64

SPLITKV_KV_BF16 = 0
SPLITKV_KV_E4M3 = 1
SPLITKV_KERNEL_GQA = 0
SPLITKV_KERNEL_MLA = 1
SPLITKV_OUT_BF16 = 0
SPLITKV_OUT_F32 = 1
SPLITKV_Q_BF16 = 0
SPLITKV_Q_E4M3 = 1

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class splitkv_plan_args(ctypes.Structure):
    _fields_ = [("B", c_i32), ("T", c_i32), ("Hq", c_i32), ("Hkv", c_i32), ("kernel", c_i32),
                ("requested_splits", c_i32), ("max_splits", c_i32), ("num_cus", c_i32),
                ("d_qk", c_i32), ("d_v", c_i32), ("kv_dtype", c_i32)]


class splitkv_args(ctypes.Structure):
    _fields_ = [
        ("q", c_vp), ("q_stride_b", c_i64), ("q_stride_t", c_i64), ("q_stride_h", c_i64),
        ("k_cache", c_vp), ("v_cache", c_vp),
        ("k_stride_page", c_i64), ("k_stride_head", c_i64), ("k_stride_tok", c_i64),
        ("v_stride_page", c_i64), ("v_stride_head", c_i64), ("v_stride_tok", c_i64),
        ("block_table", c_vp), ("bt_stride", c_i64),
        ("seq_lens", c_vp), ("num_splits", c_vp), ("slot_offset", c_vp), ("slot_info", c_vp),
        ("total_slots", c_i32),
        ("B", c_i32), ("T", c_i32), ("Hq", c_i32), ("Hkv", c_i32), ("d_qk", c_i32), ("d_v", c_i32),
        ("page_size", c_i32), ("num_pages", c_i32), ("kv_dtype", c_i32),
        ("scale", c_f32), ("k_scale", c_f32), ("v_scale", c_f32),
        ("workspace", c_vp), ("workspace_bytes", c_sz),
        ("out", c_vp), ("out_dtype", c_i32), ("lse", c_vp), ("debug", c_vp),
        ("uniform_splits", c_i32),
        ("q_dtype", c_i32), ("q_scale", c_f32),
        ("max_seq_splits", c_i32),
        ("max_range_tokens", c_i32),
        ("tickets", c_vp),
    ]


class splitkv_append_args(ctypes.Structure):
    _fields_ = [
        ("k_new", c_vp), ("v_new", c_vp),
        ("k_new_stride_b", c_i64), ("k_new_stride_t", c_i64), ("k_new_stride_h", c_i64),
        ("v_new_stride_b", c_i64), ("v_new_stride_t", c_i64), ("v_new_stride_h", c_i64),
        ("k_cache", c_vp), ("v_cache", c_vp),
        ("k_stride_page", c_i64), ("k_stride_head", c_i64), ("k_stride_tok", c_i64),
        ("v_stride_page", c_i64), ("v_stride_head", c_i64), ("v_stride_tok", c_i64),
        ("block_table", c_vp), ("bt_stride", c_i64), ("positions", c_vp),
        ("B", c_i32), ("T", c_i32), ("Hkv", c_i32), ("d_k", c_i32), ("d_v", c_i32),
        ("page_size", c_i32), ("num_pages", c_i32), ("kv_dtype", c_i32),
        ("k_scale", c_f32), ("v_scale", c_f32),
    ]


class SplitKVError(RuntimeError):
    def __init__(self, fn, status, message):
        super().__init__(f"{fn} returned {status}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()


def load():
    """dlopen the library once and declare every exported signature."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m split_kv_amd.build` "
                               "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "splitkv_plan": (c_i32, [P(splitkv_plan_args), c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
            "splitkv_split_range": (c_i32, [c_i32, c_i32, c_i32, P(c_i32), P(c_i32)]),
            "splitkv_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
            "splitkv_decode_partial": (c_i32, [P(splitkv_args), c_vp]),
            "splitkv_decode_partial_fp8": (c_i32, [P(splitkv_args), c_vp]),
            "splitkv_mla_decode_partial": (c_i32, [P(splitkv_args), c_vp]),
            "splitkv_combine": (c_i32, [P(splitkv_args), c_vp]),
            "splitkv_decode": (c_i32, [P(splitkv_args), c_i32, c_vp]),
            "splitkv_decode_noalloc": (c_i32, [P(splitkv_args), c_i32, c_vp]),
            "splitkv_decode_single_launch": (c_i32, [P(splitkv_args), c_i32, c_vp]),
            "splitkv_validate_block_table": (c_i32, [c_vp, c_vp, c_i32, c_i64, c_i32, c_i32]),
            "splitkv_e4m3_to_bf16": (c_i32, [c_vp, c_vp, c_i64, c_vp]),
            "splitkv_append_kv": (c_i32, [P(splitkv_append_args), c_vp]),
            "splitkv_append_args_size": (c_sz, []),
            "splitkv_calib_empty": (c_i32, [c_vp]),
            "splitkv_calib_stream_read": (c_i32, [c_vp, c_sz, c_i32, c_vp, c_vp]),
            "splitkv_calib_mfma": (c_i32, [c_i32, c_i32, c_vp, c_vp]),
            "splitkv_mla_short_range": (c_i32, [c_vp]),
            "splitkv_calib_lds_read": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp]),
            "splitkv_last_error": (ctypes.c_char_p, []),
            "splitkv_version": (ctypes.c_char_p, []),
            "splitkv_args_size": (c_sz, []),
            "splitkv_plan_args_size": (c_sz, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.splitkv_args_size() != ctypes.sizeof(splitkv_args) or \
                lib.splitkv_plan_args_size() != ctypes.sizeof(splitkv_plan_args) or \
                lib.splitkv_append_args_size() != ctypes.sizeof(splitkv_append_args):
            raise RuntimeError("splitkv_args layout of the binding does not match the library")
        _lib = lib
        return lib


EXPORTED = ("splitkv_plan", "splitkv_split_range", "splitkv_workspace_bytes",
            "splitkv_decode_partial", "splitkv_decode_partial_fp8", "splitkv_mla_decode_partial",
            "splitkv_combine", "splitkv_decode", "splitkv_decode_noalloc", "splitkv_decode_single_launch",
            "splitkv_validate_block_table",
            "splitkv_e4m3_to_bf16", "splitkv_append_kv", "splitkv_last_error", "splitkv_version",
            "splitkv_args_size", "splitkv_plan_args_size", "splitkv_append_args_size",
            "splitkv_calib_empty", "splitkv_calib_stream_read", "splitkv_calib_mfma", "splitkv_calib_lds_read",
            "splitkv_mla_short_range")


def _check(fn, status):
    if status != SPLITKV_OK:
        raise SplitKVError(fn, status, splitkv_last_error())


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def splitkv_last_error() -> str:
    return load().splitkv_last_error().decode()


def splitkv_version() -> str:
    return load().splitkv_version().decode()


def splitkv_plan(args: splitkv_plan_args, seq_lens):
    """Host planner -> (num_splits[B], slot_offset[B+1], slot_info[S, 4]) as int32 numpy arrays."""
    lib = load()
    lens = _i32(seq_lens)
    B = int(args.B)
    if lens.shape != (B,):
        raise ValueError(f"seq_lens has shape {lens.shape}, expected ({B},)")
    ns = np.zeros(B, np.int32)
    off = np.zeros(B + 1, np.int32)
    cap = max(1, B * max(1, int(args.max_splits)))
    info = np.zeros((cap, 4), np.int32)
    total = c_i32(0)
    st = lib.splitkv_plan(ctypes.byref(args), lens.ctypes.data, ns.ctypes.data, off.ctypes.data,
                          info.ctypes.data, cap, ctypes.byref(total))
    _check("splitkv_plan", st)
    return ns, off, info[:total.value].copy()


def splitkv_split_range(L: int, n: int, i: int):
    s, e = c_i32(0), c_i32(0)
    _check("splitkv_split_range", load().splitkv_split_range(L, n, i, ctypes.byref(s), ctypes.byref(e)))
    return s.value, e.value


def splitkv_workspace_bytes(total_slots: int, T: int, Hq: int, d_v: int) -> int:
    return int(load().splitkv_workspace_bytes(total_slots, T, Hq, d_v))


def splitkv_decode_partial(args: splitkv_args, stream: int = 0):
    _check("splitkv_decode_partial", load().splitkv_decode_partial(ctypes.byref(args), stream))


def splitkv_decode_partial_fp8(args: splitkv_args, stream: int = 0):
    _check("splitkv_decode_partial_fp8", load().splitkv_decode_partial_fp8(ctypes.byref(args), stream))


def splitkv_mla_decode_partial(args: splitkv_args, stream: int = 0):
    _check("splitkv_mla_decode_partial", load().splitkv_mla_decode_partial(ctypes.byref(args), stream))


def splitkv_mla_short_range(args: splitkv_args) -> bool:
    return bool(load().splitkv_mla_short_range(ctypes.byref(args)))


def splitkv_combine(args: splitkv_args, stream: int = 0):
    _check("splitkv_combine", load().splitkv_combine(ctypes.byref(args), stream))


def splitkv_decode(args: splitkv_args, kernel: int, stream: int = 0):
    _check("splitkv_decode", load().splitkv_decode(ctypes.byref(args), kernel, stream))


def splitkv_decode_single_launch(args: splitkv_args, kernel: int, stream: int = 0):
    _check("splitkv_decode_single_launch",
           load().splitkv_decode_single_launch(ctypes.byref(args), kernel, stream))


def splitkv_decode_noalloc(args: splitkv_args, kernel: int, stream: int = 0):
    """splitkv_decode with the partials in the library's own buffer (args.workspace is ignored)."""
    _check("splitkv_decode_noalloc", load().splitkv_decode_noalloc(ctypes.byref(args), kernel, stream))


def splitkv_validate_block_table(block_table, seq_lens, page_size: int, num_pages: int):
    bt = _i32(block_table)
    lens = _i32(seq_lens)
    st = load().splitkv_validate_block_table(bt.ctypes.data, lens.ctypes.data, lens.shape[0],
                                             bt.shape[1], page_size, num_pages)
    _check("splitkv_validate_block_table", st)


def splitkv_e4m3_to_bf16(src: int, dst: int, n: int, stream: int = 0):
    _check("splitkv_e4m3_to_bf16", load().splitkv_e4m3_to_bf16(src, dst, n, stream))


def splitkv_append_kv(args: splitkv_append_args, stream: int = 0):
    _check("splitkv_append_kv", load().splitkv_append_kv(ctypes.byref(args), stream))


def splitkv_calib_empty(stream: int = 0):
    _check("splitkv_calib_empty", load().splitkv_calib_empty(stream))


def splitkv_calib_stream_read(src: int, nbytes: int, workgroups: int, sink: int, stream: int = 0):
    _check("splitkv_calib_stream_read", load().splitkv_calib_stream_read(src, nbytes, workgroups, sink, stream))


def splitkv_calib_mfma(workgroups: int, iters: int, sink: int, stream: int = 0):
    _check("splitkv_calib_mfma", load().splitkv_calib_mfma(workgroups, iters, sink, stream))


def splitkv_calib_lds_read(workgroups: int, iters: int, mode: int, sink: int, stream: int = 0):
    _check("splitkv_calib_lds_read", load().splitkv_calib_lds_read(workgroups, iters, mode, sink, stream))

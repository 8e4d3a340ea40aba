"""ctypes view of the C ABI declared in include/paged_decode.h.

Loads ``libpaged_decode.so`` from this package directory.  There is no
fallback: if the library is missing the import fails with an error that says
how to build it.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpaged_decode.so")

PD_OK = 0
PD_ERR_INVALID = -1
PD_ERR_ALIGN = -2
PD_ERR_UNSUPPORTED = -3
PD_ERR_WORKSPACE = -4
PD_ERR_HIP = -5
PD_KV_BF16 = 0
PD_KV_FP8_E4M3FN = 1

EXPORTS = (
    "pd_status_string",
    "num_kv_splits_cap",
    "pd_gqa_split_cap",
    "pd_mla_split_cap",
    "pd_split_rule",
    "pd_workspace_bytes",
    "paged_decode_gqa",
    "paged_verify_gqa",
    "paged_verify_gqa_varlen",
    "paged_verify_gqa_noalloc",
    "paged_verify_gqa_append",
    "paged_decode_gqa_partials",
    "paged_verify_gqa_partials",
    "paged_kv_append",
    "paged_verify_mla",
    "paged_verify_mla_partials",
    "merge_splits",
    "pd_stream_read_probe",
)

_c_i32, _c_i64, _c_f32, _c_sz, _c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                        ctypes.c_size_t, ctypes.c_void_p)


class PagedDecodeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"HIP library not built: {LIB_PATH} is missing. Build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (or "
            "`python paged_split_kv_decode_amd/build.py`) on a machine with hipcc.")
    lib = ctypes.CDLL(LIB_PATH)
    lib.pd_status_string.argtypes = [ctypes.c_int]
    lib.pd_status_string.restype = ctypes.c_char_p
    lib.num_kv_splits_cap.argtypes = [_c_i32] * 8
    lib.num_kv_splits_cap.restype = _c_i32
    lib.pd_gqa_split_cap.argtypes = [_c_i32] * 5
    lib.pd_gqa_split_cap.restype = _c_i32
    lib.pd_mla_split_cap.argtypes = [_c_i32] * 5
    lib.pd_mla_split_cap.restype = _c_i32
    lib.pd_split_rule.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                  _c_i32, _c_i32, _c_i32]
    lib.pd_split_rule.restype = _c_i32
    lib.pd_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32]
    lib.pd_workspace_bytes.restype = _c_sz
    lib.paged_decode_gqa.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i64, _c_i64, _c_i32,          # kv, page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_vp, _c_i32, _c_f32,           # seq_lens, sinks, window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32, _c_vp, _c_sz,                   # splits, workspace, bytes
        _c_vp, _c_i64, _c_i64,                  # out, strides
        _c_vp, _c_i64, _c_vp,                   # lse, stride, stream
    ]
    lib.paged_decode_gqa.restype = ctypes.c_int
    lib.paged_verify_gqa.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,    # kv, kv_dtype, k_scale, v_scale, per-head flag
        _c_i64, _c_i64, _c_i32,                 # kv page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_vp, _c_i32,                   # seq_lens, real_seq_lens, qlen
        _c_vp, _c_i32, _c_f32,                  # sinks, window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32, _c_vp, _c_sz,                   # splits, workspace, bytes
        _c_vp, _c_i64, _c_i64,                  # out, strides
        _c_vp, _c_i64, _c_vp,                   # lse, stride, stream
    ]
    lib.paged_verify_gqa.restype = ctypes.c_int
    lib.paged_verify_gqa_append.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,    # kv, kv_dtype, k_scale, v_scale, per-head flag
        _c_i64, _c_i64, _c_i32,                 # kv page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_vp, _c_i32,                   # seq_lens, real_seq_lens, qlen
        _c_vp, _c_i64, _c_i64,                  # k_new, strides
        _c_vp, _c_i64, _c_i64,                  # v_new, strides
        _c_vp, _c_i32, _c_f32,                  # sinks, window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32, _c_vp, _c_sz,                   # splits, workspace, bytes
        _c_vp, _c_i64, _c_i64,                  # out, strides
        _c_vp, _c_i64, _c_vp,                   # lse, stride, stream
    ]
    lib.paged_verify_gqa_append.restype = ctypes.c_int
    lib.paged_verify_gqa_noalloc.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,    # kv, kv_dtype, k_scale, v_scale, per-head flag
        _c_i64, _c_i64, _c_i32,                 # kv page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_vp, _c_i32,                   # seq_lens, real_seq_lens, qlen
        _c_vp, _c_i32, _c_f32,                  # sinks, window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32,                                 # splits
        _c_vp, _c_i64, _c_i64,                  # out, strides
        _c_vp, _c_i64, _c_vp,                   # lse, stride, stream
    ]
    lib.paged_verify_gqa_noalloc.restype = ctypes.c_int
    lib.paged_verify_gqa_varlen.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,    # kv, kv_dtype, k_scale, v_scale, per-head flag
        _c_i64, _c_i64, _c_i32,                 # kv page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_vp,                           # seq_lens, real_seq_lens
        _c_vp, _c_i32, _c_i32,                  # cu_seqlens_q, max_qlen, total_rows
        _c_vp, _c_i32, _c_f32,                  # sinks, window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32, _c_vp, _c_sz,                   # splits, workspace, bytes
        _c_vp, _c_i64, _c_i64,                  # out, strides
        _c_vp, _c_i64, _c_vp,                   # lse, stride, stream
    ]
    lib.paged_verify_gqa_varlen.restype = ctypes.c_int
    lib.paged_kv_append.argtypes = [
        _c_vp, _c_i64, _c_i64, _c_i32,          # src0, strides, elems
        _c_vp, _c_i64, _c_i64, _c_i32,          # src1, strides, elems
        _c_i32,                                 # elem_bytes
        _c_vp, _c_i64, _c_i64, _c_i64, _c_i32,  # cache, page/head/token strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_i32, _c_i32, _c_i32, _c_i32,  # seq_lens, qlen, B, H, P
        _c_vp,                                  # stream
    ]
    lib.paged_kv_append.restype = ctypes.c_int
    lib.paged_decode_gqa_partials.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i64, _c_i64, _c_i32,          # kv, page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_i32, _c_f32,                  # seq_lens, window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32, _c_vp, _c_sz, _c_vp,            # splits, workspace, bytes, stream
    ]
    lib.paged_decode_gqa_partials.restype = ctypes.c_int
    lib.paged_verify_gqa_partials.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q, strides
        _c_vp, _c_i32, _c_vp, _c_vp, _c_i32,    # kv, kv_dtype, k_scale, v_scale, per-head flag
        _c_i64, _c_i64, _c_i32,                 # kv page/head strides, num_pages
        _c_vp, _c_i64, _c_i32,                  # block_table, row stride, max_blocks
        _c_vp, _c_vp,                           # seq_lens, real_seq_lens
        _c_vp, _c_i32, _c_i32,                  # cu_seqlens_q, qlen (max_qlen), total_rows
        _c_i32, _c_f32,                         # window, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, Hq, Hkv, D, P
        _c_i32, _c_vp, _c_sz, _c_vp,            # splits, workspace, bytes, stream
    ]
    lib.paged_verify_gqa_partials.restype = ctypes.c_int
    lib.paged_verify_mla.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q
        _c_vp, _c_i32, _c_i64, _c_i64, _c_i32,  # kv, dtype, page/token strides, num_pages
        _c_vp,                                  # k_scale
        _c_vp, _c_i64, _c_i32,                  # block table
        _c_vp, _c_vp,                           # seq_lens, real_seq_lens
        _c_i32, _c_f32,                         # qlen, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, H, Lk, Lv, P
        _c_i32, _c_vp, _c_sz,                   # splits, workspace, bytes
        _c_vp, _c_i64, _c_i64,                  # out
        _c_vp, _c_i64, _c_vp,                   # lse, stride, stream
    ]
    lib.paged_verify_mla.restype = ctypes.c_int
    lib.paged_verify_mla_partials.argtypes = [
        _c_vp, _c_i64, _c_i64,                  # q
        _c_vp, _c_i32, _c_i64, _c_i64, _c_i32,  # kv, dtype, page/token strides, num_pages
        _c_vp,                                  # k_scale
        _c_vp, _c_i64, _c_i32,                  # block table
        _c_vp, _c_vp,                           # seq_lens, real_seq_lens
        _c_i32, _c_f32,                         # qlen, sm_scale
        _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,  # B, H, Lk, Lv, P
        _c_i32, _c_vp, _c_sz, _c_vp,            # splits, workspace, bytes, stream
    ]
    lib.paged_verify_mla_partials.restype = ctypes.c_int
    lib.merge_splits.argtypes = [_c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp,
                                 _c_vp, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp]
    lib.merge_splits.restype = ctypes.c_int
    lib.pd_stream_read_probe.argtypes = [_c_vp, _c_sz, _c_vp, _c_i32, _c_vp]
    lib.pd_stream_read_probe.restype = ctypes.c_int
    return lib


lib = _load()


def check(fn: str, status: int) -> None:
    if status != PD_OK:
        raise PagedDecodeError(fn, status, lib.pd_status_string(status).decode())

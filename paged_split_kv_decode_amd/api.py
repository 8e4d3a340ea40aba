"""Thin torch binding of the C ABI: argument marshalling only.

torch supplies device memory and the current stream; every step of the
computation runs in the HIP kernels of ``libpaged_decode.so``.  Outputs and
the split workspace are allocated here with torch when the caller does not
pass them (pass them to keep a call allocation-free, e.g. under graph
capture).
"""

from __future__ import annotations

import ctypes

import torch

from . import _native
from ._native import PD_KV_BF16, PD_KV_FP8_E4M3FN, check, lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")


def _cap(fn: str, r: int) -> int:
    if r < 0:
        check(fn, r)
    return int(r)


def num_kv_splits_cap(max_seq_len: int, batch: int, qlen: int, num_q_heads: int,
                      num_kv_heads: int, head_dim_k: int, max_splits: int = 0,
                      device: int = -1) -> int:
    """Static split cap the kernels are tuned for (include/paged_decode.h:
    num_kv_splits_cap); a pure host function."""
    return _cap("num_kv_splits_cap", lib.num_kv_splits_cap(
        int(max_seq_len), int(batch), int(qlen), int(num_q_heads), int(num_kv_heads),
        int(head_dim_k), int(max_splits), int(device)))


def gqa_split_cap(batch: int, num_kv_heads: int, max_seq_len: int, window: int = 0,
                  num_cus: int = 0) -> int:
    """Split cap for the GQA calls (include/paged_decode.h: pd_gqa_split_cap)."""
    return _cap("pd_gqa_split_cap", lib.pd_gqa_split_cap(
        int(batch), int(num_kv_heads), int(max_seq_len), int(window or 0), int(num_cus)))


def mla_split_cap(batch: int, qlen: int, num_heads: int, max_seq_len: int,
                  num_cus: int = 0) -> int:
    """Split cap for paged_verify_mla (include/paged_decode.h: pd_mla_split_cap)."""
    return _cap("pd_mla_split_cap", lib.pd_mla_split_cap(
        int(batch), int(qlen), int(num_heads), int(max_seq_len), int(num_cus)))


def split_rule(max_seq_len: int, batch: int, qlen: int, num_heads: int, block_h: int,
               num_cus: int = 0, occupancy: float = 1.0, min_work_per_split: int = 64,
               max_splits: int = 8, balance_chunk: int = 0) -> int:
    """The split rule with every knob (include/paged_decode.h: pd_split_rule)."""
    return _cap("pd_split_rule", lib.pd_split_rule(
        int(max_seq_len), int(batch), int(qlen), int(num_heads), int(block_h), int(num_cus),
        float(occupancy), int(min_work_per_split), int(max_splits), int(balance_chunk)))


def workspace_bytes(rows: int, num_heads: int, num_splits: int, head_dim_v: int) -> int:
    return int(lib.pd_workspace_bytes(int(rows), int(num_heads), int(num_splits),
                                      int(head_dim_v)))


def alloc_workspace(rows, num_heads, num_splits, head_dim_v, device):
    n = workspace_bytes(rows, num_heads, num_splits, head_dim_v)
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def paged_decode_gqa(q, kv, block_table, seq_lens, sm_scale, sinks=None, window=0,
                     num_kv_splits=1, workspace=None, out=None, lse=None, stream=None,
                     return_lse=True):
    """Paged GQA decode (include/paged_decode.h: paged_decode_gqa).

    q [B, Hq, D] bf16; kv [num_pages, Hkv, P, 2D] bf16 (K | V); block_table
    [B, max_blocks] int32; seq_lens [B] int32; sinks [Hq] fp32 or None.
    Returns (out [B, Hq, D] bf16, lse [B, Hq] fp32 or None).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(kv, "kv", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be contiguous")
    B, Hq, D = q.shape
    num_pages, Hkv, P, two_d = kv.shape
    if two_d != 2 * D or kv.stride(3) != 1 or kv.stride(2) != 2 * D or q.stride(2) != 1:
        raise ValueError("kv must be [pages, Hkv, P, 2D] with contiguous token rows")
    if block_table.shape[0] != B or seq_lens.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table / seq_lens must have one row per request")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != Hq or sinks.stride(0) != 1:
            raise ValueError("sinks must be a contiguous [Hq] tensor")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    if out.stride(2) != 1:
        raise ValueError("out must have a contiguous last dim")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
        if lse.stride(1) != 1:
            raise ValueError("lse must have a contiguous last dim")
    S = int(num_kv_splits)
    if S > 1 and workspace is None:
        workspace = alloc_workspace(B, Hq, S, D, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.paged_decode_gqa(
        _ptr(q), q.stride(0), q.stride(1),
        _ptr(kv), kv.stride(0), kv.stride(1), num_pages,
        _ptr(block_table), block_table.stride(0), block_table.shape[1],
        _ptr(seq_lens), _ptr(sinks), int(window or 0), float(sm_scale),
        B, Hq, Hkv, D, P, S, _ptr(workspace), ws_bytes,
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), 0 if lse is None else lse.stride(0), _stream(stream))
    check("paged_decode_gqa", st)
    return out, lse


def paged_verify_gqa(q, kv, block_table, seq_lens, qlen, sm_scale, sinks=None, window=0,
                     real_seq_lens=None, num_kv_splits=1, workspace=None, out=None, lse=None,
                     stream=None, return_lse=True, k_scale=None, v_scale=None):
    """Paged GQA causal verify (include/paged_decode.h: paged_verify_gqa).

    q [B*qlen, Hq, D] bf16 (the qlen tokens of a request contiguous); kv
    [num_pages, Hkv, P, 2D] bf16, or FP8 E4M3FN codes (uint8 or
    float8_e4m3fn) with device fp32 k_scale / v_scale of one element (one
    scale) or Hkv elements (one per kv head), None meaning 1; block_table
    [B, max_blocks] int32; seq_lens and real_seq_lens (or None) [B] int32;
    sinks [Hq] fp32 or None.
    Returns (out [B*qlen, Hq, D] bf16, lse [B*qlen, Hq] fp32 or None).
    """
    qlen = int(qlen)
    rows = q.shape[0] if q.dim() == 3 else -1
    if qlen < 1 or rows % qlen != 0:
        raise ValueError("q must have qlen rows per request")
    return _verify_gqa(q, kv, block_table, seq_lens, rows // qlen, qlen, None, sm_scale, sinks,
                       window, real_seq_lens, num_kv_splits, workspace, out, lse, stream,
                       return_lse, k_scale, v_scale)


def paged_verify_gqa_append(q, kv, block_table, seq_lens, k_new, v_new, qlen, sm_scale,
                            sinks=None, window=0, real_seq_lens=None, num_kv_splits=1,
                            workspace=None, out=None, lse=None, stream=None, return_lse=True,
                            k_scale=None, v_scale=None):
    """The newest qlen tokens appended to the cache and attended in one call
    (include/paged_decode.h: paged_verify_gqa_append): the result of
    paged_kv_append(kv, block_table, seq_lens, k_new, v_new, qlen) followed
    by paged_verify_gqa(...), bit for bit.

    k_new, v_new [B*qlen, Hkv, D] of the cache's element type (bf16, or FP8
    codes as uint8 / float8_e4m3fn), row b*qlen + t for token t of request
    b.  kv is written in place.  Other arguments as for paged_verify_gqa.
    Returns (out, lse).
    """
    qlen = int(qlen)
    rows = q.shape[0] if q.dim() == 3 else -1
    if qlen < 1 or rows % qlen != 0:
        raise ValueError("q must have qlen rows per request")
    return _verify_gqa(q, kv, block_table, seq_lens, rows // qlen, qlen, None, sm_scale, sinks,
                       window, real_seq_lens, num_kv_splits, workspace, out, lse, stream,
                       return_lse, k_scale, v_scale, new_kv=(k_new, v_new))


def paged_verify_gqa_varlen(q, kv, block_table, seq_lens, cu_seqlens_q, max_qlen, sm_scale,
                            sinks=None, window=0, real_seq_lens=None, num_kv_splits=1,
                            workspace=None, out=None, lse=None, stream=None, return_lse=True,
                            k_scale=None, v_scale=None):
    """Paged GQA causal verify with a query length per request
    (include/paged_decode.h: paged_verify_gqa_varlen).

    q [total_rows, Hq, D] bf16 with request b's query tokens in rows
    cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1; cu_seqlens_q [B + 1] int32 on
    the device (cu[0] = 0, non-decreasing, cu[B] = total_rows); max_qlen a
    host int >= every request's query length, with max_qlen * Hq / Hkv <= 64.
    Other arguments as for paged_verify_gqa.
    Returns (out [total_rows, Hq, D] bf16, lse [total_rows, Hq] fp32 or None).
    """
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    B = seq_lens.shape[0]
    if cu_seqlens_q.shape[0] != B + 1 or cu_seqlens_q.stride(0) != 1:
        raise ValueError("cu_seqlens_q must be a contiguous [B + 1] tensor")
    max_qlen = int(max_qlen)
    if max_qlen < 1:
        raise ValueError("max_qlen must be >= 1")
    return _verify_gqa(q, kv, block_table, seq_lens, B, max_qlen, cu_seqlens_q, sm_scale, sinks,
                       window, real_seq_lens, num_kv_splits, workspace, out, lse, stream,
                       return_lse, k_scale, v_scale)


def paged_verify_gqa_partials(q, kv, block_table, seq_lens, qlen, sm_scale, window=0,
                              real_seq_lens=None, cu_seqlens_q=None, num_kv_splits=1,
                              workspace=None, stream=None, k_scale=None, v_scale=None):
    """Split partials of paged_verify_gqa (cu_seqlens_q None) or of
    paged_verify_gqa_varlen (qlen is then max_qlen) without the merge
    (include/paged_decode.h: paged_verify_gqa_partials).  No sinks: they
    enter in merge_splits.  Returns the fp32 workspace viewed as
    [rows, Hq, S, D + 1]."""
    qlen = int(qlen)
    if qlen < 1:
        raise ValueError("qlen must be >= 1")
    if cu_seqlens_q is None:
        rows = q.shape[0] if q.dim() == 3 else -1
        if rows % qlen != 0:
            raise ValueError("q must have qlen rows per request")
        B = rows // qlen
    else:
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
        B = seq_lens.shape[0]
        if cu_seqlens_q.shape[0] != B + 1 or cu_seqlens_q.stride(0) != 1:
            raise ValueError("cu_seqlens_q must be a contiguous [B + 1] tensor")
    return _verify_gqa(q, kv, block_table, seq_lens, B, qlen, cu_seqlens_q, sm_scale, None,
                       window, real_seq_lens, num_kv_splits, workspace, None, None, stream,
                       False, k_scale, v_scale, partials_only=True)


def _verify_gqa(q, kv, block_table, seq_lens, B, qlen, cu_seqlens_q, sm_scale, sinks, window,
                real_seq_lens, num_kv_splits, workspace, out, lse, stream, return_lse, k_scale,
                v_scale, partials_only=False, new_kv=None):
    _need(q, "q", torch.bfloat16, 3)
    fp8 = kv.dtype in (torch.uint8, torch.float8_e4m3fn)
    if not fp8:
        _need(kv, "kv", torch.bfloat16, 4)
    elif not kv.is_cuda or kv.dim() != 4:
        raise ValueError("kv must be a 4-D device tensor")
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be contiguous")
    rows, Hq, D = q.shape
    num_pages, Hkv, P, two_d = kv.shape
    if two_d != 2 * D or kv.stride(3) != 1 or kv.stride(2) != 2 * D or q.stride(2) != 1:
        raise ValueError("kv must be [pages, Hkv, P, 2D] with contiguous token rows")
    if block_table.shape[0] != B or seq_lens.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table / seq_lens must have one row per request")
    if real_seq_lens is not None:
        _need(real_seq_lens, "real_seq_lens", torch.int32, 1)
        if real_seq_lens.shape[0] != B or real_seq_lens.stride(0) != 1:
            raise ValueError("real_seq_lens must be a contiguous [B] tensor")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != Hq or sinks.stride(0) != 1:
            raise ValueError("sinks must be a contiguous [Hq] tensor")
    if not partials_only:
        if out is None:
            out = torch.empty((rows, Hq, D), dtype=torch.bfloat16, device=q.device)
        _need(out, "out", torch.bfloat16, 3)
        if out.stride(2) != 1:
            raise ValueError("out must have a contiguous last dim")
        if lse is None and return_lse:
            lse = torch.empty((rows, Hq), dtype=torch.float32, device=q.device)
        if lse is not None:
            _need(lse, "lse", torch.float32, 2)
            if lse.stride(1) != 1:
                raise ValueError("lse must have a contiguous last dim")
    per_head = 0
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is None:
            continue
        _need(t, name, torch.float32)
        if t.numel() not in (1, Hkv) or not t.is_contiguous():
            raise ValueError(f"{name} must hold 1 or Hkv contiguous values")
        if t.numel() == Hkv and Hkv > 1:
            per_head = 1
    if per_head and any(t is not None and t.numel() != Hkv for t in (k_scale, v_scale)):
        raise ValueError("k_scale and v_scale must both be scalars or both per kv head")
    S = int(num_kv_splits)
    if partials_only:
        n = rows * Hq * S * (D + 1)
        if workspace is None:
            workspace = torch.empty(max(n, 1), dtype=torch.float32, device=q.device)
        _need(workspace, "workspace", torch.float32)
    elif S > 1 and workspace is None:
        workspace = alloc_workspace(rows, Hq, S, D, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    common = (_ptr(q), q.stride(0), q.stride(1),
              _ptr(kv), PD_KV_FP8_E4M3FN if fp8 else PD_KV_BF16, _ptr(k_scale), _ptr(v_scale),
              per_head, kv.stride(0), kv.stride(1), num_pages,
              _ptr(block_table), block_table.stride(0), block_table.shape[1],
              _ptr(seq_lens), _ptr(real_seq_lens))
    if partials_only:
        st = lib.paged_verify_gqa_partials(
            *common, _ptr(cu_seqlens_q), qlen, rows, int(window or 0), float(sm_scale),
            B, Hq, Hkv, D, P, S, _ptr(workspace), ws_bytes, _stream(stream))
        check("paged_verify_gqa_partials", st)
        return workspace[:n].view(rows, Hq, S, D + 1)
    tail_args = (_ptr(sinks), int(window or 0), float(sm_scale),
                 B, Hq, Hkv, D, P, S, _ptr(workspace), ws_bytes,
                 _ptr(out), out.stride(0), out.stride(1),
                 _ptr(lse), 0 if lse is None else lse.stride(0), _stream(stream))
    if new_kv is not None:
        srcs = []
        for name, t in zip(("k_new", "v_new"), new_kv):
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != kv.dtype or \
                    t.dim() != 3 or tuple(t.shape) != (rows, Hkv, D) or t.stride(2) != 1:
                raise ValueError(f"{name} must be a [B*qlen, Hkv, D] device tensor of the "
                                 "cache's dtype with a contiguous last dim")
            srcs += [_ptr(t), t.stride(0), t.stride(1)]
        st = lib.paged_verify_gqa_append(*common, qlen, *srcs, *tail_args)
        check("paged_verify_gqa_append", st)
    elif cu_seqlens_q is None:
        st = lib.paged_verify_gqa(*common, qlen, *tail_args)
        check("paged_verify_gqa", st)
    else:
        st = lib.paged_verify_gqa_varlen(*common, _ptr(cu_seqlens_q), qlen, rows, *tail_args)
        check("paged_verify_gqa_varlen", st)
    return out, lse


def paged_kv_append(cache, block_table, seq_lens, src0, src1=None, qlen=1, layout="hnd",
                    stream=None):
    """Write the qlen newest tokens of each request into the paged cache
    (include/paged_decode.h: paged_kv_append).  In place; returns ``cache``.

    layout "hnd": cache [num_pages, H, P, row] (the GQA cache; src0 = K and
    src1 = V, each [B*qlen, H, D]); layout "nhd": cache [num_pages, P, H, row]
    (the MLA latent cache with H = 1; src0 = latent rows [B*qlen, 1, Lk] or
    [B*qlen, Lk]).  Elements are bf16 or FP8 codes (uint8); the copy is
    byte-exact.
    """
    if not isinstance(cache, torch.Tensor) or not cache.is_cuda or cache.dim() != 4:
        raise ValueError("cache must be a 4-D device tensor")
    if cache.dtype not in (torch.bfloat16, torch.uint8, torch.float8_e4m3fn):
        raise TypeError("cache must be bf16 or FP8 (uint8 / float8_e4m3fn) elements")
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be contiguous")
    qlen = int(qlen)
    if src0.dim() == 2:
        src0 = src0.unsqueeze(1)
    if src1 is not None and src1.dim() == 2:
        src1 = src1.unsqueeze(1)
    for name, t in (("src0", src0), ("src1", src1)):
        if t is None:
            continue
        if t.dtype != cache.dtype or not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be a [rows, H, n] device tensor of the cache dtype "
                             "with a contiguous last dim")
    if layout == "hnd":
        num_pages, H, P, row = cache.shape
        sp, sh, st = cache.stride(0), cache.stride(1), cache.stride(2)
    elif layout == "nhd":
        num_pages, P, H, row = cache.shape
        sp, st, sh = cache.stride(0), cache.stride(1), cache.stride(2)
    else:
        raise ValueError("layout must be 'hnd' or 'nhd'")
    if cache.stride(3) != 1:
        raise ValueError("cache rows must be contiguous")
    B = block_table.shape[0]
    if seq_lens.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table / seq_lens must have one row per request")
    if src0.shape[0] != B * qlen or src0.shape[1] != H or \
            (src1 is not None and tuple(src1.shape[:2]) != (B * qlen, H)):
        raise ValueError("sources must be [B * qlen, H, n]")
    eb = cache.element_size()
    st_ = lib.paged_kv_append(
        _ptr(src0), src0.stride(0), src0.stride(1), src0.shape[2],
        _ptr(src1), 0 if src1 is None else src1.stride(0), 0 if src1 is None else src1.stride(1),
        0 if src1 is None else src1.shape[2], eb,
        _ptr(cache), sp, sh, st, num_pages,
        _ptr(block_table), block_table.stride(0), block_table.shape[1],
        _ptr(seq_lens), qlen, B, H, P, _stream(stream))
    check("paged_kv_append", st_)
    return cache


def paged_decode_gqa_partials(q, kv, block_table, seq_lens, sm_scale, window=0,
                              num_kv_splits=1, workspace=None, stream=None):
    """Split partials of paged_decode_gqa without the merge
    (include/paged_decode.h: paged_decode_gqa_partials).  Returns the fp32
    workspace viewed as [B, Hq, S, D + 1]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv, "kv", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be contiguous")
    B, Hq, D = q.shape
    num_pages, Hkv, P, two_d = kv.shape
    if two_d != 2 * D or kv.stride(3) != 1 or kv.stride(2) != 2 * D or q.stride(2) != 1:
        raise ValueError("kv must be [pages, Hkv, P, 2D] with contiguous token rows")
    if block_table.shape[0] != B or seq_lens.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table / seq_lens must have one row per request")
    S = int(num_kv_splits)
    n = B * Hq * S * (D + 1)
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.float32, device=q.device)
    _need(workspace, "workspace", torch.float32)
    st = lib.paged_decode_gqa_partials(
        _ptr(q), q.stride(0), q.stride(1),
        _ptr(kv), kv.stride(0), kv.stride(1), num_pages,
        _ptr(block_table), block_table.stride(0), block_table.shape[1],
        _ptr(seq_lens), int(window or 0), float(sm_scale),
        B, Hq, Hkv, D, P, S, _ptr(workspace), workspace.numel() * 4, _stream(stream))
    check("paged_decode_gqa_partials", st)
    return workspace[:n].view(B, Hq, S, D + 1)


def paged_verify_mla(q, kv, block_table, seq_lens, real_seq_lens, qlen, sm_scale,
                     head_dim_v=512, page_size=None, k_scale=None, num_kv_splits=1,
                     workspace=None, out=None, lse=None, stream=None):
    """Causal MLA verify (include/paged_decode.h: paged_verify_mla).

    q [B*qlen, H, Lk] bf16; kv [num_pages, P, 1, Lk] (or [num_pages*P, 1, Lk])
    as bf16, or as uint8 FP8 E4M3FN codes with ``k_scale`` a 1-element fp32
    device tensor.  Returns (out [B*qlen, H, Lv] bf16, lse [B*qlen, H] fp32).
    """
    return _verify_mla(q, kv, block_table, seq_lens, real_seq_lens, qlen, sm_scale,
                       head_dim_v, page_size, k_scale, num_kv_splits, workspace, out, lse,
                       stream, False)


def paged_verify_mla_partials(q, kv, block_table, seq_lens, real_seq_lens, qlen, sm_scale,
                              head_dim_v=512, page_size=None, k_scale=None, num_kv_splits=1,
                              workspace=None, stream=None):
    """Split partials of paged_verify_mla without the merge
    (include/paged_decode.h: paged_verify_mla_partials).  Returns the fp32
    workspace viewed as [B*qlen, H, S, Lv + 1]."""
    return _verify_mla(q, kv, block_table, seq_lens, real_seq_lens, qlen, sm_scale,
                       head_dim_v, page_size, k_scale, num_kv_splits, workspace, None, None,
                       stream, True)


def _verify_mla(q, kv, block_table, seq_lens, real_seq_lens, qlen, sm_scale, head_dim_v,
                page_size, k_scale, num_kv_splits, workspace, out, lse, stream, partials_only):
    _need(q, "q", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.stride(0) != 1:
        raise ValueError("seq_lens must be contiguous")
    rows, H, Lk = q.shape
    if kv.dtype == torch.bfloat16:
        kv_dtype = PD_KV_BF16
    elif kv.dtype in (torch.uint8, torch.float8_e4m3fn):
        kv_dtype = PD_KV_FP8_E4M3FN
    else:
        raise TypeError(f"kv must be bf16 or FP8 E4M3FN codes, got {kv.dtype}")
    if not kv.is_cuda:
        raise ValueError("kv must be a device tensor")
    if kv.dim() == 4:
        num_pages, P = kv.shape[0], kv.shape[1]
        if kv.shape[2] != 1:
            raise ValueError("the verify path expects a single latent KV head")
        s_page, s_tok = kv.stride(0), kv.stride(1)
    elif kv.dim() == 3:
        if page_size is None:
            raise ValueError("page_size is required for a 3-D cache view")
        P = int(page_size)
        if kv.shape[0] % P or kv.shape[1] != 1:
            raise ValueError("3-D cache must be [num_pages * P, 1, Lk]")
        num_pages = kv.shape[0] // P
        s_tok = kv.stride(0)
        s_page = s_tok * P
    else:
        raise ValueError("kv must be 3-D or 4-D")
    if kv.shape[-1] != Lk or kv.stride(-1) != 1 or q.stride(2) != 1:
        raise ValueError("cache / q last dims must match Lk and be contiguous")
    qlen = int(qlen)
    if qlen < 1 or rows % qlen:
        raise ValueError("q rows must be a multiple of qlen")
    B = rows // qlen
    if block_table.shape[0] != B or seq_lens.shape[0] != B or block_table.stride(1) != 1:
        raise ValueError("block_table / seq_lens must have one contiguous row per request")
    if real_seq_lens is not None:
        _need(real_seq_lens, "real_seq_lens", torch.int32, 1)
        if real_seq_lens.shape[0] != B or real_seq_lens.stride(0) != 1:
            raise ValueError("real_seq_lens must be a contiguous [B] tensor")
    if k_scale is not None:
        _need(k_scale, "k_scale", torch.float32)
        if k_scale.numel() < 1:
            raise ValueError("k_scale must hold one value")
    Lv = int(head_dim_v)
    S = int(num_kv_splits)
    head = (_ptr(q), q.stride(0), q.stride(1),
            _ptr(kv), kv_dtype, s_page, s_tok, num_pages, _ptr(k_scale),
            _ptr(block_table), block_table.stride(0), block_table.shape[1],
            _ptr(seq_lens), _ptr(real_seq_lens), int(qlen), float(sm_scale),
            B, H, Lk, Lv, P, S)
    if partials_only:
        n = rows * H * S * (Lv + 1)
        if workspace is None:
            workspace = torch.empty(max(n, 1), dtype=torch.float32, device=q.device)
        _need(workspace, "workspace", torch.float32)
        st = lib.paged_verify_mla_partials(*head, _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream))
        check("paged_verify_mla_partials", st)
        return workspace[:n].view(rows, H, S, Lv + 1)
    if out is None:
        out = torch.empty((rows, H, Lv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((rows, H), dtype=torch.float32, device=q.device)
    if S > 1 and workspace is None:
        workspace = alloc_workspace(rows, H, S, Lv, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.paged_verify_mla(
        *head, _ptr(workspace), ws_bytes,
        _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), lse.stride(0), _stream(stream))
    check("paged_verify_mla", st)
    return out, lse


def merge_splits(workspace, rows, num_heads, num_splits, head_dim_v, sinks=None, out=None,
                 lse=None, stream=None):
    """Merge fp32 split partials [rows, H, S, Dv + 1] into bf16 O and fp32 LSE."""
    _need(workspace, "workspace", torch.float32)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    need = int(rows) * int(num_heads) * int(num_splits) * (int(head_dim_v) + 1)
    if workspace.numel() < need:
        raise ValueError("workspace smaller than rows * H * S * (Dv + 1)")
    dev = workspace.device
    if out is None:
        out = torch.empty((rows, num_heads, head_dim_v), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((rows, num_heads), dtype=torch.float32, device=dev)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != int(num_heads) or sinks.stride(0) != 1:
            raise ValueError("sinks must be a contiguous [num_heads] tensor")
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    for name, t, shape in (("out", out, (rows, num_heads, head_dim_v)),
                           ("lse", lse, (rows, num_heads))):
        if tuple(t.shape) != tuple(int(x) for x in shape) or t.stride(-1) != 1:
            raise ValueError(f"{name} must be {tuple(shape)} with a contiguous last dim")
    st = lib.merge_splits(_ptr(workspace), int(rows), int(num_heads), int(num_splits),
                          int(head_dim_v), _ptr(sinks), _ptr(out), out.stride(0),
                          out.stride(1), _ptr(lse), lse.stride(0), _stream(stream))
    check("merge_splits", st)
    return out, lse


def stream_read_probe(buf, sink, workgroups, stream=None):
    """Streaming-read ceiling probe (include/paged_decode.h:
    pd_stream_read_probe): reads ``buf`` once; ``sink`` is an int32 device
    tensor of at least ``workgroups`` elements."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _need(sink, "sink", torch.int32, 1)
    if sink.numel() < int(workgroups):
        raise ValueError("sink must hold one value per workgroup")
    st = lib.pd_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                  int(workgroups), _stream(stream))
    check("pd_stream_read_probe", st)


__all__ = [
    "PD_KV_BF16", "PD_KV_FP8_E4M3FN", "alloc_workspace", "gqa_split_cap", "merge_splits",
    "mla_split_cap", "num_kv_splits_cap", "paged_decode_gqa", "paged_decode_gqa_partials",
    "paged_kv_append", "paged_verify_gqa", "paged_verify_gqa_partials",
    "paged_verify_gqa_varlen", "paged_verify_mla", "paged_verify_mla_partials",
    "split_rule", "stream_read_probe", "workspace_bytes", "_native",
]

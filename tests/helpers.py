"""Shared test plumbing: moving seeded inputs between torch and the oracle,
compact per-request gathers for oracle runs on samples of large workloads,
and the parity gates."""

from __future__ import annotations

import numpy as np
import torch

import oracle

O_ATOL, O_RTOL = 2e-2, 1e-2          # bf16 O vs the fp64 oracle
O_ATOL_FP8 = 5e-2                    # fp8 cache
LSE_ATOL = 1e-3                      # fp32 LSE
NORM_TOL = 1e-2                      # per (row, head) ||O - O_ref|| / ||O_ref||


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def compact_gqa(w, vals, requests):
    """Oracle inputs for a subset of requests: the pages those requests
    reference are copied to the host into a compact pool and the block table
    is renumbered.  Returns (q_bits, kv_bits, bt, seq_lens, sinks)."""
    requests = list(requests)
    bt = w.block_table[requests]
    used = np.unique(bt[bt >= 0])
    remap = np.full(w.num_pages, -1, np.int64)
    remap[used] = np.arange(len(used))
    idx = torch.from_numpy(used).to(vals["kv"].device)
    raw_dtype = np.uint8 if vals["kv"].dtype == torch.uint8 else np.uint16
    if not len(used):
        kv = np.zeros((0,) + tuple(vals["kv"].shape[1:]), raw_dtype)
    elif raw_dtype == np.uint8:
        kv = vals["kv"].index_select(0, idx).cpu().numpy()
    else:
        kv = bits16(vals["kv"].index_select(0, idx))
    bt2 = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    rows = [b * w.qlen + t for b in requests for t in range(w.qlen)]
    q = bits16(vals["q"][rows])
    sinks = None if vals["sinks"] is None else vals["sinks"].cpu().numpy().astype(np.float64)
    return q, kv, bt2, w.seq_lens[requests], sinks


def oracle_gqa(w, vals, requests=None):
    """Oracle O, LSE of a GQA workload's requests (rows b * qlen + t for verify)."""
    requests = range(w.B) if requests is None else list(requests)
    q, kv, bt, sl, sk = compact_gqa(w, vals, requests)
    fp8 = vals["kv"].dtype == torch.uint8
    if w.qlen == 1 and w.real_seq_lens is None and not fp8:
        return oracle.gqa_decode(q, kv, bt, sl, w.sm_scale, sinks=sk, window=w.window)
    real = None if w.real_seq_lens is None else w.real_seq_lens[list(requests)]
    if fp8:
        return oracle.gqa_verify(q, kv, bt, sl, w.qlen, w.sm_scale, sinks=sk, window=w.window,
                                 real_seq_lens=real, kv_dtype="fp8_e4m3fn",
                                 k_scale=vals["k_scale"].cpu().numpy().astype(np.float64),
                                 v_scale=vals["v_scale"].cpu().numpy().astype(np.float64))
    return oracle.gqa_verify(q, kv, bt, sl, w.qlen, w.sm_scale, sinks=sk, window=w.window,
                             real_seq_lens=real)


def compact_mla(w, vals, requests):
    requests = list(requests)
    bt = w.block_table[requests]
    used = np.unique(bt[bt >= 0])
    remap = np.full(w.num_pages, -1, np.int64)
    remap[used] = np.arange(len(used))
    idx = torch.from_numpy(used).to(vals["kv"].device)
    kvt = vals["kv"].index_select(0, idx)
    kv = kvt.cpu().numpy() if kvt.dtype == torch.uint8 else bits16(kvt)
    bt2 = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    rows = [b * w.qlen + t for b in requests for t in range(w.qlen)]
    q = bits16(vals["q"][rows])
    real = None if w.real_seq_lens is None else w.real_seq_lens[requests]
    return q, kv, bt2, w.seq_lens[requests], real


def oracle_mla(w, vals, requests=None, fp8=False):
    requests = range(w.B) if requests is None else requests
    q, kv, bt, sl, real = compact_mla(w, vals, requests)
    return oracle.mla_verify(q, kv, bt, sl, real, w.qlen, w.sm_scale, w.Lv,
                             kv_dtype="fp8_e4m3fn" if fp8 else "bf16",
                             k_scale=vals.get("k_scale", 1.0))


def check_attention(o_gpu, lse_gpu, O_ref, lse_ref, o_atol=O_ATOL, o_rtol=O_RTOL,
                    lse_atol=LSE_ATOL, norm_tol=NORM_TOL, what=""):
    """The parity gates: elementwise O and LSE tolerances, exact -inf / zero
    for keyless rows, no NaN, and a per-(row, head) normalised error."""
    o = to_f64(o_gpu)
    lse = None if lse_gpu is None else to_f64(lse_gpu)
    assert o.shape == O_ref.shape, (o.shape, O_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    err = np.abs(o - O_ref)
    bad = err > o_atol + o_rtol * np.abs(O_ref)
    assert not bad.any(), (f"{what}: O mismatch at {np.argwhere(bad)[:5].tolist()}, "
                           f"max err {err.max():.3e}")
    keyless = np.isneginf(lse_ref)
    assert np.all(o[keyless] == 0.0), f"{what}: keyless rows must be exactly 0"
    nref = np.linalg.norm(O_ref, axis=-1)
    nerr = np.linalg.norm(o - O_ref, axis=-1)
    ok = nref > 0
    if ok.any():
        rel = nerr[ok] / nref[ok]
        assert rel.max() <= norm_tol, f"{what}: normalised O error {rel.max():.3e}"
    if lse is not None:
        assert np.array_equal(np.isneginf(lse), keyless), f"{what}: -inf LSE pattern differs"
        fin = ~keyless
        assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite LSE"
        d = np.abs(lse[fin] - lse_ref[fin])
        assert d.size == 0 or d.max() <= lse_atol, f"{what}: LSE max err {d.max():.3e}"
    return float(err.max()) if err.size else 0.0

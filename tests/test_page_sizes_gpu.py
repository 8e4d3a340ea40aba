"""GPU parity of the GQA and MLA paths at general page sizes against the fp64
oracle.

"vllm.v1.attention.ops.triton_decode_attention" states support for any page
size of at least one token, and so does the library.  Power-of-two pages
smaller than a 32-token tile put several pages in one tile (1, 2, 4, 8 and
16 tokens: one block-table entry per page, and for 1 and 2 tokens a page per
lane within one load); power-of-two pages of 32 tokens or more hold whole
tiles at an offset inside the page; every other size (3, 5, 12, 33, 48 and
96 here) goes through the general class, whose loads may straddle a page
boundary anywhere in a tile.  Covered: decode with sinks, verify with
windows and real lengths, the FP8 cache, split counts, out-of-range entries
and bitwise equality of the outputs for one logical cache stored at
different page sizes (the kernel's arithmetic does not depend on where a key
lives).  The MLA verify kernel reads 16-row regions of its 32-token tiles:
power-of-two pages of 16 tokens or more hold whole regions, smaller and
non-power-of-two pages are picked per lane; covered at 1 to 96 tokens per
page, bf16 and FP8, with rows that have no key, an out-of-range entry (NaN
for its request) and bitwise equality across page sizes.
"""

import numpy as np
import pytest
import torch

from helpers import O_ATOL_FP8, check_attention, oracle_gqa, oracle_mla
from synth import gqa_workload, mla_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

PAGE_SIZES = [1, 2, 3, 4, 8, 12, 48, 64, 96, 256]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _run(pd, w, vals, S, kv=None, bt=None, fp8=False):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    scales = dict(k_scale=vals["k_scale"], v_scale=vals["v_scale"]) if fp8 else {}
    out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"] if kv is None else kv,
                                   torch.from_numpy(w.block_table if bt is None else bt).cuda(),
                                   torch.from_numpy(w.seq_lens).cuda(), w.qlen, w.sm_scale,
                                   sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                                   num_kv_splits=S, **scales)
    torch.cuda.synchronize()
    return out, lse


def _cap(pd, w):
    return pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)


@pytest.mark.parametrize("P", PAGE_SIZES + [5, 33])
@pytest.mark.parametrize("S", ["cap", 1, 3])
def test_decode_with_sinks(pd, P, S):
    w = gqa_workload("gqa_sinks", batch=6, len_range=(1, 700), page_size=P, pool="tight",
                     seed_offset=P)
    vals = w.values("cuda", poison=True)
    S = _cap(pd, w) if S == "cap" else S
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what=f"decode P={P} S={S}")


@pytest.mark.parametrize("P", PAGE_SIZES)
@pytest.mark.parametrize("window", [0, 37])
def test_verify_with_window(pd, P, window):
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 600), qlen=4, heads=(32, 8),
                     real_drop=(0, 2), window=window, page_size=P, pool="tight",
                     seed_offset=P + window)
    vals = w.values("cuda", poison=True)
    for S in (1, 4):
        out, lse = _run(pd, w, vals, S)
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, what=f"verify P={P} window={window} S={S}")


@pytest.mark.parametrize("P", PAGE_SIZES)
def test_fp8_cache(pd, P):
    w = gqa_workload("gqa_sinks", batch=6, len_range=(1, 700), qlen=2, real_drop=(0, 1),
                     page_size=P, pool="tight", seed_offset=3 * P)
    vals = w.values("cuda", poison=True, fp8=True)
    for S in (1, 3):
        out, lse = _run(pd, w, vals, S, fp8=True)
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, o_atol=O_ATOL_FP8, what=f"fp8 P={P} S={S}")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("P", [3, 12, 48])
def test_out_of_range_entry_gives_nan(pd, P, fp8):
    """An attended out-of-range entry NaNs its request (every kv head); the
    neighbour request, read by the same waves, stays exact."""
    w = gqa_workload("gqa_sinks", fixed_lens=[300, 300], page_size=P, pool="tight")
    vals = w.values("cuda", poison=True, fp8=fp8)
    bt = w.block_table.copy()
    bt[1, 170 // P] = w.num_pages + 3
    for S in (1, 2):
        out, lse = _run(pd, w, vals, S, bt=bt, fp8=fp8)
        assert torch.all(torch.isnan(out[1].float())) and torch.all(torch.isnan(lse[1]))
        O, L = oracle_gqa(w, vals, requests=[0])
        check_attention(out[:1], lse[:1], O, L, o_atol=O_ATOL_FP8 if fp8 else 2e-2,
                        what=f"valid neighbour P={P}")


def _relayout(w, kv, P2, rng):
    """The workload's cache stored with page size P2 in a shuffled pool, with
    every never-attended slot copied from the source (NaN poison included)."""
    P = w.P
    src = kv.cpu()
    Hkv, row = src.shape[1], src.shape[3]
    cap = [-(-int(L) // P2) for L in w.seq_lens]
    n_pages = sum(cap) + 2
    perm = rng.permutation(n_pages)
    bt = np.full((w.B, max(cap + [1]) + 1), -1, np.int32)
    dst = torch.full((n_pages, Hkv, P2, row), float("nan"), dtype=src.dtype)
    off = 0
    for b, L in enumerate(w.seq_lens):
        L = int(L)
        bt[b, :cap[b]] = perm[off:off + cap[b]]
        off += cap[b]
        if L == 0:
            continue
        pos = np.arange(L)
        rows = src[torch.from_numpy(w.block_table[b, pos // P]).long(), :,
                   torch.from_numpy(pos % P).long()]                       # [L, Hkv, row]
        dst[torch.from_numpy(bt[b, pos // P2]).long(), :, torch.from_numpy(pos % P2).long()] = rows
    return dst.cuda(), bt


@pytest.mark.parametrize("qlen,window", [(1, 0), (3, 50)])
def test_outputs_bitwise_equal_across_page_sizes(pd, qlen, window):
    w = gqa_workload("gqa_verify", batch=6, len_range=(1, 500), qlen=qlen, heads=(32, 8),
                     real_drop=(0, 2) if qlen > 1 else None, window=window, page_size=16,
                     pool="tight", seed_offset=7 + qlen)
    vals = w.values("cuda", poison=True)
    rng = np.random.default_rng(11)
    for S in (1, 3):
        ref_o, ref_l = _run(pd, w, vals, S)
        for P2 in (1, 2, 3, 8, 12, 48, 64, 96):
            kv2, bt2 = _relayout(w, vals["kv"], P2, rng)
            o, l = _run(pd, w, vals, S, kv=kv2, bt=bt2)
            assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), (P2, S)
            assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32)), (P2, S)


# ---------------------------------------------------------------------------
# MLA causal verify
# ---------------------------------------------------------------------------

MLA_PAGE_SIZES = [1, 2, 3, 4, 8, 12, 32, 48, 64, 96]


def _run_mla(pd, w, vals, S, fp8=False, kv=None, bt=None):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    ks = torch.tensor([vals["k_scale"]], dtype=torch.float32, device="cuda") if fp8 else None
    out, lse = pd.paged_verify_mla(vals["q"], vals["kv"] if kv is None else kv,
                                   torch.from_numpy(w.block_table if bt is None else bt).cuda(),
                                   torch.from_numpy(w.seq_lens).cuda(), real, w.qlen, w.sm_scale,
                                   head_dim_v=w.Lv, k_scale=ks, num_kv_splits=S)
    torch.cuda.synchronize()
    return out, lse


def _check_mla(w, vals, out, lse, fp8, what, requests=None):
    O, L = oracle_mla(w, vals, requests=requests, fp8=fp8)
    check_attention(out, lse, O.reshape(out.shape), L, o_atol=O_ATOL_FP8 if fp8 else 2e-2,
                    what=what)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("P", MLA_PAGE_SIZES)
def test_mla_verify(pd, P, fp8):
    w = mla_workload(batch=3, len_range=(1, 400), page_size=P, seed_offset=P)
    vals = w.values("cuda", poison=True, fp8=fp8)
    for S in (1, 3):
        out, lse = _run_mla(pd, w, vals, S, fp8)
        _check_mla(w, vals, out, lse, fp8, f"mla P={P} fp8={fp8} S={S}")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("P", [1, 3, 4, 48, 64])
def test_mla_rows_without_keys(pd, P, fp8):
    """L < qlen and L = 0 at small and large pages, 16 heads (rows past the
    request's 64 rows in the 128-row block)."""
    w = mla_workload(fixed_lens=[2, 5, 40, 0, 97], fixed_real=[2, 4, 39, 0, 95], heads=16,
                     page_size=P)
    vals = w.values("cuda", poison=True, fp8=fp8)
    out, lse = _run_mla(pd, w, vals, 2, fp8)
    _check_mla(w, vals, out, lse, fp8, f"mla keyless P={P}")
    assert torch.all(out[0:2].float() == 0) and torch.all(torch.isneginf(lse[0:2]))
    assert torch.all(out[12:16].float() == 0)                 # L = 0


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("P", [1, 2, 3, 8, 12, 32, 96])
def test_mla_out_of_range_entry_gives_nan(pd, P, fp8):
    """An attended out-of-range entry NaNs its request's rows; every wave
    learns it through the end-of-piece exchange, whichever wave read it."""
    w = mla_workload(fixed_lens=[90, 90], fixed_real=[90, 90], heads=16, page_size=P)
    vals = w.values("cuda", poison=True, fp8=fp8)
    bt = w.block_table.copy()
    bt[1, (70 // P)] = w.num_pages + 3
    for S in (1, 2):
        out, lse = _run_mla(pd, w, vals, S, fp8, bt=bt)
        rows = slice(w.qlen, 2 * w.qlen)
        assert torch.all(torch.isnan(out[rows].float())) and torch.all(torch.isnan(lse[rows]))
        _check_mla(w, vals, out[:w.qlen], lse[:w.qlen], fp8, f"valid neighbour P={P}",
                   requests=[0])


def _relayout_mla(w, kv, P2, rng):
    P = w.P
    src = kv.cpu()
    cap = [-(-int(L) // P2) for L in w.seq_lens]
    n_pages = sum(cap) + 2
    perm = rng.permutation(n_pages)
    bt = np.full((w.B, max(cap + [1]) + 1), -1, np.int32)
    dst = torch.zeros((n_pages, P2, 1, src.shape[-1]), dtype=src.dtype)
    off = 0
    for b, L in enumerate(w.seq_lens):
        L = int(L)
        bt[b, :cap[b]] = perm[off:off + cap[b]]
        off += cap[b]
        pos = np.arange(L)
        if L:
            dst[torch.from_numpy(bt[b, pos // P2]).long(), torch.from_numpy(pos % P2).long()] = \
                src[torch.from_numpy(w.block_table[b, pos // P]).long(), torch.from_numpy(pos % P).long()]
    return dst.cuda(), bt


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_mla_outputs_bitwise_equal_across_page_sizes(pd, fp8):
    w = mla_workload(batch=3, len_range=(1, 300), page_size=16, seed_offset=5)
    vals = w.values("cuda", poison=True, fp8=fp8)
    rng = np.random.default_rng(13)
    for S in (1, 2):
        ref_o, ref_l = _run_mla(pd, w, vals, S, fp8)
        for P2 in (1, 2, 3, 4, 8, 12, 48, 64):
            kv2, bt2 = _relayout_mla(w, vals["kv"], P2, rng)
            o, l = _run_mla(pd, w, vals, S, fp8, kv=kv2, bt=bt2)
            assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), (P2, S)
            assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32)), (P2, S)

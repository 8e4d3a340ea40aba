"""GPU parity of paged_verify_gqa_append: the KV append fused into the GQA
decode / verify call.

The newest qlen tokens' rows are taken out of a seeded workload's cache into
the k_new / v_new sources, and their cache rows are overwritten with NaN
bytes.  The fused call must then
  1. write the rows back: the whole cache equals the workload's again, byte
     for byte (nothing else written);
  2. give the oracle's attention over the workload's cache (the NaN rows
     would poison any row that read them from the cache);
  3. equal paged_kv_append followed by paged_verify_gqa bit for bit (out,
     lse and the cache).
Covers decode and verify (1, 2 and 4 column groups), bf16 and FP8 caches,
page sizes 16, 1, 3, 4, 12 and 64, windows, real lengths, split counts,
requests shorter than qlen or empty, and an invalid block-table entry on a
new token's page (its request turns NaN and that row is not written, as in
the two-call sequence).
"""

import numpy as np
import pytest
import torch

from helpers import O_ATOL_FP8, check_attention, oracle_gqa
from synth import gqa_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

NAN16 = 0x7FC1     # bf16 NaN
NAN8 = 0x7F        # E4M3FN NaN


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _raw(t):
    return t if t.dtype == torch.uint8 else t.view(torch.int16)


def _take_new(w, kv, qlen, bt):
    """(cache with the new tokens' rows NaN, k_new, v_new): token t of
    request b sits at position seq_lens[b] - qlen + t; tokens at negative
    positions or behind an entry outside the pool get random source rows."""
    num_pages, Hkv, P, two_d = kv.shape
    D = two_d // 2
    fp8 = kv.dtype == torch.uint8
    g = torch.Generator(device="cuda").manual_seed(17 + qlen)
    rows = w.B * qlen
    src = torch.randint(0, 256 if fp8 else 1 << 16, (rows, Hkv, two_d), generator=g,
                        device="cuda", dtype=torch.int32)
    src = src.to(torch.uint8) if fp8 else src.to(torch.int16)
    if not fp8:
        src &= 0x3FFF    # finite bf16 values
    cache = kv.clone()
    craw = _raw(cache)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for t in range(qlen):
            pos = L - qlen + t
            if pos < 0 or pos // P >= bt.shape[1]:
                continue
            page = int(bt[b, pos // P])
            if not 0 <= page < num_pages:
                continue
            src[b * qlen + t] = craw[page, :, pos % P, :]
            craw[page, :, pos % P, :] = NAN8 if fp8 else NAN16
    if fp8:
        return cache, src[..., :D], src[..., D:]
    return cache, src[..., :D].view(torch.bfloat16), src[..., D:].view(torch.bfloat16)


def _call(pd, fused, w, vals, cache, k_new, v_new, S, bt):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    bt_d = torch.from_numpy(bt).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    kw = dict(sinks=vals["sinks"], window=w.window, real_seq_lens=real, num_kv_splits=S,
              k_scale=vals.get("k_scale"), v_scale=vals.get("v_scale"))
    if fused:
        out, lse = pd.paged_verify_gqa_append(vals["q"], cache, bt_d, sl, k_new, v_new, w.qlen,
                                              w.sm_scale, **kw)
    else:
        pd.paged_kv_append(cache, bt_d, sl, k_new, v_new, qlen=w.qlen)
        out, lse = pd.paged_verify_gqa(vals["q"], cache, bt_d, sl, w.qlen, w.sm_scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def _check(pd, w, vals, S, fp8=False, bt=None, oracle_rows=True):
    bt = w.block_table if bt is None else bt
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    cache, k_new, v_new = _take_new(w, vals["kv"], w.qlen, bt)
    two = cache.clone()
    out, lse = _call(pd, True, w, vals, cache, k_new, v_new, S, bt)
    out2, lse2 = _call(pd, False, w, vals, two, k_new, v_new, S, bt)
    what = f"qlen={w.qlen} G={w.Hq // w.Hkv} P={w.P} S={S} fp8={fp8}"
    assert torch.equal(_raw(cache), _raw(two)), f"{what}: cache differs from the two-call result"
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), f"{what}: out differs"
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)), f"{what}: lse differs"
    if oracle_rows:
        assert torch.equal(_raw(cache), _raw(vals["kv"])), f"{what}: cache not restored"
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, o_atol=O_ATOL_FP8 if fp8 else 2e-2, what=what)
    return out, lse, cache


CASES = [
    ("decode", dict(batch=7, len_range=(1, 700))),
    ("decode_g16", dict(batch=5, len_range=(1, 600), heads=(64, 4))),
    ("window", dict(batch=6, len_range=(1, 700), window=40)),
    ("verify2", dict(batch=6, len_range=(1, 700), qlen=2, real_drop=(0, 2))),
    ("verify4_cols32", dict(batch=5, len_range=(1, 600), qlen=4, real_drop=(0, 3))),
    ("verify8_cols64", dict(batch=4, len_range=(1, 500), qlen=8, window=100)),
    # 12 tokens x 8 heads: two slices, the second attends the first's new
    # tokens from the cache the first launch wrote
    ("verify12_sliced", dict(batch=4, len_range=(1, 500), qlen=12, real_drop=(0, 2))),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("P", [16, 1, 12, 64])
@pytest.mark.parametrize("S", ["cap", 1, 3])
def test_fused_append_bf16(pd, name, kw, P, S):
    w = gqa_workload("gqa_verify" if "verify" in name else "gqa_sinks", page_size=P,
                     seed_offset=P + len(name), pool="tight", **kw)
    vals = w.values("cuda", poison=True)
    _check(pd, w, vals, S)


@pytest.mark.parametrize("name,kw", [c for c in CASES if c[0] in ("decode", "verify2",
                                                                 "verify4_cols32")],
                         ids=["decode", "verify2", "verify4_cols32"])
@pytest.mark.parametrize("P", [16, 3, 1, 4])
@pytest.mark.parametrize("S", ["cap", 1])
def test_fused_append_fp8(pd, name, kw, P, S):
    w = gqa_workload("gqa_verify" if "verify" in name else "gqa_sinks", page_size=P,
                     seed_offset=3 * P + len(name), pool="tight", **kw)
    vals = w.values("cuda", poison=True, fp8=True)
    _check(pd, w, vals, S, fp8=True)


@pytest.mark.parametrize("S", [1, 2])
def test_short_and_empty_requests(pd, S):
    """Requests with L = 0 and L < qlen: tokens at negative positions are
    neither written nor attended."""
    w = gqa_workload("gqa_verify", fixed_lens=[0, 1, 3, 2, 40, 5, 0, 33], qlen=3,
                     heads=(32, 8), pool="tight")
    vals = w.values("cuda", poison=True)
    _check(pd, w, vals, S)


def test_invalid_entry_on_a_new_page(pd):
    """An entry outside the pool on the page of a request's new token: that
    request's rows are NaN, its row is not written, the rest is exact."""
    w = gqa_workload("gqa_sinks", batch=6, len_range=(40, 400), seed_offset=9, pool="tight")
    vals = w.values("cuda", poison=True)
    bt = w.block_table.copy()
    b = 2
    bt[b, (int(w.seq_lens[b]) - 1) // w.P] = w.num_pages + 7
    for S in (1, 3):
        out, lse, cache = _check(pd, w, vals, S, bt=bt, oracle_rows=False)
        assert torch.isnan(out[b].float()).all() and torch.isnan(lse[b]).all()
        keep = [i for i in range(w.B) if i != b]
        O, L = oracle_gqa(w, vals, keep)
        check_attention(out[keep], lse[keep], O, L, what=f"valid requests S={S}")


def test_full_size_decode_sampled(pd):
    """The sinks configuration at full size (B = 64, Hq 64, Hkv 8, 16-token
    pages), the fused call against the two-call sequence bit for bit and
    sampled requests against the oracle."""
    w = gqa_workload("gqa_sinks")
    vals = w.values("cuda", poison=False)
    S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse, cache = _check(pd, w, vals, S, oracle_rows=False)
    assert torch.equal(_raw(cache), _raw(vals["kv"]))
    sample = [0, 17, 40, 63]
    O, L = oracle_gqa(w, vals, sample)
    check_attention(out[sample], lse[sample], O, L, what="full sinks config, sampled")

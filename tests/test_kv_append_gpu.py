"""GPU parity of paged_kv_append against the oracle, bit for bit.

The whole cache is compared after the append, so a write to any wrong slot
or page, or outside the tokens' rows, shows up.  Covers the GQA HND cache (K
and V from separate, also strided, sources), the MLA latent cache in bf16 and
as FP8 codes, qlen 1..4, requests shorter than qlen, positions past the
block-table row, out-of-range entries, the worked example's placement, and
append followed by decode.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import bits16, check_attention, oracle_gqa
from synth import gqa_workload, mla_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _rand_bits(shape, seed, dtype=torch.int16):
    g = torch.Generator().manual_seed(seed)
    lo, hi = (-32768, 32767) if dtype == torch.int16 else (0, 255)
    return torch.randint(lo, hi, shape, generator=g, dtype=torch.int32).to(dtype)


def _host(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("qlen", [1, 2, 4])
@pytest.mark.parametrize("P", [16, 32])
def test_gqa_cache_append_is_bit_exact(pd, qlen, P):
    w = gqa_workload("gqa_sinks", batch=9, len_range=(0, 300), page_size=P, seed_offset=qlen,
                     pool="tight")
    Hkv, D = w.Hkv, w.D
    cache = _rand_bits((w.num_pages, Hkv, P, 2 * D), 7 + P).view(torch.bfloat16).cuda()
    rows = w.B * qlen
    k = _rand_bits((rows, Hkv, D), 8).view(torch.bfloat16).cuda()
    v = _rand_bits((rows, Hkv, D), 9).view(torch.bfloat16).cuda()
    before = _host(cache)
    sl = w.seq_lens.copy()
    sl[0] = min(qlen - 1, sl[0])                 # a request shorter than qlen
    pd.paged_kv_append(cache, torch.from_numpy(w.block_table).cuda(), torch.from_numpy(sl).cuda(),
                       k, v, qlen=qlen)
    torch.cuda.synchronize()
    want = oracle.kv_append(before, w.block_table, sl, qlen, _host(k), _host(v))
    assert np.array_equal(_host(cache), want)
    assert not np.array_equal(want, before)


def test_strided_sources_and_invalid_entries(pd):
    """K and V as views of one [rows, 2, Hkv, D] tensor; entries -1, past the
    pool, and positions past the table row are skipped."""
    w = gqa_workload("gqa_sinks", batch=6, len_range=(20, 200), seed_offset=3, pool="tight")
    Hkv, D, P = w.Hkv, w.D, w.P
    cache = _rand_bits((w.num_pages, Hkv, P, 2 * D), 11).view(torch.bfloat16).cuda()
    kv_new = _rand_bits((w.B, 2, Hkv, D), 12).view(torch.bfloat16).cuda()
    k, v = kv_new[:, 0], kv_new[:, 1]
    bt = w.block_table.copy()
    sl = w.seq_lens.copy()
    bt[1, (sl[1] - 1) // P] = w.num_pages + 3      # outside the pool
    bt[2, (sl[2] - 1) // P] = -1                   # unallocated
    sl[3] = bt.shape[1] * P + 5                    # past the table row
    before = _host(cache)
    pd.paged_kv_append(cache, torch.from_numpy(bt).cuda(), torch.from_numpy(sl).cuda(), k, v)
    torch.cuda.synchronize()
    want = oracle.kv_append(before, bt, sl, 1, _host(k.contiguous()), _host(v.contiguous()))
    assert np.array_equal(_host(cache), want)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("qlen", [1, 4])
def test_mla_latent_append_is_bit_exact(pd, fp8, qlen):
    w = mla_workload("mla_verify", batch=5, len_range=(1, 200), qlen=qlen, seed_offset=2)
    Lk, P = w.Lk, w.P
    if fp8:
        cache = _rand_bits((w.num_pages, P, 1, Lk), 13, torch.uint8).cuda()
        src = _rand_bits((w.rows, Lk), 14, torch.uint8).cuda()
    else:
        cache = _rand_bits((w.num_pages, P, 1, Lk), 13).view(torch.bfloat16).cuda()
        src = _rand_bits((w.rows, Lk), 14).view(torch.bfloat16).cuda()
    before = _host(cache)
    pd.paged_kv_append(cache, torch.from_numpy(w.block_table).cuda(),
                       torch.from_numpy(w.seq_lens).cuda(), src, qlen=qlen, layout="nhd")
    torch.cuda.synchronize()
    # the oracle's cache view is [pages, H, P, row]: the latent cache with H = 1
    want = oracle.kv_append(before.transpose(0, 2, 1, 3), w.block_table, w.seq_lens, qlen,
                            _host(src)[:, None, :])
    assert np.array_equal(_host(cache), want.transpose(0, 2, 1, 3))


def test_worked_example_placement(pd):
    with open(os.path.join(GOLDEN, "worked_example_append.json")) as f:
        ex = json.load(f)
    P, D = ex["page_size"], 128
    cache = torch.zeros((ex["num_pages"], 1, P, 2 * D), dtype=torch.bfloat16, device="cuda")
    k = torch.full((3, 1, D), 1.0, dtype=torch.bfloat16, device="cuda") * \
        torch.arange(1, 4, device="cuda", dtype=torch.bfloat16)[:, None, None]
    v = -k
    pd.paged_kv_append(cache, torch.tensor(ex["block_table"], dtype=torch.int32, device="cuda"),
                       torch.tensor(ex["seq_lens_after"], dtype=torch.int32, device="cuda"), k, v)
    torch.cuda.synchronize()
    nz = torch.nonzero(cache.float().abs().sum(-1)).cpu().numpy().tolist()
    want = sorted([[p, 0, s] for p, s in zip(ex["new_token_page"], ex["new_token_slot"])])
    assert sorted(nz) == want
    for b, (p, s) in enumerate(zip(ex["new_token_page"], ex["new_token_slot"])):
        assert torch.all(cache[p, 0, s, :D].float() == b + 1)
        assert torch.all(cache[p, 0, s, D:].float() == -(b + 1))


def test_append_then_decode_matches_oracle(pd):
    """Append the current token with paged_kv_append, then decode: the same
    result as the oracle's append followed by the oracle's decode."""
    w = gqa_workload("gqa_sinks", batch=5, len_range=(1, 700), seed_offset=5, pool="tight")
    vals = w.values("cuda", poison=True)
    g = torch.Generator(device="cuda").manual_seed(17)
    k = torch.randn((w.B, w.Hkv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((w.B, w.Hkv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    before = bits16(vals["kv"])
    pd.paged_kv_append(vals["kv"], bt, sl, k, v)
    out, lse = pd.paged_decode_gqa(vals["q"], vals["kv"], bt, sl, w.sm_scale, sinks=vals["sinks"],
                                   num_kv_splits=3)
    torch.cuda.synchronize()
    kv_ref = oracle.kv_append(before, w.block_table, w.seq_lens, 1, bits16(k), bits16(v))
    assert np.array_equal(bits16(vals["kv"]), kv_ref)
    O, L = oracle.gqa_decode(bits16(vals["q"]), kv_ref, w.block_table, w.seq_lens, w.sm_scale,
                             sinks=vals["sinks"].cpu().numpy().astype(np.float64))
    check_attention(out, lse, O, L, what="append+decode")


def test_append_in_a_graph_replays_exactly(pd):
    """Appends captured in a HIP graph (as bench.py times them): every replay,
    with eager work and synchronisations in between, leaves exactly the
    oracle's cache."""
    w = gqa_workload("gqa_sinks", batch=7, len_range=(1, 400), seed_offset=9, pool="tight")
    cache = _rand_bits((w.num_pages, w.Hkv, w.P, 2 * w.D), 21).view(torch.bfloat16).cuda()
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    k = _rand_bits((w.B, w.Hkv, w.D), 22).view(torch.bfloat16).cuda()
    v = _rand_bits((w.B, w.Hkv, w.D), 23).view(torch.bfloat16).cuda()
    before = _host(cache)
    want = oracle.kv_append(before, w.block_table, w.seq_lens, 1, _host(k), _host(v))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            pd.paged_kv_append(cache, bt, sl, k, v)
    torch.cuda.synchronize()
    for rep in range(4):
        cache.copy_(torch.from_numpy(before).view(torch.bfloat16).cuda())   # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_host(cache), want), rep

"""Graph capture of the library's calls (the header states every call is
capture safe: no allocation, no synchronisation, launch shapes from integer
arguments only, no memset).

Each test captures one call with preallocated outputs and workspace, then
replays it several times, changing the query eagerly between replays, and
requires every replay to equal an eager call on the same inputs bit for bit.
"""

import numpy as np
import pytest
import torch

from synth import gqa_workload, mla_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _replays(call, q, eager, n=3, seed=0):
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = call()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(seed)
    for i in range(n):
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype))    # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        want = eager()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), i


@pytest.mark.parametrize("S", [1, 3])
def test_gqa_decode_graph(pd, S):
    w = gqa_workload("gqa_sinks", batch=4, len_range=(1, 500), pool="tight", seed_offset=60)
    vals = w.values("cuda", poison=True)
    bt, sl = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    q = vals["q"].clone()
    ws = pd.alloc_workspace(w.B, w.Hq, max(S, 2), w.D, "cuda")
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")

    def call():
        pd.paged_decode_gqa(q, vals["kv"], bt, sl, w.sm_scale, sinks=vals["sinks"],
                            num_kv_splits=S, workspace=ws, out=out, lse=lse)
        return out, lse

    _replays(call, q, lambda: pd.paged_decode_gqa(q, vals["kv"], bt, sl, w.sm_scale,
                                                  sinks=vals["sinks"], num_kv_splits=S), seed=S)


def test_gqa_verify_fp8_varlen_graph(pd):
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 400), qlen=2, real_drop=(0, 1),
                     page_size=4, pool="tight", seed_offset=61)
    vals = w.values("cuda", poison=True, fp8=True)
    bt, sl = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    real = torch.from_numpy(w.real_seq_lens).cuda()
    cu = torch.tensor([0, 2, 3, 3, 5, 7], dtype=torch.int32, device="cuda")
    q = vals["q"][:7].clone()
    S = 3
    ws = pd.alloc_workspace(7, w.Hq, S, w.D, "cuda")
    out = torch.empty((7, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((7, w.Hq), dtype=torch.float32, device="cuda")
    kw = dict(sinks=vals["sinks"], real_seq_lens=real, num_kv_splits=S,
              k_scale=vals["k_scale"], v_scale=vals["v_scale"])

    def call():
        pd.paged_verify_gqa_varlen(q, vals["kv"], bt, sl, cu, 2, w.sm_scale, workspace=ws,
                                   out=out, lse=lse, **kw)
        return out, lse

    _replays(call, q, lambda: pd.paged_verify_gqa_varlen(q, vals["kv"], bt, sl, cu, 2,
                                                         w.sm_scale, **kw), seed=7)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_mla_verify_graph(pd, fp8):
    w = mla_workload(batch=2, len_range=(50, 300), heads=32, seed_offset=62)
    vals = w.values("cuda", poison=True, fp8=fp8)
    bt, sl = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    real = torch.from_numpy(w.real_seq_lens).cuda()
    ks = torch.tensor([vals["k_scale"]], dtype=torch.float32, device="cuda") if fp8 else None
    q = vals["q"].clone()
    S = 2
    ws = pd.alloc_workspace(w.rows, w.H, S, w.Lv, "cuda")
    out = torch.empty((w.rows, w.H, w.Lv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.rows, w.H), dtype=torch.float32, device="cuda")

    def call():
        pd.paged_verify_mla(q, vals["kv"], bt, sl, real, w.qlen, w.sm_scale, head_dim_v=w.Lv,
                            k_scale=ks, num_kv_splits=S, workspace=ws, out=out, lse=lse)
        return out, lse

    _replays(call, q, lambda: pd.paged_verify_mla(q, vals["kv"], bt, sl, real, w.qlen,
                                                  w.sm_scale, head_dim_v=w.Lv, k_scale=ks,
                                                  num_kv_splits=S), seed=11)

"""GPU parity of paged_verify_gqa_varlen (a query length per request, rows
indexed by cumulative query lengths) against the fp64 oracle.

Covers mixed query lengths including requests with none, lengths shorter
than the request's query count (keyless rows: O = 0, LSE = -inf exactly),
real lengths, windows, sinks, bf16 and FP8 caches and split counts; bitwise
agreement with paged_verify_gqa when every request has the same query
length; and the worked varlen example of "Atención paginada" (query lengths
[10, 3, 1], key lengths [0, 1, 7]).
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import O_ATOL_FP8, bits16, check_attention
from synth import gqa_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _q(total, Hq, D, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((total, Hq, D), generator=g).to(torch.bfloat16).cuda()


def _run(pd, w, vals, q, cu, max_qlen, S, fp8=False):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    scales = dict(k_scale=vals["k_scale"], v_scale=vals["v_scale"]) if fp8 else {}
    out, lse = pd.paged_verify_gqa_varlen(
        q, vals["kv"], torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(),
        torch.from_numpy(np.asarray(cu, np.int32)).cuda(), max_qlen, w.sm_scale,
        sinks=vals["sinks"], window=w.window, real_seq_lens=real, num_kv_splits=S, **scales)
    torch.cuda.synchronize()
    return out, lse


def _oracle(w, vals, q, cu, fp8=False):
    kv = vals["kv"].cpu().numpy() if fp8 else bits16(vals["kv"])
    sinks = None if vals["sinks"] is None else vals["sinks"].cpu().numpy().astype(np.float64)
    kw = {}
    if fp8:
        kw = dict(kv_dtype="fp8_e4m3fn", k_scale=vals["k_scale"].cpu().numpy().astype(np.float64),
                  v_scale=vals["v_scale"].cpu().numpy().astype(np.float64))
    return oracle.gqa_verify_varlen(bits16(q), kv, w.block_table, w.seq_lens, np.asarray(cu),
                                    w.sm_scale, sinks=sinks, window=w.window,
                                    real_seq_lens=w.real_seq_lens, **kw)


def _cu(qlens):
    return np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)


CASES = [
    # (query lengths, key lengths, real drop, heads, window)
    ([2, 0, 1, 2, 1, 2], [300, 50, 1, 2, 700, 33], 1, (64, 8), 0),
    ([4, 1, 3, 0, 2], [90, 5, 2, 40, 400], 2, (32, 8), 37),
    ([16, 1, 7], [200, 3, 100], 0, (8, 8), 0),
    ([3, 3, 1, 2], [1, 64, 65, 500], 1, (20, 4), 5),
    ([8, 2, 0, 5], [400, 9, 30, 120], 1, (64, 8), 0),
    ([6, 13, 1], [77, 260, 3], 0, (16, 4), 50),
]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S", ["cap", 1, 3])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_against_oracle(pd, case, S, fp8):
    qlens, lens, drop, heads, window = CASES[case]
    real = [max(L - drop, 0) for L in lens]
    w = gqa_workload("gqa_verify", fixed_lens=lens, fixed_real=real, heads=heads, window=window,
                     qlen=max(qlens), pool="tight", seed_offset=case)
    vals = w.values("cuda", poison=True, fp8=fp8)
    cu = _cu(qlens)
    q = _q(int(cu[-1]), w.Hq, w.D, 17 + case)
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(max(lens)), w.window)
    out, lse = _run(pd, w, vals, q, cu, max(qlens), S, fp8)
    O, L = _oracle(w, vals, q, cu, fp8)
    check_attention(out, lse, O, L, o_atol=O_ATOL_FP8 if fp8 else 2e-2,
                    what=f"varlen case={case} S={S} fp8={fp8}")


@pytest.mark.parametrize("S", [1, 4])
def test_uniform_query_lengths_match_verify_bitwise(pd, S):
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 600), qlen=2, real_drop=(0, 1),
                     pool="tight", seed_offset=9)
    vals = w.values("cuda", poison=True)
    cu = _cu([2] * w.B)
    o1, l1 = _run(pd, w, vals, vals["q"], cu, 2, S)
    o2, l2 = pd.paged_verify_gqa(vals["q"], vals["kv"], torch.from_numpy(w.block_table).cuda(),
                                 torch.from_numpy(w.seq_lens).cuda(), 2, w.sm_scale,
                                 sinks=vals["sinks"], window=w.window,
                                 real_seq_lens=torch.from_numpy(w.real_seq_lens).cuda(),
                                 num_kv_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("heads", [(4, 4), (16, 4)], ids=["g1", "g4"])
@pytest.mark.parametrize("S", [1, 2])
def test_worked_varlen_example(pd, S, heads):
    """Query lengths [10, 3, 1] over key lengths [0, 1, 7] with the verify
    rule: request 0 has no key (10 keyless rows), request 1's first two rows
    have none, its last row sees key 0, request 2's row sees all 7.  With 4
    query heads per kv head, request 0's 10 rows fill 40 score columns."""
    w = gqa_workload("gqa_verify", fixed_lens=[0, 1, 7], fixed_real=[0, 1, 7], heads=heads,
                     qlen=10, pool="tight", seed_offset=3)
    vals = w.values("cuda", poison=True)
    cu = [0, 10, 13, 14]
    q = _q(14, w.Hq, w.D, 5)
    out, lse = _run(pd, w, vals, q, cu, 10, S)
    O, L = _oracle(w, vals, q, cu)
    check_attention(out, lse, O, L, what=f"worked example S={S}")
    keyless = list(range(0, 12))
    assert torch.all(out[keyless].float() == 0) and torch.all(torch.isneginf(lse[keyless]))
    assert torch.all(torch.isfinite(lse[12:]))


@pytest.mark.parametrize("seed", range(6))
def test_random_query_lengths(pd, seed):
    rng = np.random.default_rng(700 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    max_q = min(64 // G, 12)
    B = int(rng.integers(1, 8))
    qlens = rng.integers(0, max_q + 1, size=B)
    lens = rng.integers(0, 500, size=B)
    Hkv = int(rng.choice([1, 2, 8]))
    w = gqa_workload("gqa_verify", fixed_lens=lens, fixed_real=np.maximum(lens - 1, 0),
                     heads=(G * Hkv, Hkv), window=int(rng.choice([0, 20])),
                     page_size=int(rng.choice([1, 16, 64])), qlen=max(int(qlens.max()), 1),
                     pool="tight", seed_offset=40 + seed)
    vals = w.values("cuda", poison=True)
    cu = _cu(qlens)
    if cu[-1] == 0:
        return
    q = _q(int(cu[-1]), w.Hq, w.D, 80 + seed)
    out, lse = _run(pd, w, vals, q, cu, max(int(qlens.max()), 1), int(rng.choice([1, 3])))
    O, L = _oracle(w, vals, q, cu)
    check_attention(out, lse, O, L, what=f"seed={seed} qlens={list(qlens)} lens={list(lens)}")


@pytest.mark.parametrize("S", [1, 3])
def test_request_past_max_qlen_is_nan(pd, S):
    """A request with more query rows than max_qlen breaks the call's
    contract: all its rows are NaN (O and LSE), as for an invalid
    block-table entry; every other request stays exact.  Covered for a
    request with keys and for one with none."""
    qlens, lens = [3, 1, 5, 2, 4], [200, 40, 300, 90, 0]
    w = gqa_workload("gqa_verify", fixed_lens=lens, fixed_real=lens, heads=(32, 8), qlen=5,
                     pool="tight", seed_offset=61)
    vals = w.values("cuda", poison=True)
    cu = _cu(qlens)
    q = _q(int(cu[-1]), w.Hq, w.D, 62)
    out, lse = _run(pd, w, vals, q, cu, 3, S)
    O, L = _oracle(w, vals, q, cu)
    over = list(range(int(cu[2]), int(cu[3]))) + list(range(int(cu[4]), int(cu[5])))
    keep = [r for r in range(int(cu[-1])) if r not in over]
    assert torch.all(torch.isnan(out[over].float())) and torch.all(torch.isnan(lse[over]))
    check_attention(out[keep], lse[keep], O[keep], L[keep], what=f"past max_qlen S={S}")

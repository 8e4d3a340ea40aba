"""GPU parity of paged_verify_mla against the fp64 oracle (bf16 and FP8 cache).

Every call goes through the C ABI.  Never-attended cache slots are NaN
(bf16 0x7FC0 / fp8 code 0x7F), so any stray read shows.  Besides the
tolerance gates the tests check causal row limits with marker keys (the key
at hi - 1 wins bit-exactly, the NaN at hi never leaks), keyless rows (O = 0,
LSE = -inf exactly), FP8 against the bf16 path on the exactly dequantised
cache (bitwise), physical-page permutation (bitwise), the 3-D cache view,
and the NaN contract for an out-of-range block-table entry.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from helpers import O_ATOL_FP8, bits16, check_attention, oracle_mla
from synth import bf16_bits_from_f32, fp8_codes_from_f32, mla_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _run(pd, w, vals, S, fp8=False, **kw):
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    ks = torch.tensor([vals["k_scale"]], dtype=torch.float32, device="cuda") if fp8 else None
    out, lse = pd.paged_verify_mla(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                                   head_dim_v=w.Lv, k_scale=ks, num_kv_splits=S, **kw)
    torch.cuda.synchronize()
    return out, lse


def _check(w, vals, out, lse, fp8, what):
    O, L = oracle_mla(w, vals, fp8=fp8)
    O = O.reshape(out.shape)
    check_attention(out, lse, O, L, o_atol=O_ATOL_FP8 if fp8 else 2e-2, what=what)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S", [1, 2, 3])
def test_small_causal_cases(pd, S, fp8):
    """Short requests where the causal limit cuts inside tiles and some rows
    have no key at all (L < qlen)."""
    w = mla_workload(fixed_lens=[2, 5, 40, 33, 0, 97], fixed_real=[2, 4, 39, 33, 0, 95],
                     heads=16)
    vals = w.values("cuda", poison=True, fp8=fp8)
    out, lse = _run(pd, w, vals, S, fp8)
    _check(w, vals, out, lse, fp8, f"small S={S}")
    # L = 2, qlen = 4: rows t = 0, 1 have no key
    assert torch.all(out[0:2].float() == 0) and torch.all(torch.isneginf(lse[0:2]))
    assert torch.all(out[16:20].float() == 0)                 # L = 0


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S", ["cap", 1, 2, 4])
def test_reduced_config(pd, S, fp8):
    """The verify configuration's shapes (qlen 4, 128 heads, 576/512 dims,
    page 16, L - U{0,1,2} real lengths) at oracle-sized lengths."""
    w = mla_workload(batch=3, len_range=(100, 700))
    vals = w.values("cuda", poison=True, fp8=fp8)
    if S == "cap":
        S = pd.mla_split_cap(w.B, w.qlen, w.H, int(w.seq_lens.max()))
    out, lse = _run(pd, w, vals, S, fp8)
    _check(w, vals, out, lse, fp8, f"reduced S={S} fp8={fp8}")


@pytest.mark.parametrize("H,qlen", [(128, 4), (16, 2), (32, 1), (64, 3), (16, 1), (8, 1),
                                    (16, 3), (128, 3), (32, 5), (8, 7), (1, 1), (20, 2)])
def test_head_and_qlen_shapes(pd, H, qlen):
    w = mla_workload(batch=2, len_range=(30, 300), heads=H, qlen=qlen)
    vals = w.values("cuda", poison=True)
    for S in (1, 2):
        out, lse = _run(pd, w, vals, S)
        _check(w, vals, out, lse, False, f"H={H} qlen={qlen} S={S}")


@pytest.mark.parametrize("P,H", [(16, 16), (16, 8), (3, 16), (12, 6), (48, 16)])
def test_marker_keys_at_the_row_limit(pd, P, H):
    """q = e0 for every row, so a key's score is its K[0].  Request b targets
    row t = b: the key at hi_t - 1 (the last one row t may attend) carries a
    marker (K[0] = 300) and the key at hi_t (the first one it must not
    attend) a larger decoy (K[0] = 600); all other keys score 0.  Row t must
    return V_marker bit for bit: an off-by-one in either direction returns
    the decoy's or another key's V.  Keys past the request's largest limit
    are NaN and must never leak (keys that some row of the request attends
    hold finite data, as a real cache does)."""
    qlen, Lk, Lv = 4, 576, 512
    L = 53
    B = qlen - 1                       # t = qlen - 1 has no key past its limit
    rng = np.random.default_rng(9)
    pages = -(-L // P)
    n_pages = B * pages + 2
    perm = rng.permutation(n_pages)
    bt = np.full((B, pages + 1), -1, np.int32)
    kv = np.full((n_pages, P, 1, Lk), 0x7FC0, np.uint16)
    markers = []
    for b in range(B):
        bt[b, :pages] = perm[b * pages:(b + 1) * pages]
        hi = L - qlen + 1 + b
        markers.append(hi - 1)
        for j in range(L):
            row = np.zeros(Lk, np.float32)
            row[1:] = rng.integers(-8, 8, Lk - 1)
            row[0] = 300.0 if j == hi - 1 else (600.0 if j == hi else 0.0)
            kv[bt[b, j // P], j % P, 0] = bf16_bits_from_f32(row)
    qv = np.zeros((B * qlen, H, Lk), np.float32)
    qv[..., 0] = 1.0
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    for S in (1, 2):
        out, lse = pd.paged_verify_mla(to_dev(bf16_bits_from_f32(qv)), to_dev(kv),
                                       torch.from_numpy(bt).cuda(),
                                       torch.full((B,), L, dtype=torch.int32).cuda(), None, qlen,
                                       1.0, num_kv_splits=S)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        got = bits16(out)
        for b in range(B):
            r = b * qlen + b                                   # row t = b of request b
            want = kv[bt[b, markers[b] // P], markers[b] % P, 0, :Lv]
            for h in range(H):
                assert np.array_equal(got[r, h], want), (S, b, h)
            np.testing.assert_allclose(lse[r].cpu().numpy(), 300.0, atol=1e-3)


def test_fp8_equals_bf16_on_exactly_dequantised_cache(pd):
    """With a power-of-two k_scale every code * k_scale is exact in bf16, so
    the FP8 path must reproduce the bf16 path bit for bit."""
    w = mla_workload(batch=2, len_range=(200, 500))
    vals = w.values("cuda", poison=True, fp8=True)
    k_scale = 2.0 ** -6
    codes = vals["kv"]
    deq = (codes.view(torch.float8_e4m3fn).float() * k_scale).to(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    real = torch.from_numpy(w.real_seq_lens).cuda()
    ks = torch.tensor([k_scale], dtype=torch.float32, device="cuda")
    for S in (1, 2):
        o8, l8 = pd.paged_verify_mla(vals["q"], codes, bt, sl, real, w.qlen, w.sm_scale,
                                     k_scale=ks, num_kv_splits=S)
        ob, lb = pd.paged_verify_mla(vals["q"], deq, bt, sl, real, w.qlen, w.sm_scale,
                                     num_kv_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o8.view(torch.int16), ob.view(torch.int16))
        assert torch.equal(l8, lb)


def test_page_permutation_invariance_and_3d_view(pd):
    w = mla_workload(batch=2, len_range=(150, 400))
    vals = w.values("cuda", poison=True)
    out1, lse1 = _run(pd, w, vals, 2)
    g = torch.Generator().manual_seed(11)
    perm = torch.randperm(w.num_pages, generator=g)
    kv2 = torch.empty_like(vals["kv"])
    kv2[perm.cuda()] = vals["kv"]
    bt2 = np.where(w.block_table >= 0, perm.numpy()[np.maximum(w.block_table, 0)], -1)
    out2, lse2 = pd.paged_verify_mla(vals["q"], kv2.view(-1, 1, w.Lk),
                                     torch.from_numpy(bt2.astype(np.int32)).cuda(),
                                     torch.from_numpy(w.seq_lens).cuda(),
                                     torch.from_numpy(w.real_seq_lens).cuda(), w.qlen, w.sm_scale,
                                     page_size=w.P, num_kv_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_out_of_range_block_table_entry_gives_nan(pd):
    w = mla_workload(fixed_lens=[90, 90], fixed_real=[90, 90], heads=16)
    vals = w.values("cuda", poison=True)
    bt = w.block_table.copy()
    bt[1, 2] = w.num_pages + 3
    for S in (1, 2):
        out, lse = pd.paged_verify_mla(vals["q"], vals["kv"], torch.from_numpy(bt).cuda(),
                                       torch.from_numpy(w.seq_lens).cuda(),
                                       torch.from_numpy(w.real_seq_lens).cuda(), w.qlen,
                                       w.sm_scale, num_kv_splits=S)
        torch.cuda.synchronize()
        rows = slice(w.qlen, 2 * w.qlen)
        assert torch.all(torch.isnan(out[rows].float())) and torch.all(torch.isnan(lse[rows]))
        O, L = oracle_mla(w, vals, requests=[0])
        check_attention(out[:w.qlen], lse[:w.qlen], O.reshape(out[:w.qlen].shape), L,
                        what="valid neighbour")


@pytest.mark.slow
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_full_size_config_sampled(pd, fp8):
    """The full verify configuration in the benchmark's launch configuration,
    checked on the shortest, the longest and two seeded requests."""
    w = mla_workload()
    vals = w.values("cuda", poison=True, fp8=fp8)
    S = pd.mla_split_cap(w.B, w.qlen, w.H, int(w.seq_lens.max()))
    out, lse = _run(pd, w, vals, S, fp8)
    assert torch.isfinite(out.float()).all()
    order = np.argsort(w.seq_lens)
    pick = sorted({int(order[0]), int(order[-1]), 7, 19})
    O, L = oracle_mla(w, vals, requests=pick, fp8=fp8)
    rows = [b * w.qlen + t for b in pick for t in range(w.qlen)]
    check_attention(out[rows], lse[rows], O.reshape(len(rows), w.H, w.Lv), L,
                    o_atol=O_ATOL_FP8 if fp8 else 2e-2, what=f"mla full S={S} fp8={fp8}")


def test_batch_beyond_one_wave_of_requests(pd):
    """B = 70 requests (the plan scans requests 64 at a time)."""
    w = mla_workload(batch=70, len_range=(0, 40), heads=16, seed_offset=21)
    vals = w.values("cuda", poison=True)
    for S in (1, 2):
        out, lse = _run(pd, w, vals, S)
        _check(w, vals, out, lse, False, f"B=70 S={S}")

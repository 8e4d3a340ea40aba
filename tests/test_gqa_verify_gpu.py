"""GPU parity of paged_verify_gqa (GQA causal verify) against the fp64 oracle.

Every call goes through the C ABI (ctypes binding).  Inputs are seeded
``synth`` workloads with every never-attended cache slot NaN-poisoned.  The
tests cover qlen x G up to 64 columns (one to four score tiles of 16) and
longer verify rows (run as slices of whole tokens),
decode with up to 64 heads per kv head, windows, real lengths, both page sizes and split counts, rows with no key, bit-exact
marker keys at each row's own causal limit and window start, bitwise
agreement with paged_decode_gqa at qlen = 1, invariance to page placement,
determinism, the NaN contract, and the full-size verify configuration on
sampled requests.
"""

import numpy as np
import pytest
import torch

from helpers import bits16, check_attention, oracle_gqa
from synth import bf16_bits_from_f32, gqa_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _dev(w):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    return torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), real


def _run(pd, w, vals, S, kv=None, bt=None):
    bt_d, sl, real = _dev(w)
    if bt is not None:
        bt_d = torch.from_numpy(bt).cuda()
    out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"] if kv is None else kv, bt_d, sl, w.qlen,
                                   w.sm_scale, sinks=vals["sinks"], window=w.window,
                                   real_seq_lens=real, num_kv_splits=S)
    torch.cuda.synchronize()
    return out, lse


# (qlen, (Hq, Hkv)): qlen * G from 2 to 64 (1, 2 or 4 column groups of 16)
SHAPES = [(2, (64, 8)), (4, (32, 8)), (8, (16, 8)), (16, (8, 8)), (3, (20, 4)), (1, (64, 8)),
          (3, (64, 8)), (4, (64, 8)), (8, (64, 8)), (5, (48, 4)), (2, (64, 2)), (64, (8, 8)),
          (7, (18, 2))]


@pytest.mark.parametrize("qlen,heads", SHAPES, ids=[f"q{q}g{h[0] // h[1]}" for q, h in SHAPES])
@pytest.mark.parametrize("S", ["cap", 1, 2, 3, 7])
def test_reduced_verify(pd, qlen, heads, S):
    w = gqa_workload("gqa_verify", batch=6, len_range=(1, 900), qlen=qlen, heads=heads,
                     real_drop=(0, 3), seed_offset=qlen)
    vals = w.values("cuda", poison=True)
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what=f"qlen={qlen} heads={heads} S={S}")


# qlen * G above 64: the library runs slices of whole tokens, one launch each
SLICED = [(9, (64, 8)), (16, (64, 8)), (20, (32, 4)), (3, (64, 1)), (5, (128, 4)), (33, (16, 8))]


@pytest.mark.parametrize("qlen,heads", SLICED, ids=[f"q{q}g{h[0] // h[1]}" for q, h in SLICED])
@pytest.mark.parametrize("S", ["cap", 1, 3])
@pytest.mark.parametrize("window", [0, 37])
def test_sliced_verify(pd, qlen, heads, S, window):
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 700), qlen=qlen, heads=heads,
                     real_drop=(0, 3), window=window or None, seed_offset=qlen + window)
    vals = w.values("cuda", poison=True)
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what=f"sliced qlen={qlen} heads={heads} S={S} W={window}")


def test_sliced_verify_fp8(pd):
    from helpers import O_ATOL_FP8
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 700), qlen=12, heads=(64, 8),
                     real_drop=(0, 2), seed_offset=5)
    vals = w.values("cuda", poison=True, fp8=True)
    for S in (1, 4):
        bt_d, sl, real = _dev(w)
        out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"], bt_d, sl, w.qlen, w.sm_scale,
                                       sinks=vals["sinks"], real_seq_lens=real, num_kv_splits=S,
                                       k_scale=vals["k_scale"], v_scale=vals["v_scale"])
        torch.cuda.synchronize()
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, o_atol=O_ATOL_FP8, what=f"sliced fp8 S={S}")


@pytest.mark.parametrize("qlen,heads", [(4, (32, 8)), (8, (64, 8))])
@pytest.mark.parametrize("window", [1, 5, 100])
@pytest.mark.parametrize("P", [16, 32, 12])
def test_verify_window_and_page_size(pd, window, P, qlen, heads):
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 700), qlen=qlen, heads=heads,
                     real_drop=(0, 2), window=window, page_size=P, seed_offset=window)
    vals = w.values("cuda", poison=True)
    for S in (1, 4):
        out, lse = _run(pd, w, vals, S)
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, what=f"window={window} P={P} S={S}")


@pytest.mark.parametrize("S", [1, 3])
def test_rows_without_keys_are_exact(pd, S):
    """L < qlen and real lengths of 0: the first rows have no key."""
    w = gqa_workload("gqa_verify", fixed_lens=[0, 1, 3, 2, 40, 5], fixed_real=[0, 1, 3, 0, 38, 2],
                     qlen=4, heads=(32, 8))
    vals = w.values("cuda", poison=True)
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what=f"keyless S={S}")
    for b in range(w.B):
        for t in range(w.qlen):
            lo, hi = w.row_range(b, t)
            if hi <= lo:
                r = b * w.qlen + t
                assert torch.all(out[r].float() == 0), (b, t)
                assert torch.all(torch.isneginf(lse[r])), (b, t)


@pytest.mark.parametrize("qlen", [4, 12], ids=["q4", "q12"])
@pytest.mark.parametrize("heads", [(16, 4), (64, 4)], ids=["cols16", "cols64"])
@pytest.mark.parametrize("order", ["last", "first"])
@pytest.mark.parametrize("P", [16, 32])
def test_marker_at_each_rows_limit_is_bit_exact(pd, order, P, heads, qlen):
    """Key j scores 128 * m_j with m_j = j ("last") or 200 - j ("first"), so
    each row's result is exactly the V row of its largest attended key: its
    own last key hi_t - 1, or its first key lo_t (window start).  Keys past a
    row's limit are still attended by the later rows, so a causal-mask slip
    selects a different V row."""
    D, W = 128, 37   # qlen 12 at 16 heads per kv head: three slices of 4 tokens
    Hq, Hkv = heads
    lens = [70, 33, 95, 4]
    B = len(lens)
    rng = np.random.default_rng(11 + P)
    pages_per = [-(-L // P) for L in lens]
    n_pages = sum(pages_per) + 2
    perm = rng.permutation(n_pages)
    maxb = max(pages_per) + 1
    bt = np.full((B, maxb), -1, np.int32)
    kv = np.full((n_pages, Hkv, P, 2 * D), 0x7FC0, np.uint16)
    off = 0
    for b, L in enumerate(lens):
        bt[b, :pages_per[b]] = perm[off:off + pages_per[b]]
        off += pages_per[b]
        for j in range(L):
            row = np.zeros((Hkv, 2 * D), np.float32)
            row[:, 0] = j if order == "last" else 200 - j
            row[:, 1:D] = rng.standard_normal((Hkv, D - 1)) * 0.01
            row[:, D:] = rng.integers(-100, 100, (Hkv, D))
            kv[bt[b, j // P], :, j % P] = bf16_bits_from_f32(row)
    q = np.zeros((B * qlen, Hq, D), np.float32)
    q[:, :, 0] = 1.0
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    window = W if order == "first" else 0
    for S in (1, 3):
        out, lse = pd.paged_verify_gqa(to_dev(bf16_bits_from_f32(q)), to_dev(kv),
                                       torch.from_numpy(bt).cuda(),
                                       torch.tensor(lens, dtype=torch.int32).cuda(), qlen, 128.0,
                                       window=window, num_kv_splits=S)
        torch.cuda.synchronize()
        got = bits16(out)
        for b, L in enumerate(lens):
            for t in range(qlen):
                r = b * qlen + t
                hi = max(L - qlen + 1 + t, 0)
                lo = max(hi - window, 0) if window else 0
                if hi <= lo:
                    assert np.all(got[r] == 0)
                    continue
                j = hi - 1 if order == "last" else lo
                for h in range(Hq):
                    want = kv[bt[b, j // P], h // (Hq // Hkv), j % P, D:]
                    assert np.array_equal(got[r, h], want), (S, b, t, h)


def test_qlen1_matches_decode_bitwise(pd):
    w = gqa_workload("gqa_sinks", batch=7, len_range=(1, 1200))
    vals = w.values("cuda", poison=True)
    bt, sl, _ = _dev(w)
    for S in (1, 3):
        o1, l1 = pd.paged_decode_gqa(vals["q"], vals["kv"], bt, sl, w.sm_scale, sinks=vals["sinks"],
                                     num_kv_splits=S)
        o2, l2 = pd.paged_verify_gqa(vals["q"], vals["kv"], bt, sl, 1, w.sm_scale,
                                     sinks=vals["sinks"], num_kv_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_page_permutation_invariance_and_determinism(pd):
    w = gqa_workload("gqa_verify", batch=5, len_range=(100, 900), qlen=2)
    vals = w.values("cuda", poison=True)
    out1, lse1 = _run(pd, w, vals, 3)
    out1b, lse1b = _run(pd, w, vals, 3)
    assert torch.equal(out1.view(torch.int16), out1b.view(torch.int16)) and torch.equal(lse1, lse1b)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(w.num_pages, generator=g)
    kv2 = torch.empty_like(vals["kv"])
    kv2[perm.cuda()] = vals["kv"]
    bt2 = np.where(w.block_table >= 0, perm.numpy()[np.maximum(w.block_table, 0)], -1)
    out2, lse2 = _run(pd, w, vals, 3, kv=kv2, bt=bt2.astype(np.int32))
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_out_of_range_block_table_entry_gives_nan(pd):
    w = gqa_workload("gqa_verify", fixed_lens=[300, 300], qlen=2, real_drop=(0, 0))
    vals = w.values("cuda", poison=True)
    bt = w.block_table.copy()
    bt[1, 3] = w.num_pages + 5                        # attended entry, out of range
    for S in (1, 2):
        out, lse = _run(pd, w, vals, S, bt=bt)
        assert torch.all(torch.isnan(out[2:4].float()))
        assert torch.all(torch.isnan(lse[2:4]))
        assert not torch.any(torch.isnan(out[0:2].float()))


def test_full_size_verify_config_sampled(pd):
    """The full gqa_verify configuration in the launch configuration bench.py
    times, checked against the oracle on sampled requests."""
    w = gqa_workload("gqa_verify")
    vals = w.values("cuda", poison=True)
    S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    sample = [0, 1, int(np.argmax(w.seq_lens)), int(np.argmin(w.seq_lens)), w.B - 1]
    O, L = oracle_gqa(w, vals, sample)
    rows = [b * w.qlen + t for b in sample for t in range(w.qlen)]
    check_attention(out[rows], lse[rows], O, L, what="gqa_verify full")


@pytest.mark.parametrize("qlen", [1, 2])
def test_batch_beyond_cached_lengths(pd, qlen):
    """B = 300 requests: the plan keeps the first 256 lengths in registers and
    reads the rest in its loops; every request checked against the oracle."""
    w = gqa_workload("gqa_verify", batch=300, len_range=(0, 90), qlen=qlen, heads=(16, 8),
                     real_drop=(0, 1), pool="tight", seed_offset=31 + qlen)
    vals = w.values("cuda", poison=True)
    for S in (1, 3):
        out, lse = _run(pd, w, vals, S)
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, what=f"B=300 qlen={qlen} S={S}")


@pytest.mark.parametrize("heads", [(256, 8), (128, 2), (96, 3)], ids=["g32", "g64", "g32b"])
def test_decode_with_large_head_groups(pd, heads):
    """paged_decode_gqa with more than 16 query heads per kv head (the
    verify kernel's column groups at qlen = 1)."""
    w = gqa_workload("gqa_sinks", batch=5, len_range=(1, 800), heads=heads, seed_offset=heads[0])
    vals = w.values("cuda", poison=True)
    bt, sl, _ = _dev(w)
    for S in (1, 3):
        out, lse = pd.paged_decode_gqa(vals["q"], vals["kv"], bt, sl, w.sm_scale,
                                       sinks=vals["sinks"], num_kv_splits=S)
        torch.cuda.synchronize()
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, what=f"decode heads={heads} S={S}")

"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test ties one oracle function to something the pages or mathematics fix:
the worked block-table example of "Atención paginada", closed forms with a
zero query, brute-force dense attention written with explicit loops, torch's
fp64 scaled_dot_product_attention as a textbook second source, OCP FP8 spot
values, hand-evaluated split caps, invariances (physical page permutation,
split count) and marker keys.  The mutation tests at the end plant plausible
mistakes in the oracle (on the CPU) and check that these pins catch them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from synth import bf16_bits_from_f32, fp8_codes_from_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAN16 = np.uint16(0x7FC0)


def _bf16(x):
    return bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def test_bf16_spot_values():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x4049, 0x0000, 0x8000], np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == np.inf
    assert v[3] == 2.0 ** -133                      # smallest bf16 subnormal
    assert v[4] == 3.140625                         # 0x4049 = 1.5703125 * 2
    assert v[5] == 0.0 and np.signbit(v[6])
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([NAN16]))[0])


def test_bf16_matches_torch_widening():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-30, 30, 4096)).astype(np.float32)
    bits = _bf16(x)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), ref)


def test_fp8_e4m3fn_spot_values():
    t = oracle.fp8_e4m3fn_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0       # largest finite
    assert t[0x08] == 2.0 ** -6                          # smallest normal
    assert t[0x01] == 2.0 ** -9                          # smallest subnormal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x00] == 0.0 and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])       # the only NaNs, no inf
    assert np.sum(np.isnan(t)) == 2 and np.all(np.isfinite(t[~np.isnan(t)]))


def test_fp8_table_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.fp8_bits_to_f64(codes)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


# ---------------------------------------------------------------------------
# row limits
# ---------------------------------------------------------------------------

def test_causal_row_limit_closed_forms():
    # L = 5, qlen = 4, L_real = 4: hi = min(5 - 4 + 1 + t, 4) = [2, 3, 4, 4]
    assert [oracle.row_key_range(5, 4, t, 4)[1] for t in range(4)] == [2, 3, 4, 4]
    # L = 2, qlen = 4: hi = max(t - 1, 0) = [0, 0, 1, 2]
    assert [oracle.row_key_range(2, 4, t)[1] for t in range(4)] == [0, 0, 1, 2]
    # L_real <= 0 empties every row
    assert [oracle.row_key_range(9, 3, t, 0)[1] for t in range(3)] == [0, 0, 0]
    # one decode token: all L keys
    assert oracle.row_key_range(70) == (0, 70)
    # window: the last W keys, or all when W >= L
    assert oracle.row_key_range(70, window=32) == (38, 70)
    assert oracle.row_key_range(70, window=100) == (0, 70)
    assert oracle.row_key_range(0, window=128) == (0, 0)


# ---------------------------------------------------------------------------
# the attention definition
# ---------------------------------------------------------------------------

def _loop_attention(q, K, V, scale, mask, sinks=None):
    """Textbook attention with explicit Python loops (tiny sizes only)."""
    n, m = q.shape[0], K.shape[0]
    O = np.zeros((n, V.shape[1]))
    lse = np.full(n, -np.inf)
    for i in range(n):
        keys = [j for j in range(m) if mask[i, j]]
        if not keys:
            continue
        x = {j: scale * sum(q[i, d] * K[j, d] for d in range(q.shape[1])) for j in keys}
        mx = max(x.values())
        w = {j: math.exp(x[j] - mx) for j in keys}
        s = sum(w.values())
        den = s + (math.exp(sinks[i] - mx) if sinks is not None else 0.0)
        for d in range(V.shape[1]):
            O[i, d] = sum(w[j] * V[j, d] for j in keys) / den
        lse[i] = mx + math.log(s)
    return O, lse


def test_attend_matches_loop_brute_force():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 8))
    K = rng.standard_normal((11, 8))
    V = rng.standard_normal((11, 5))
    sinks = rng.standard_normal(3)
    full = np.ones((3, 11), dtype=bool)
    for sk in (None, sinks):
        O, lse = oracle.attend(q, K, V, 0.37, sk)
        O2, lse2 = _loop_attention(q, K, V, 0.37, full, sk)
        np.testing.assert_allclose(O, O2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((40, 16))
    V = rng.standard_normal((40, 16))
    O, _ = oracle.attend(q, K, V, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        scale=0.25)[0].numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_attend_uniform_closed_form_and_empty():
    rng = np.random.default_rng(3)
    V = rng.standard_normal((9, 4))
    O, lse = oracle.attend(np.zeros((2, 6)), rng.standard_normal((9, 6)), V, 1.0,
                           np.array([-np.inf, 0.7]))
    np.testing.assert_allclose(O[0], V.mean(0), atol=1e-15)
    np.testing.assert_allclose(O[1], V.sum(0) / (9 + math.exp(0.7)), atol=1e-15)
    np.testing.assert_allclose(lse, [math.log(9)] * 2, atol=1e-15)
    O, lse = oracle.attend(np.ones((2, 6)), np.zeros((0, 6)), np.zeros((0, 4)), 1.0,
                           np.array([0.5, 0.5]))
    assert np.all(O == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------------------
# GQA paged decode
# ---------------------------------------------------------------------------

def _worked_example():
    with open(os.path.join(GOLDEN, "worked_example_block_table.json")) as f:
        return json.load(f)


def _page_id_cache(ex, seq_lens, D=128):
    """Cache whose V dim 0 holds the physical page id at attended slots;
    everything never attended is NaN."""
    P, n_pages = ex["page_size"], ex["num_pages"]
    kv = np.full((n_pages, 1, P, 2 * D), NAN16, dtype=np.uint16)
    rng = np.random.default_rng(4)
    bt = np.asarray(ex["block_table"], np.int64)
    for b, L in enumerate(seq_lens):
        for j in range(L):
            page, slot = bt[b, j // P], j % P
            kv[page, 0, slot, :D] = _bf16(rng.standard_normal(D))
            kv[page, 0, slot, D:] = _bf16(rng.standard_normal(D))
            kv[page, 0, slot, D] = _bf16([float(page)])[0]
    return kv


@pytest.mark.parametrize("reading", ["reading_L", "reading_L_plus_1"])
def test_gqa_worked_block_table_example(reading):
    ex = _worked_example()
    lens = ex[reading]["seq_lens"]
    kv = _page_id_cache(ex, lens)
    for p in ex["unreferenced_pages"]:
        assert np.all(kv[p] == NAN16)
    q = np.zeros((3, 8, 128), np.uint16)                 # q = 0: uniform softmax
    O, lse = oracle.gqa_decode(q, kv, np.asarray(ex["block_table"], np.int32),
                               np.asarray(lens, np.int32), 1.0 / math.sqrt(128))
    want0 = [float(Fraction(s)) for s in ex[reading]["o_dim0"]]
    for b in range(3):
        np.testing.assert_allclose(O[b, :, 0], want0[b], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], math.log(lens[b]), rtol=0, atol=1e-14)
    assert np.all(np.isfinite(O))


def _rand_gqa(rng, B, Hq, Hkv, D, P, lens, extra_pages=3, sinks=False):
    """Tiny random GQA inputs with a shuffled pool and NaN everywhere unattended."""
    pages_per = [-(-L // P) for L in lens]
    n_pages = sum(pages_per) + extra_pages
    perm = rng.permutation(n_pages)
    max_blocks = max(pages_per + [1]) + 2
    bt = np.full((B, max_blocks), -1, np.int32)
    kv = np.full((n_pages, Hkv, P, 2 * D), NAN16, np.uint16)
    off = 0
    for b, L in enumerate(lens):
        bt[b, :pages_per[b]] = perm[off:off + pages_per[b]]
        off += pages_per[b]
        for j in range(L):
            kv[bt[b, j // P], :, j % P, :] = _bf16(rng.standard_normal((Hkv, 2 * D)))
    q = _bf16(rng.standard_normal((B, Hq, D)))
    sk = rng.standard_normal(Hq) if sinks else None
    return q, kv, bt, np.asarray(lens, np.int32), sk


def test_gqa_matches_dense_loop_brute_force():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, P = 2, 4, 2, 8, 4
    lens = [7, 10]
    q, kv, bt, sl, sk = _rand_gqa(rng, B, Hq, Hkv, D, P, lens, sinks=True)
    O, lse = oracle.gqa_decode(q, kv, bt, sl, 0.3, sinks=sk, window=6)
    qf = oa.bf16_bits_to_f64(q)
    for b in range(B):
        L = lens[b]
        # contiguous copy of the request's cache, built position by position
        rows = np.stack([oa.bf16_bits_to_f64(kv[bt[b, j // P], :, j % P, :]) for j in range(L)])
        for kvh in range(Hkv):
            hs = slice(2 * kvh, 2 * kvh + 2)
            mask = np.zeros((2, L), bool)
            mask[:, max(L - 6, 0):] = True
            O2, lse2 = _loop_attention(qf[b, hs], rows[:, kvh, :D], rows[:, kvh, D:], 0.3,
                                       mask, sk[hs])
            np.testing.assert_allclose(O[b, hs], O2, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[b, hs], lse2, atol=1e-13, rtol=0)


def test_gqa_page_permutation_invariance_is_bitwise():
    rng = np.random.default_rng(6)
    q, kv, bt, sl, sk = _rand_gqa(rng, 3, 8, 2, 16, 4, [5, 13, 9], sinks=True)
    O, lse = oracle.gqa_decode(q, kv, bt, sl, 0.25, sinks=sk)
    perm = rng.permutation(kv.shape[0])                    # new physical placement
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    O2, lse2 = oracle.gqa_decode(q, kv2, bt2, sl, 0.25, sinks=sk)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)


def test_gqa_marker_keys_select_exact_value():
    """A key whose score beats every other by >= 200 takes all the weight, so
    O equals that key's V exactly; checked at every position of every page
    (first and last slot included)."""
    P, D, L = 4, 8, 11
    rng = np.random.default_rng(7)
    for target in range(L):
        q, kv, bt, sl, _ = _rand_gqa(rng, 1, 2, 1, D, P, [L])
        qv = np.zeros((1, 2, D), np.float32)
        qv[..., 0] = 1.0
        q = _bf16(qv)
        for j in range(L):
            page, slot = bt[0, j // P], j % P
            kv[page, 0, slot, 0] = _bf16([256.0 if j == target else 0.0])[0]
            kv[page, 0, slot, D:] = _bf16(rng.integers(-50, 50, D).astype(np.float32))
        O, lse = oracle.gqa_decode(q, kv, bt, sl, 1.0)
        want = oa.bf16_bits_to_f64(kv[bt[0, target // P], 0, target % P, D:])
        # the other keys carry weight <= exp(-256): far below any bf16 ulp
        np.testing.assert_allclose(O[0, 0], want, rtol=0, atol=1e-100)
        np.testing.assert_allclose(O[0, 1], want, rtol=0, atol=1e-100)
        np.testing.assert_allclose(lse[0], 256.0, atol=1e-12)


def test_gqa_window_special_cases():
    rng = np.random.default_rng(8)
    q, kv, bt, sl, sk = _rand_gqa(rng, 2, 4, 1, 8, 4, [9, 14], sinks=True)
    full = oracle.gqa_decode(q, kv, bt, sl, 0.5, sinks=sk)
    wide = oracle.gqa_decode(q, kv, bt, sl, 0.5, sinks=sk, window=14)
    np.testing.assert_array_equal(full[0], wide[0])
    np.testing.assert_array_equal(full[1], wide[1])
    O1, lse1 = oracle.gqa_decode(q, kv, bt, sl, 0.5, window=1)
    qf = oa.bf16_bits_to_f64(q)
    for b, L in enumerate([9, 14]):
        last = oa.bf16_bits_to_f64(kv[bt[b, (L - 1) // 4], 0, (L - 1) % 4])
        np.testing.assert_allclose(O1[b], np.broadcast_to(last[8:], (4, 8)), atol=1e-15)
        np.testing.assert_allclose(lse1[b], 0.5 * qf[b] @ last[:8], atol=1e-13)


def test_gqa_sink_special_cases():
    rng = np.random.default_rng(9)
    q, kv, bt, sl, sk = _rand_gqa(rng, 2, 4, 2, 8, 4, [6, 11], sinks=True)
    none = oracle.gqa_decode(q, kv, bt, sl, 0.5)
    neg = oracle.gqa_decode(q, kv, bt, sl, 0.5, sinks=np.full(4, -np.inf))
    np.testing.assert_array_equal(none[0], neg[0])
    np.testing.assert_array_equal(none[1], neg[1])
    q0 = np.zeros_like(q)
    O, lse = oracle.gqa_decode(q0, kv, bt, sl, 0.5, sinks=sk)
    for b, L in enumerate([6, 11]):
        V = np.stack([oa.bf16_bits_to_f64(kv[bt[b, j // 4], :, j % 4, 8:]) for j in range(L)])
        for h in range(4):
            np.testing.assert_allclose(O[b, h], V[:, h // 2].sum(0) / (L + math.exp(sk[h])),
                                       atol=1e-14)
            assert abs(lse[b, h] - math.log(L)) < 1e-14


def test_gqa_empty_request_zero_output():
    rng = np.random.default_rng(10)
    q, kv, bt, sl, sk = _rand_gqa(rng, 3, 4, 1, 8, 4, [0, 5, 0], sinks=True)
    O, lse = oracle.gqa_decode(q, kv, bt, sl, 0.5, sinks=sk)
    for b in (0, 2):
        assert np.all(O[b] == 0.0) and np.all(lse[b] == -np.inf)
    assert np.all(np.isfinite(O[1])) and np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------------------
# split partials and the merge
# ---------------------------------------------------------------------------

def _edges_factory(S, rng, aligned_to=1):
    def edges(b, lo, hi):
        if S == 1:
            return [lo, hi]
        cuts = sorted(rng.integers(lo, hi + 1, size=S - 1).tolist()) if hi > lo else [lo] * (S - 1)
        if aligned_to > 1:
            cuts = sorted(min(max(lo, (c // aligned_to) * aligned_to), hi) for c in cuts)
        return [lo] + cuts + [hi]
    return edges


@pytest.mark.parametrize("S", [1, 2, 3, 7, 16])
def test_split_merge_equals_one_split(S):
    rng = np.random.default_rng(11 + S)
    q, kv, bt, sl, sk = _rand_gqa(rng, 3, 8, 2, 16, 4, [1, 23, 40], sinks=True)
    O, lse = oracle.gqa_decode(q, kv, bt, sl, 0.3, sinks=sk, window=30)
    for aligned in (1, 4):
        Op, lp = oracle.gqa_partials(q, kv, bt, sl, 0.3, _edges_factory(S, rng, aligned),
                                     window=30)
        Om, lm = oracle.merge_partials(Op, lp, sinks=sk)
        np.testing.assert_allclose(Om, O, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lm, lse, atol=1e-12, rtol=0)


def test_lse_consistency_of_partials():
    rng = np.random.default_rng(12)
    q, kv, bt, sl, _ = _rand_gqa(rng, 2, 4, 1, 16, 4, [19, 33])
    O, lse = oracle.gqa_decode(q, kv, bt, sl, 0.3)
    Op, lp = oracle.gqa_partials(q, kv, bt, sl, 0.3, _edges_factory(5, rng))
    # logsumexp of the split LSEs is the one-split LSE (scipy as a 2nd source)
    from scipy.special import logsumexp
    np.testing.assert_allclose(logsumexp(lp, axis=-1), lse, atol=1e-12)
    # sum_s exp(lse_s - LSE) O_s is the one-split O
    w = np.exp(lp - lse[..., None])
    np.testing.assert_allclose((w[..., None] * Op).sum(-2), O, atol=1e-12)


def test_merge_all_empty_and_nan_in_empty_slots():
    Op = np.full((2, 3, 4, 5), np.nan)
    lp = np.full((2, 3, 4), -np.inf)
    O, lse = oracle.merge_partials(Op, lp, sinks=np.zeros(3))
    assert np.all(O == 0) and np.all(lse == -np.inf)
    lp[0, 0, 2] = 0.5
    Op[0, 0, 2] = 1.0
    O, lse = oracle.merge_partials(Op, lp)
    np.testing.assert_array_equal(O[0, 0], np.ones(5))
    assert lse[0, 0] == 0.5 and np.all(O[1] == 0)


# ---------------------------------------------------------------------------
# GQA causal verify
# ---------------------------------------------------------------------------

def _rand_gqa_verify(rng, lens, qlen, Hq, Hkv, D, P):
    """Tiny random GQA verify inputs: q has qlen rows per request."""
    q1, kv, bt, sl, sk = _rand_gqa(rng, len(lens), Hq, Hkv, D, P, lens, sinks=True)
    q = _bf16(rng.standard_normal((len(lens) * qlen, Hq, D)))
    return q, kv, bt, sl, sk


def test_gqa_verify_qlen1_is_decode():
    rng = np.random.default_rng(21)
    lens = [7, 10, 0, 3]
    q, kv, bt, sl, sk = _rand_gqa(rng, 4, 8, 2, 8, 4, lens, sinks=True)
    for window in (0, 4):
        O, lse = oracle.gqa_decode(q, kv, bt, sl, 0.3, sinks=sk, window=window)
        O2, lse2 = oracle.gqa_verify(q, kv, bt, sl, 1, 0.3, sinks=sk, window=window)
        assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


def test_gqa_verify_rows_are_prefix_decodes():
    """Row t of a request is a one-token decode over the request's first
    hi_t keys (limits worked out by hand for L = [9, 5, 2], L_real = [7, 5, 2],
    qlen = 3), with its own sliding window."""
    rng = np.random.default_rng(22)
    lens, real, qlen, Hq, Hkv, D, P = [9, 5, 2], [7, 5, 2], 3, 4, 2, 8, 4
    his = [[7, 7, 7], [3, 4, 5], [0, 1, 2]]
    q, kv, bt, sl, sk = _rand_gqa_verify(rng, lens, qlen, Hq, Hkv, D, P)
    for window in (0, 2):
        O, lse = oracle.gqa_verify(q, kv, bt, sl, qlen, 0.3, sinks=sk, window=window,
                                   real_seq_lens=np.array(real))
        for b in range(3):
            for t in range(qlen):
                r = b * qlen + t
                O1, lse1 = oracle.gqa_decode(q[r:r + 1], kv, bt[b:b + 1],
                                             np.array([his[b][t]]), 0.3, sinks=sk, window=window)
                np.testing.assert_array_equal(O[r], O1[0])
                np.testing.assert_array_equal(lse[r], lse1[0])
    # rows with no key: O = 0, LSE = -inf
    assert np.all(O[6] == 0) and np.all(lse[6] == -np.inf)


def test_gqa_verify_matches_causal_dense_brute_force():
    _check_gqa_verify_brute_force(np.random.default_rng(23), [11, 6], 4, 4, 2, 8, 4, 5)


def _check_gqa_verify_brute_force(rng, lens, qlen, Hq, Hkv, D, P, W):
    q, kv, bt, sl, sk = _rand_gqa_verify(rng, lens, qlen, Hq, Hkv, D, P)
    O, lse = oracle.gqa_verify(q, kv, bt, sl, qlen, 0.3, sinks=sk, window=W)
    qf = oa.bf16_bits_to_f64(q)
    for b, L in enumerate(lens):
        rows = np.stack([oa.bf16_bits_to_f64(kv[bt[b, j // P], :, j % P, :]) for j in range(L)])
        for t in range(qlen):
            r = b * qlen + t
            last = L - qlen + t          # the token's own position: it sees keys 0..last
            for kvh in range(Hkv):
                hs = slice(2 * kvh, 2 * kvh + 2)
                mask = np.zeros((2, L), bool)
                mask[:, max(last + 1 - W, 0):last + 1] = True
                O2, lse2 = _loop_attention(qf[r, hs], rows[:, kvh, :D], rows[:, kvh, D:], 0.3,
                                           mask, sk[hs])
                np.testing.assert_allclose(O[r, hs], O2, atol=1e-13, rtol=0)
                np.testing.assert_allclose(lse[r, hs], lse2, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# MLA causal verify
# ---------------------------------------------------------------------------

def _rand_mla(rng, lens, qlen, H, Lk, P, fp8=False):
    B = len(lens)
    pages_per = [-(-max(L, 0) // P) for L in lens]
    n_pages = sum(pages_per) + 2
    perm = rng.permutation(n_pages)
    bt = np.full((B, max(pages_per + [1]) + 1), -1, np.int32)
    vals = np.full((n_pages, P, 1, Lk), np.nan, np.float32)
    off = 0
    for b, L in enumerate(lens):
        bt[b, :pages_per[b]] = perm[off:off + pages_per[b]]
        off += pages_per[b]
        for j in range(L):
            vals[bt[b, j // P], j % P, 0] = rng.standard_normal(Lk).astype(np.float32)
    q = _bf16(0.5 * rng.standard_normal((B * qlen, H, Lk)))
    if fp8:
        codes = np.where(np.isnan(vals), np.uint8(0x7F),
                         fp8_codes_from_f32(np.nan_to_num(vals * 16.0)))
        return q, codes, bt
    return q, _bf16(vals), bt


def test_mla_matches_causal_dense_brute_force():
    _check_mla_brute_force(np.random.default_rng(13), [9, 3, 6], [8, 3, 4], 3, 2, 12, 8, 4)


def _check_mla_brute_force(rng, lens, real, qlen, H, Lk, Lv, P):
    q, kv, bt = _rand_mla(rng, lens, qlen, H, Lk, P)
    O, lse = oracle.mla_verify(q, kv, bt, np.array(lens), np.array(real), qlen, 0.3, Lv)
    qf = oa.bf16_bits_to_f64(q)
    for b, L in enumerate(lens):
        lat = np.stack([oa.bf16_bits_to_f64(kv[bt[b, j // P], j % P, 0]) for j in range(L)])
        for t in range(qlen):
            r = b * qlen + t
            hi = max(min(L - qlen + 1 + t, real[b]), 0)
            mask = np.zeros((H, L), bool)
            mask[:, :hi] = True
            O2, lse2 = _loop_attention(qf[r], lat, lat[:, :Lv], 0.3, mask)
            np.testing.assert_allclose(O[r], O2, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[r], lse2, atol=1e-13, rtol=0)


def test_mla_marker_at_row_limit_and_empty_rows():
    """Row t attends exactly [0, hi): a marker at hi - 1 wins, a NaN at hi
    (just past the limit) never reaches the output; rows with hi = 0 give
    O = 0 and LSE = -inf."""
    rng = np.random.default_rng(14)
    qlen, H, Lk, Lv, P = 4, 2, 8, 4, 4
    L = 2                                                   # hi = [0, 0, 1, 2]
    q, kv, bt = _rand_mla(rng, [L], qlen, H, Lk, P)
    O, lse = oracle.mla_verify(q, kv, bt, np.array([L]), None, qlen, 0.5, Lv)
    assert np.all(O[0:2] == 0) and np.all(lse[0:2] == -np.inf)
    assert np.all(np.isfinite(O[2:]))
    L = 7
    q, kv, bt = _rand_mla(rng, [L], qlen, H, Lk, P)
    qv = np.zeros((qlen, H, Lk), np.float32)
    qv[..., 0] = 1.0
    q = _bf16(qv)
    for t in range(qlen):
        hi = L - qlen + 1 + t
        kv2 = kv.copy()
        for j in range(L):
            kv2[bt[0, j // P], j % P, 0, 0] = _bf16([300.0 if j == hi - 1 else 0.0])[0]
        if hi < L:
            kv2[bt[0, hi // P], hi % P, 0, :] = NAN16
        O, _ = oracle.mla_verify(q, kv2, bt, np.array([L]), None, qlen, 1.0, Lv)
        want = oa.bf16_bits_to_f64(kv2[bt[0, (hi - 1) // P], (hi - 1) % P, 0, :Lv])
        np.testing.assert_allclose(O[t, 0], want, rtol=0, atol=1e-100)


def test_mla_fp8_equals_bf16_of_dequantised_cache():
    rng = np.random.default_rng(15)
    lens, qlen, H, Lk, Lv, P = [10, 5], 2, 3, 16, 8, 4
    q, codes, bt = _rand_mla(rng, lens, qlen, H, Lk, P, fp8=True)
    k_scale = 0.0625                                        # power of two: exact
    deq = np.where(codes == 0x7F, np.float32(np.nan),
                   (oa.fp8_bits_to_f64(codes) * k_scale).astype(np.float32))
    O8, l8 = oracle.mla_verify(q, codes, bt, np.array(lens), None, qlen, 0.4, Lv,
                               kv_dtype="fp8_e4m3fn", k_scale=k_scale)
    Ob, lb = oracle.mla_verify(q, _bf16(deq), bt, np.array(lens), None, qlen, 0.4, Lv)
    np.testing.assert_array_equal(O8, Ob)
    np.testing.assert_array_equal(l8, lb)


def test_mla_3d_cache_view_is_the_same_cache():
    rng = np.random.default_rng(16)
    q, kv, bt = _rand_mla(rng, [6, 9], 2, 2, 8, 4)
    a = oracle.mla_verify(q, kv, bt, np.array([6, 9]), None, 2, 0.5, 4)
    b = oracle.mla_verify(q, kv.reshape(-1, 1, 8), bt, np.array([6, 9]), None, 2, 0.5, 4,
                          page_size=4)
    np.testing.assert_array_equal(a[0], b[0])


# ---------------------------------------------------------------------------
# variable query length per request ("Atención paginada", Ruta Varlen)
# ---------------------------------------------------------------------------

def test_varlen_row_requests_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_varlen.json")))
    cu = np.concatenate([[0], np.cumsum(ex["query_lengths"])])
    assert list(cu) == ex["cu_seq_lens_q"]
    assert list(oracle.varlen_row_requests(ex["cu_seq_lens_q"])) == ex["q_request_index"]
    assert max(np.diff(cu)) == ex["max_length_q"]


def test_gqa_verify_varlen_uniform_qlen_is_verify():
    rng = np.random.default_rng(90)
    lens, qlen = [11, 6, 0, 30], 3
    q, kv, bt, sl, sk = _rand_gqa_verify(rng, lens, qlen, 4, 2, 8, 4)
    cu = np.arange(len(lens) + 1) * qlen
    for window in (0, 5):
        a = oracle.gqa_verify(q, kv, bt, sl, qlen, 0.3, sinks=sk, window=window,
                              real_seq_lens=np.array([10, 6, 0, 29]))
        b = oracle.gqa_verify_varlen(q, kv, bt, sl, cu, 0.3, sinks=sk, window=window,
                                     real_seq_lens=np.array([10, 6, 0, 29]))
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_gqa_verify_varlen_matches_causal_dense_brute_force():
    """Per-request query lengths [2, 0, 4, 1] (the second request has no
    query row): row t of request b sees keys 0 .. L - qlen_b + t, the last
    W of them, through the block table."""
    rng = np.random.default_rng(91)
    lens, qlens, Hq, Hkv, D, P, W = [9, 5, 13, 3], [2, 0, 4, 1], 4, 2, 8, 4, 6
    q1, kv, bt, sl, sk = _rand_gqa(rng, len(lens), Hq, Hkv, D, P, lens, sinks=True)
    cu = np.concatenate([[0], np.cumsum(qlens)])
    q = _bf16(rng.standard_normal((int(cu[-1]), Hq, D)))
    O, lse = oracle.gqa_verify_varlen(q, kv, bt, sl, cu, 0.3, sinks=sk, window=W)
    qf = oa.bf16_bits_to_f64(q)
    req = oracle.varlen_row_requests(cu)
    for r in range(int(cu[-1])):
        b = int(req[r])
        t = r - int(cu[b])
        L = lens[b]
        rows = np.stack([oa.bf16_bits_to_f64(kv[bt[b, j // P], :, j % P, :]) for j in range(L)])
        last = L - qlens[b] + t          # the token's own position
        for kvh in range(Hkv):
            hs = slice(2 * kvh, 2 * kvh + 2)
            mask = np.zeros((2, L), bool)
            mask[:, max(last + 1 - W, 0):max(last + 1, 0)] = True
            O2, lse2 = _loop_attention(qf[r, hs], rows[:, kvh, :D], rows[:, kvh, D:], 0.3,
                                       mask, sk[hs])
            np.testing.assert_allclose(O[r, hs], O2, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[r, hs], lse2, atol=1e-13, rtol=0)


# ---------------------------------------------------------------------------
# general page sizes ("vllm.v1.attention.ops.triton_decode_attention": the
# module supports any page size >= 1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 3, 8, 64])
def test_gqa_verify_brute_force_at_page_size(P):
    # lengths below, at and past one page, several pages, and a window
    _check_gqa_verify_brute_force(np.random.default_rng(60 + P), [13, 1, 70], 2, 4, 2, 8, P, 9)


@pytest.mark.parametrize("P", [1, 3, 32])
def test_mla_brute_force_at_page_size(P):
    _check_mla_brute_force(np.random.default_rng(70 + P), [9, 2, 40], [8, 2, 39], 3, 2, 12, 8, P)


def _relayout_gqa(kv, bt, lens, P2, rng):
    """The same logical cache stored with page size P2 in a shuffled pool."""
    P = kv.shape[2]
    pages_per = [-(-L // P2) for L in lens]
    n_pages = sum(pages_per) + 1
    perm = rng.permutation(n_pages)
    bt2 = np.full((len(lens), max(pages_per + [1]) + 1), -1, np.int32)
    kv2 = np.full((n_pages, kv.shape[1], P2, kv.shape[3]), NAN16, np.uint16)
    off = 0
    for b, L in enumerate(lens):
        bt2[b, :pages_per[b]] = perm[off:off + pages_per[b]]
        off += pages_per[b]
        for j in range(L):
            kv2[bt2[b, j // P2], :, j % P2] = kv[bt[b, j // P], :, j % P]
    return kv2, bt2


def test_gqa_result_does_not_depend_on_page_size():
    """One logical cache laid out with page sizes 1, 2, 5, 16 and 64 gives
    bitwise the same result: the page size only changes where a key lives."""
    rng = np.random.default_rng(80)
    lens, qlen = [37, 4, 0, 20], 2
    q, kv, bt, sl, sk = _rand_gqa_verify(rng, lens, qlen, 4, 2, 8, 4)
    ref = oracle.gqa_verify(q, kv, bt, sl, qlen, 0.3, sinks=sk, window=11)
    for P2 in (1, 2, 5, 16, 64):
        kv2, bt2 = _relayout_gqa(kv, bt, lens, P2, rng)
        got = oracle.gqa_verify(q, kv2, bt2, sl, qlen, 0.3, sinks=sk, window=11)
        np.testing.assert_array_equal(ref[0], got[0])
        np.testing.assert_array_equal(ref[1], got[1])


def test_mla_result_does_not_depend_on_page_size():
    rng = np.random.default_rng(81)
    lens, real, qlen, Lk = [21, 3], [20, 3], 2, 12
    q, kv, bt = _rand_mla(rng, lens, qlen, 2, Lk, 4)
    ref = oracle.mla_verify(q, kv, bt, np.array(lens), np.array(real), qlen, 0.3, 8)
    for P2 in (1, 3, 8, 32):
        pages_per = [-(-L // P2) for L in lens]
        perm = rng.permutation(sum(pages_per))
        bt2 = np.full((len(lens), max(pages_per)), -1, np.int32)
        kv2 = np.full((sum(pages_per), P2, 1, Lk), NAN16, np.uint16)
        off = 0
        for b, L in enumerate(lens):
            bt2[b, :pages_per[b]] = perm[off:off + pages_per[b]]
            off += pages_per[b]
            for j in range(L):
                kv2[bt2[b, j // P2], j % P2] = kv[bt[b, j // 4], j % 4]
        got = oracle.mla_verify(q, kv2, bt2, np.array(lens), np.array(real), qlen, 0.3, 8)
        np.testing.assert_array_equal(ref[0], got[0])
        np.testing.assert_array_equal(ref[1], got[1])


# ---------------------------------------------------------------------------
# static split cap
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("args,kw,want", [
    ((70, 3, 1, 1, 256, 1), {}, 2),
    ((100000, 300, 1, 1, 256, 1), dict(max_splits=8), 4),
    ((4096, 1, 1, 32, 256, 32), {}, 64),
    ((64, 1, 1, 32, 256, 32), {}, 1),
    ((16384, 4, 4, 128, 256, 64), dict(max_splits=16), 8),
    ((16384, 32, 4, 128, 256, 64), dict(max_splits=16), 1),
])
def test_verify_num_kv_splits_hand_values(args, kw, want):
    assert oracle.verify_num_kv_splits(*args, **kw) == want


# ---------------------------------------------------------------------------
# mutation checks: plausible oracle mistakes must fail the pins above
# ---------------------------------------------------------------------------

def _fails(fn, *a, **k):
    try:
        fn(*a, **k)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_gqa_verify_fp8_cache_equals_bf16_of_dequantised_values():
    """An FP8 cache with per-kv-head K and V scales gives the bf16 result of
    the cache holding its dequantised values.  The values come from torch's
    float8_e4m3fn decoding, and power-of-two scales keep them exact in bf16."""
    rng = np.random.default_rng(24)
    lens, qlen, Hq, Hkv, D, P = [13, 6], 2, 4, 2, 8, 4
    q, kv, bt, sl, sk = _rand_gqa_verify(rng, lens, qlen, Hq, Hkv, D, P)
    codes = rng.integers(0, 256, kv.shape, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                  # no NaN codes
    ks, vs = np.array([0.5, 4.0]), np.array([2.0, 0.25])
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    vals = vals.astype(np.float64)
    vals[..., :D] *= ks[None, :, None, None]
    vals[..., D:] *= vs[None, :, None, None]
    kv_bf = _bf16(vals.astype(np.float32))
    assert np.array_equal(oa.bf16_bits_to_f64(kv_bf), vals)          # exact in bf16
    O1, l1 = oracle.gqa_verify(q, codes, bt, sl, qlen, 0.3, sinks=sk, kv_dtype="fp8_e4m3fn",
                               k_scale=ks, v_scale=vs)
    O2, l2 = oracle.gqa_verify(q, kv_bf, bt, sl, qlen, 0.3, sinks=sk)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(l1, l2)
    # a scalar scale is the same as one per head
    O3, _ = oracle.gqa_verify(q, codes, bt, sl, qlen, 0.3, sinks=sk, kv_dtype="fp8_e4m3fn",
                              k_scale=2.0, v_scale=0.5)
    O4, _ = oracle.gqa_verify(q, codes, bt, sl, qlen, 0.3, sinks=sk, kv_dtype="fp8_e4m3fn",
                              k_scale=np.array([2.0, 2.0]), v_scale=np.array([0.5, 0.5]))
    np.testing.assert_array_equal(O3, O4)


# ---------------------------------------------------------------------------
# KV append
# ---------------------------------------------------------------------------

def test_kv_append_worked_example_placement():
    """Each sequence's new token lands where the worked example places it;
    every other element of the cache is unchanged."""
    with open(os.path.join(GOLDEN, "worked_example_append.json")) as f:
        ex = json.load(f)
    P, D = ex["page_size"], 4
    cache = np.arange(ex["num_pages"] * 1 * P * 2 * D, dtype=np.uint16).reshape(
        ex["num_pages"], 1, P, 2 * D)
    k = np.full((3, 1, D), 0xAAAA, np.uint16) + np.arange(3, dtype=np.uint16)[:, None, None]
    v = np.full((3, 1, D), 0xBBBB, np.uint16) + np.arange(3, dtype=np.uint16)[:, None, None]
    out = oracle.kv_append(cache, np.asarray(ex["block_table"]), np.asarray(ex["seq_lens_after"]),
                           1, k, v)
    changed = np.argwhere(np.any(out != cache, axis=-1))
    want = sorted((p, 0, s) for p, s in zip(ex["new_token_page"], ex["new_token_slot"]))
    assert sorted(map(tuple, changed.tolist())) == want
    for b, (p, s) in enumerate(zip(ex["new_token_page"], ex["new_token_slot"])):
        assert np.array_equal(out[p, 0, s, :D], k[b, 0]) and np.array_equal(out[p, 0, s, D:], v[b, 0])


def test_kv_append_verify_rows_and_skips():
    """qlen tokens land at positions L - qlen .. L - 1; a negative position or
    an entry outside the table / pool writes nothing."""
    P, H, n = 4, 2, 3
    bt = np.array([[5, 1, -1], [0, 9, -1], [2, 3, 4]])
    lens = np.array([6, 1, 12])       # request 1: positions -1, 0; request 2: 10, 11
    cache = np.zeros((6, H, P, n), np.int32)
    src = np.arange(3 * 2 * H * n, dtype=np.int32).reshape(6, H, n) + 100
    out = oracle.kv_append(cache, bt, lens, 2, src)
    assert np.array_equal(out[1, :, 0], src[0]) and np.array_equal(out[1, :, 1], src[1])
    assert np.array_equal(out[0, :, 0], src[3])          # request 1, position 0 (t = 1)
    assert np.array_equal(out[4, :, 2], src[4]) and np.array_equal(out[4, :, 3], src[5])
    assert np.count_nonzero(out) == 5 * H * n            # nothing else was written
    # entry 9 is outside the 6-page pool, position 12 // 4 = 3 is past the row
    out2 = oracle.kv_append(cache, bt, np.array([0, 6, 13]), 1, src[::2])
    assert np.count_nonzero(out2) == 0


def test_kv_append_then_decode_attends_the_new_token():
    """A marker written by kv_append at position L - 1 is the last key the
    decode attends: with a dominant score its V comes out exactly."""
    rng = np.random.default_rng(31)
    lens, Hq, Hkv, D, P = [9, 16], 4, 2, 8, 4
    q, kv, bt, sl, _ = _rand_gqa(rng, 2, Hq, Hkv, D, P, lens)
    qf = np.zeros((2, Hq, D), np.float32)
    qf[:, :, 0] = 1.0
    k = np.zeros((2, Hkv, D), np.float32)
    k[:, :, 0] = 200.0
    v = rng.integers(-50, 50, (2, Hkv, D)).astype(np.float32)
    kv2 = oracle.kv_append(kv, bt, sl, 1, _bf16(k), _bf16(v))
    O, lse = oracle.gqa_decode(_bf16(qf), kv2, bt, sl, 1.0)
    for b in range(2):
        for h in range(Hq):
            np.testing.assert_allclose(O[b, h], v[b, h // 2], atol=1e-12)


def test_mutant_row_limit_plus_one_is_caught(monkeypatch):
    orig = oa.row_key_range
    monkeypatch.setattr(oa, "row_key_range",
                        lambda L, qlen=1, t=0, real_len=None, window=0:
                        (orig(L, qlen, t, real_len, window)[0],
                         orig(L, qlen, t, real_len, window)[1] + 1))
    assert _fails(test_mla_matches_causal_dense_brute_force)
    assert _fails(test_gqa_worked_block_table_example, "reading_L")


def test_mutant_row_limit_minus_one_is_caught(monkeypatch):
    orig = oa.row_key_range
    monkeypatch.setattr(oa, "row_key_range",
                        lambda L, qlen=1, t=0, real_len=None, window=0:
                        (orig(L, qlen, t, real_len, window)[0],
                         max(orig(L, qlen, t, real_len, window)[1] - 1, 0)))
    assert _fails(test_mla_marker_at_row_limit_and_empty_rows)
    assert _fails(test_gqa_worked_block_table_example, "reading_L")


def test_mutant_verify_row_index_ignored_is_caught(monkeypatch):
    orig = oa.row_key_range
    monkeypatch.setattr(oa, "row_key_range",
                        lambda L, qlen=1, t=0, real_len=None, window=0:
                        orig(L, qlen, qlen - 1, real_len, window))
    assert _fails(test_gqa_verify_rows_are_prefix_decodes)
    assert _fails(test_gqa_verify_matches_causal_dense_brute_force)


def test_mutant_row_limit_plus_one_is_caught_in_gqa_verify(monkeypatch):
    orig = oa.row_key_range
    monkeypatch.setattr(oa, "row_key_range",
                        lambda L, qlen=1, t=0, real_len=None, window=0:
                        (orig(L, qlen, t, real_len, window)[0],
                         orig(L, qlen, t, real_len, window)[1] + 1))
    assert _fails(test_gqa_verify_matches_causal_dense_brute_force)


def test_mutant_append_position_off_by_one_is_caught(monkeypatch):
    orig = oa.kv_append

    def shifted(cache, block_table, seq_lens, qlen, src0, src1=None):
        return orig(cache, block_table, np.asarray(seq_lens) + 1, qlen, src0, src1)
    monkeypatch.setattr(oracle, "kv_append", shifted)
    assert _fails(test_kv_append_worked_example_placement)
    assert _fails(test_kv_append_then_decode_attends_the_new_token)


def test_mutant_swapped_kv_scales_are_caught(monkeypatch):
    orig = oa.gqa_verify

    def swapped(*a, k_scale=1.0, v_scale=1.0, **kw):
        return orig(*a, k_scale=v_scale, v_scale=k_scale, **kw)
    monkeypatch.setattr(oracle, "gqa_verify", swapped)
    assert _fails(test_gqa_verify_fp8_cache_equals_bf16_of_dequantised_values)


def test_mutant_window_off_by_one_is_caught(monkeypatch):
    orig = oa.row_key_range
    monkeypatch.setattr(oa, "row_key_range",
                        lambda L, qlen=1, t=0, real_len=None, window=0:
                        (max(orig(L, qlen, t, real_len, window)[0] - (1 if window else 0), 0),
                         orig(L, qlen, t, real_len, window)[1]))
    assert _fails(test_gqa_window_special_cases)


def test_mutant_dropped_page_is_caught(monkeypatch):
    orig = oa._gather_positions

    def drop_first_page(row, positions, page_size):
        pos = np.asarray(positions)
        keep = pos >= page_size if pos.size > page_size else np.ones_like(pos, bool)
        return orig(row, pos[keep], page_size)
    monkeypatch.setattr(oa, "_gather_positions", drop_first_page)
    assert _fails(test_gqa_worked_block_table_example, "reading_L")
    assert _fails(test_gqa_matches_dense_loop_brute_force)


def test_mutant_fixed_page_size_is_caught(monkeypatch):
    """A gather that assumes 16-token pages whatever the cache holds."""
    orig = oa._gather_positions
    monkeypatch.setattr(oa, "_gather_positions", lambda row, positions, page_size:
                        orig(row, positions, 16))
    assert _fails(test_gqa_verify_brute_force_at_page_size, 1)
    assert _fails(test_gqa_verify_brute_force_at_page_size, 64)
    assert _fails(test_mla_brute_force_at_page_size, 3)


def test_mutant_uniform_qlen_in_varlen_is_caught(monkeypatch):
    """A varlen oracle that used the batch's largest qlen for every request."""
    orig = oa.row_key_range
    monkeypatch.setattr(oa, "row_key_range", lambda L, qlen=1, t=0, real_len=None, window=0:
                        orig(L, 4, t, real_len, window))
    assert _fails(test_gqa_verify_varlen_matches_causal_dense_brute_force)


def test_mutant_sink_omitted_is_caught(monkeypatch):
    orig = oa.attend
    monkeypatch.setattr(oa, "attend", lambda q, K, V, s, sinks=None: orig(q, K, V, s, None))
    assert _fails(test_gqa_sink_special_cases)
    assert _fails(test_gqa_matches_dense_loop_brute_force)


def test_mutant_wrong_kv_head_map_is_caught(monkeypatch):
    orig = oa.gqa_decode

    def interleaved(q_bits, kv_bits, block_table, seq_lens, sm_scale, sinks=None, window=0):
        # maps query head h to kv head h % Hkv instead of h // G
        q = np.asarray(q_bits)
        Hq, Hkv = q.shape[1], np.asarray(kv_bits).shape[1]
        G = Hq // Hkv
        order = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
        O, lse = orig(q[:, order], kv_bits, block_table, seq_lens, sm_scale,
                      None if sinks is None else np.asarray(sinks)[order], window)
        inv = np.argsort(order)
        return O[:, inv], lse[:, inv]
    monkeypatch.setattr(oracle, "gqa_decode", interleaved)
    monkeypatch.setattr(oa, "gqa_decode", interleaved)
    assert _fails(test_gqa_matches_dense_loop_brute_force)


def test_mutant_transposed_merge_weight_is_caught(monkeypatch):
    orig = oa.merge_partials
    monkeypatch.setattr(oracle, "merge_partials",
                        lambda O, l, sinks=None: orig(O, -np.asarray(l), sinks))
    assert _fails(test_split_merge_equals_one_split, 3)

"""GPU parity of paged_decode_gqa (and merge_splits) against the fp64 oracle.

Every call goes through the C ABI (ctypes binding).  Inputs are the seeded
workloads of ``synth`` with every never-attended cache slot NaN-poisoned, so
a stray read shows up as a NaN output.  Besides the tolerance gates
(tests/helpers.check_attention) the tests check bit-exact indexing with
marker keys, bitwise invariance to the physical placement of pages, exact
zeros / -inf for keyless requests, run-to-run determinism, and the NaN
contract for an out-of-range block-table entry.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import bits16, check_attention, compact_gqa, oracle_gqa
from synth import bf16_bits_from_f32, gqa_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _dev(w):
    return (torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda())


def _run(pd, w, vals, S, **kw):
    bt, sl = _dev(w)
    out, lse = pd.paged_decode_gqa(vals["q"], vals["kv"], bt, sl, w.sm_scale,
                                   sinks=vals["sinks"], window=w.window, num_kv_splits=S, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("S", [1, 2])
def test_tiny_config(pd, S):
    w = gqa_workload("tiny_gqa")
    vals = w.values("cuda", poison=True)
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what=f"tiny S={S}")


@pytest.mark.parametrize("reading", ["reading_L", "reading_L_plus_1"])
@pytest.mark.parametrize("S", [1, 2])
def test_worked_example_block_table(pd, reading, S):
    """The literal block table of the worked example, with q = 0 and V dim 0
    holding the physical page id: O[..., 0] is the mean page id and LSE is
    ln(n) (closed forms stored in tests/golden)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    P, D = ex["page_size"], 128
    lens = ex[reading]["seq_lens"]
    bt = np.asarray(ex["block_table"], np.int32)
    rng = np.random.default_rng(21)
    kv = np.full((ex["num_pages"], 1, P, 2 * D), 0x7FC0, np.uint16)
    for b, L in enumerate(lens):
        for j in range(L):
            page, slot = bt[b, j // P], j % P
            kv[page, 0, slot] = bf16_bits_from_f32(rng.standard_normal(2 * D))
            kv[page, 0, slot, D] = bf16_bits_from_f32(np.float32([page]))[0]
    q = np.zeros((3, 8, D), np.uint16)
    kv_t = torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).cuda()
    q_t = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse = pd.paged_decode_gqa(q_t, kv_t, torch.from_numpy(bt).cuda(),
                                   torch.tensor(lens, dtype=torch.int32).cuda(),
                                   1.0 / math.sqrt(D), num_kv_splits=S)
    torch.cuda.synchronize()
    O, Lr = oracle.gqa_decode(q, kv, bt, np.asarray(lens), 1.0 / math.sqrt(D))
    check_attention(out, lse, O, Lr, what=reading)
    from fractions import Fraction
    want = [float(Fraction(s)) for s in ex[reading]["o_dim0"]]
    o = out.float().cpu().numpy()
    for b in range(3):
        np.testing.assert_allclose(o[b, :, 0], want[b], atol=2e-2)
        np.testing.assert_allclose(lse[b].cpu().numpy(), math.log(lens[b]), atol=1e-5)


@pytest.mark.parametrize("P,G", [(16, 8), (32, 8), (16, 4), (16, 1), (32, 16),
                                 (1, 8), (2, 4), (4, 8), (8, 8), (64, 8), (128, 2),
                                 (3, 8), (5, 1), (12, 4), (33, 16), (48, 8), (96, 2)])
def test_marker_keys_are_bit_exact(pd, P, G):
    """Request b attends L keys; key `target_b` scores 256 above every other
    (scale 1), so all other weights underflow to exactly 0 in fp32 and O must
    equal V_target bit for bit.  Targets cover the first and last slot of
    every page and of every 32-token tile."""
    D, L = 128, 5 * P + 7
    targets = sorted({0, L - 1} | {p * P for p in range(6)} | {p * P - 1 for p in range(1, 6)}
                     | {t * 32 for t in range(L // 32 + 1)} | {t * 32 + 31 for t in range(L // 32)})
    targets = [t for t in targets if 0 <= t < L]
    B = len(targets)
    n_pages = B * (-(-L // P)) + 3
    rng = np.random.default_rng(P * 100 + G)
    perm = rng.permutation(n_pages)
    maxb = -(-L // P) + 1
    bt = np.full((B, maxb), -1, np.int32)
    kv = np.full((n_pages, 1, P, 2 * D), 0x7FC0, np.uint16)
    q = np.zeros((B, G, D), np.float32)
    q[:, :, 0] = 1.0
    for b, tgt in enumerate(targets):
        bt[b, :maxb - 1] = perm[b * (maxb - 1):(b + 1) * (maxb - 1)]
        for j in range(L):
            row = np.zeros(2 * D, np.float32)
            row[1:D] = rng.standard_normal(D - 1)
            row[0] = 256.0 if j == tgt else 0.0
            row[D:] = rng.integers(-100, 100, D)
            kv[bt[b, j // P], 0, j % P] = bf16_bits_from_f32(row)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    for S in (1, 3):
        out, lse = pd.paged_decode_gqa(to_dev(bf16_bits_from_f32(q)), to_dev(kv),
                                       torch.from_numpy(bt).cuda(),
                                       torch.full((B,), L, dtype=torch.int32).cuda(), 1.0,
                                       num_kv_splits=S)
        torch.cuda.synchronize()
        got = bits16(out)
        for b, tgt in enumerate(targets):
            want = kv[bt[b, tgt // P], 0, tgt % P, D:]
            for h in range(G):
                assert np.array_equal(got[b, h], want), (S, b, tgt, h)
        np.testing.assert_allclose(lse.cpu().numpy(), 256.0, atol=1e-3)


def test_page_permutation_invariance_is_bitwise(pd):
    w = gqa_workload("gqa_sinks", batch=5, len_range=(200, 900))
    vals = w.values("cuda", poison=True)
    out1, lse1 = _run(pd, w, vals, 3)
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(w.num_pages, generator=g)
    kv2 = torch.empty_like(vals["kv"])
    kv2[perm.cuda()] = vals["kv"]
    bt2 = np.where(w.block_table >= 0, perm.numpy()[np.maximum(w.block_table, 0)], -1)
    out2, lse2 = pd.paged_decode_gqa(vals["q"], kv2, torch.from_numpy(bt2.astype(np.int32)).cuda(),
                                     torch.from_numpy(w.seq_lens).cuda(), w.sm_scale,
                                     sinks=vals["sinks"], num_kv_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


REDUCED = [
    ("gqa_sinks", dict(batch=6, len_range=(40, 1500))),
    ("gqa_window", dict(batch=6, len_range=(60, 3000))),
    ("gqa_skewed", dict(batch=12, loguniform=(16, 6000), zero_lens=2)),
    ("tiny_gqa", dict(batch=4, len_range=(1, 300))),
]


@pytest.mark.parametrize("name,kw", REDUCED, ids=[r[0] for r in REDUCED])
@pytest.mark.parametrize("S", ["cap", 1, 2, 3, 7])
def test_reduced_configs(pd, name, kw, S):
    w = gqa_workload(name, **kw)
    vals = w.values("cuda", poison=True)
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what=f"{name} S={S}")


@pytest.mark.parametrize("S", [1, 4])
def test_empty_requests_are_exact(pd, S):
    w = gqa_workload("gqa_sinks", fixed_lens=[0, 37, 0, 600, 0])
    vals = w.values("cuda", poison=True)
    out, lse = _run(pd, w, vals, S)
    for b in (0, 2, 4):
        assert torch.all(out[b].float() == 0)
        assert torch.all(torch.isneginf(lse[b]))
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, what="empty")


def test_window_larger_than_length_and_window_one(pd):
    w = gqa_workload("gqa_window", fixed_lens=[1, 5, 127, 128, 129, 700])
    vals = w.values("cuda", poison=True)
    for S in (1, 2):
        out, lse = _run(pd, w, vals, S)
        O, L = oracle_gqa(w, vals)
        check_attention(out, lse, O, L, what=f"window S={S}")


def test_out_of_range_block_table_entry_gives_nan(pd):
    w = gqa_workload("gqa_sinks", fixed_lens=[300, 300])
    vals = w.values("cuda", poison=True)
    bt = w.block_table.copy()
    bt[1, 3] = w.num_pages + 5                        # attended entry, out of range
    for S in (1, 2):
        out, lse = pd.paged_decode_gqa(vals["q"], vals["kv"], torch.from_numpy(bt).cuda(),
                                       torch.from_numpy(w.seq_lens).cuda(), w.sm_scale,
                                       sinks=vals["sinks"], num_kv_splits=S)
        torch.cuda.synchronize()
        assert torch.all(torch.isnan(out[1].float())) and torch.all(torch.isnan(lse[1]))
        q, kv, bt0, sl, sk = compact_gqa(w, vals, [0])
        O, L = oracle.gqa_decode(q, kv, bt0, sl, w.sm_scale, sinks=sk)
        check_attention(out[:1], lse[:1], O, L, what="valid neighbour")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_one_split_unit_per_wave_boundary(pd, fp8):
    """One split with exactly as many units (request, kv head) as the grid has
    waves (one unit per wave, no plan scan) and with one request more (the
    scanned whole-unit plan): both agree with the oracle on sampled requests,
    and the first batch's requests are bit for bit the larger batch's."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    waves = n_cu * (8 if fp8 else 4)
    b_unit = waves // 8                              # Hkv = 8: units == waves
    w = gqa_workload("gqa_sinks", batch=b_unit + 1, len_range=(1, 300), seed_offset=41 + fp8,
                     pool="tight")
    assert w.B * w.Hkv == waves + w.Hkv
    vals = w.values("cuda", poison=True, fp8=fp8)
    bt, sl = _dev(w)
    scales = dict(k_scale=vals.get("k_scale"), v_scale=vals.get("v_scale")) if fp8 else {}

    def call(nb):
        # qlen = 1 without real lengths: the decode kernel (8 waves per
        # workgroup for the FP8 cache)
        out, lse = pd.paged_verify_gqa(vals["q"][:nb], vals["kv"], bt[:nb], sl[:nb], 1, w.sm_scale,
                                       sinks=vals["sinks"], num_kv_splits=1, **scales)
        torch.cuda.synchronize()
        return out, lse

    big = call(w.B)
    unit = call(b_unit)
    assert torch.equal(big[0][:b_unit].view(torch.int16), unit[0].view(torch.int16))
    assert torch.equal(big[1][:b_unit].view(torch.int32), unit[1].view(torch.int32))
    sample = [0, 1, b_unit // 2, b_unit - 1, b_unit]
    O, L = oracle_gqa(w, vals, sample)
    check_attention(big[0][sample], big[1][sample], O, L,
                    o_atol=5e-2 if fp8 else 2e-2, what=f"one split, fp8={fp8}")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_one_split_pair_mode_boundary(pd, fp8):
    """One split with two waves per unit (at most 2 units per compute unit)
    and just past that bound (one wave per unit): both agree with the oracle
    on sampled requests, including units of one tile (the second wave of the
    pair streams nothing), empty requests and a window."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    b_pair = 2 * n_cu // 8                           # Hkv = 8: 2 units per CU
    lens = np.random.default_rng(5).integers(1, 400, size=b_pair + 1)
    lens[[0, 3, b_pair]] = [0, 1, 33]               # empty, one key, two tiles
    lens[1:3] = [31, 32]                             # one tile
    for nb, window in ((b_pair, 0), (b_pair + 1, 0), (b_pair, 40)):
        w = gqa_workload("gqa_sinks", fixed_lens=lens[:nb], seed_offset=43 + fp8, pool="tight",
                         window=window)
        vals = w.values("cuda", poison=True, fp8=fp8)
        bt, sl = _dev(w)
        scales = dict(k_scale=vals.get("k_scale"), v_scale=vals.get("v_scale")) if fp8 else {}
        out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"], bt, sl, 1, w.sm_scale,
                                       sinks=vals["sinks"], window=w.window, num_kv_splits=1,
                                       **scales)
        torch.cuda.synchronize()
        assert torch.all(out[0].float() == 0) and torch.all(torch.isneginf(lse[0]))
        sample = [0, 1, 2, 3, 4, nb // 2, nb - 1]
        O, L = oracle_gqa(w, vals, sample)
        check_attention(out[sample], lse[sample], O, L, o_atol=5e-2 if fp8 else 2e-2,
                        what=f"one split B={nb} window={window} fp8={fp8}")


def test_repeated_calls_are_bitwise_deterministic(pd):
    w = gqa_workload("gqa_skewed", batch=16, loguniform=(16, 5000), zero_lens=1)
    vals = w.values("cuda", poison=True)
    a = _run(pd, w, vals, 5)
    b = _run(pd, w, vals, 5)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


@pytest.mark.parametrize("S,Dv", [(1, 128), (5, 128), (16, 512), (70, 128)])
def test_merge_splits_against_oracle(pd, S, Dv):
    """Oracle-made partials (some splits empty, with NaN in their O slots)
    merged on the GPU vs the oracle's merge."""
    rng = np.random.default_rng(S + Dv)
    rows, H = 7, 6
    Op = rng.standard_normal((rows, H, S, Dv))
    lp = rng.standard_normal((rows, H, S)) * 3.0
    lp[rng.random((rows, H, S)) < 0.3] = -np.inf
    lp[0, 0, :] = -np.inf                              # a keyless (row, head)
    Op[np.isneginf(lp)] = np.nan
    sinks = rng.standard_normal(H)
    ws = np.concatenate([Op, lp[..., None]], axis=-1).astype(np.float32)
    O, L = oracle.merge_partials(ws[..., :Dv].astype(np.float64),
                                 ws[..., Dv].astype(np.float64), sinks)
    out, lse = pd.merge_splits(torch.from_numpy(ws).cuda(), rows, H, S, Dv,
                               sinks=torch.from_numpy(sinks.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    check_attention(out, lse, O, L, lse_atol=1e-5, what="merge")


@pytest.mark.parametrize("S", [2, 8, 9, 70])
def test_merge_stops_at_the_end_of_list_marker(pd, S):
    """lse = +inf ends a (row, head)'s slot list: the merge equals the
    oracle's merge of the slots before it, whatever lies after (NaN, huge
    lse values); a list ending at slot 0 is keyless (O = 0, LSE = -inf)."""
    rng = np.random.default_rng(S)
    rows, H, Dv = 5, 4, 128
    Op = rng.standard_normal((rows, H, S, Dv))
    lp = rng.standard_normal((rows, H, S)) * 3.0
    lp[rng.random((rows, H, S)) < 0.2] = -np.inf
    ends = rng.integers(0, S + 1, size=(rows, H))        # S: no marker
    ends[0, 0] = 0
    ends[1, 1] = min(S, 8)
    keep = np.arange(S)[None, None, :] < ends[..., None]
    lp_ref = np.where(keep, lp, -np.inf)
    O, L = oracle.merge_partials(Op, lp_ref, None)
    for r in range(rows):
        for h in range(H):
            e = ends[r, h]
            if e < S:
                lp[r, h, e] = np.inf
                lp[r, h, e + 1:] = 1e30                  # never read
                Op[r, h, e:] = np.nan
    ws = np.concatenate([Op, lp[..., None]], axis=-1).astype(np.float32)
    out, lse = pd.merge_splits(torch.from_numpy(ws).cuda(), rows, H, S, Dv)
    torch.cuda.synchronize()
    check_attention(out, lse, O, L, lse_atol=1e-5, what=f"merge S={S} with end markers")


FULL = ["gqa_sinks", "gqa_window", "gqa_skewed"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_config_sampled(pd, name):
    """Full-size configuration in the launch configuration the benchmark
    times (split cap from the library), checked on sampled requests: the
    shortest, the longest, keyless ones and a seeded random handful."""
    w = gqa_workload(name)
    vals = w.values("cuda", poison=True)
    S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(3)
    order = np.argsort(w.seq_lens)
    pick = {int(order[0]), int(order[-1])} | set(int(i) for i in rng.choice(w.B, 5, replace=False))
    pick |= set(int(i) for i in np.nonzero(w.seq_lens == 0)[0])
    pick = sorted(pick)
    O, L = oracle_gqa(w, vals, pick)
    check_attention(out[pick], lse[pick], O, L, what=f"{name} full S={S}")

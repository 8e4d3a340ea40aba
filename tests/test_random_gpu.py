"""Seeded random-shape parity of every GPU path against the fp64 oracle.

Each case draws its own shapes from a fixed seed: batch, head counts and
group size, verify tokens, page size (every power-of-two class), lengths
(zero, shorter than qlen, within one page, ragged multi-tile), real lengths,
window, sinks, bf16 or FP8 cache and split count, with up to 64 score
columns per kv head on the verify path.  The hand-written tests
pin each feature alone; these check that the features compose.  Every call
goes through the C ABI; never-attended cache slots are NaN-poisoned.
"""

import numpy as np
import pytest
import torch

from helpers import O_ATOL_FP8, check_attention, oracle_gqa, oracle_mla
from synth import gqa_workload, mla_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

PAGES = [1, 2, 3, 4, 8, 12, 16, 32, 48, 64, 96, 128]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _lengths(rng, B, hi):
    kind = rng.integers(0, 4, size=B)
    lens = np.where(kind == 0, rng.integers(0, 4, size=B),            # empty / shorter than qlen
                    np.where(kind == 1, rng.integers(1, 40, size=B),  # within a page or tile
                             rng.integers(1, hi + 1, size=B)))       # ragged, several tiles
    return lens.astype(np.int64)


def _gqa_case(seed):
    rng = np.random.default_rng(9000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    qlen = int(rng.choice([1, 1, 2, 3, 4]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if qlen * g <= 16]))
    B = int(rng.integers(1, 7))
    lens = _lengths(rng, B, 700)
    verify = qlen > 1 or rng.random() < 0.3
    real = np.maximum(lens - rng.integers(0, 3, size=B), 0) if verify else None
    return dict(name="gqa_sinks" if rng.random() < 0.6 else "gqa_skewed",
                fixed_lens=lens, qlen=qlen, fixed_real=real, heads=(G * Hkv, Hkv),
                window=int(rng.choice([0, 0, 1, 7, 50, 333])), page_size=int(rng.choice(PAGES)),
                fp8=bool(rng.random() < 0.4), S=rng.choice(["cap", 1, 2, 3, 5]))


@pytest.mark.parametrize("seed", range(32))
def test_gqa_random(pd, seed):
    c = _gqa_case(seed)
    w = gqa_workload(c["name"], fixed_lens=c["fixed_lens"], qlen=c["qlen"],
                     fixed_real=c["fixed_real"], heads=c["heads"], window=c["window"],
                     page_size=c["page_size"], pool="tight", seed_offset=seed)
    vals = w.values("cuda", poison=True, fp8=c["fp8"])
    S = c["S"]
    S = pd.gqa_split_cap(w.B, w.Hkv, max(int(w.seq_lens.max()), 1), w.window) if S == "cap" else int(S)
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    scales = dict(k_scale=vals["k_scale"], v_scale=vals["v_scale"]) if c["fp8"] else {}
    out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"], torch.from_numpy(w.block_table).cuda(),
                                   torch.from_numpy(w.seq_lens).cuda(), w.qlen, w.sm_scale,
                                   sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                                   num_kv_splits=S, **scales)
    torch.cuda.synchronize()
    O, L = oracle_gqa(w, vals)
    what = (f"seed={seed} B={w.B} Hq={w.Hq} Hkv={w.Hkv} qlen={w.qlen} P={w.P} "
            f"window={w.window} fp8={c['fp8']} S={S} lens={list(w.seq_lens)}")
    check_attention(out, lse, O, L, o_atol=O_ATOL_FP8 if c["fp8"] else 2e-2, what=what)


def _gqa_wide_case(seed):
    """Verify with 17 to 64 score columns (2 or 4 column groups)."""
    rng = np.random.default_rng(9300 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    qlen, G = [(2, 16), (3, 8), (4, 8), (8, 8), (5, 4), (16, 4), (4, 16), (9, 4)][seed % 8]
    B = int(rng.integers(1, 6))
    lens = _lengths(rng, B, 600)
    real = np.maximum(lens - rng.integers(0, 4, size=B), 0)
    return dict(fixed_lens=lens, qlen=qlen, fixed_real=real, heads=(G * Hkv, Hkv),
                window=int(rng.choice([0, 0, 9, 100])), page_size=int(rng.choice(PAGES)),
                fp8=bool(rng.random() < 0.4), S=rng.choice(["cap", 1, 2, 4]))


@pytest.mark.parametrize("seed", range(16))
def test_gqa_random_wide(pd, seed):
    c = _gqa_wide_case(seed)
    w = gqa_workload("gqa_verify", fixed_lens=c["fixed_lens"], qlen=c["qlen"],
                     fixed_real=c["fixed_real"], heads=c["heads"], window=c["window"],
                     page_size=c["page_size"], pool="tight", seed_offset=100 + seed)
    vals = w.values("cuda", poison=True, fp8=c["fp8"])
    S = c["S"]
    S = pd.gqa_split_cap(w.B, w.Hkv, max(int(w.seq_lens.max()), 1), w.window) if S == "cap" else int(S)
    real = torch.from_numpy(w.real_seq_lens).cuda()
    scales = dict(k_scale=vals["k_scale"], v_scale=vals["v_scale"]) if c["fp8"] else {}
    out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"], torch.from_numpy(w.block_table).cuda(),
                                   torch.from_numpy(w.seq_lens).cuda(), w.qlen, w.sm_scale,
                                   sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                                   num_kv_splits=S, **scales)
    torch.cuda.synchronize()
    O, L = oracle_gqa(w, vals)
    what = (f"seed={seed} B={w.B} Hq={w.Hq} Hkv={w.Hkv} qlen={w.qlen} P={w.P} "
            f"window={w.window} fp8={c['fp8']} S={S} lens={list(w.seq_lens)}")
    check_attention(out, lse, O, L, o_atol=O_ATOL_FP8 if c["fp8"] else 2e-2, what=what)


@pytest.mark.parametrize("seed", range(16))
def test_mla_random(pd, seed):
    rng = np.random.default_rng(9500 + seed)
    qlen = int(rng.integers(1, 5))
    H = int(rng.choice([8, 16, 24, 32, 64, 128]))
    B = int(rng.integers(1, 4))
    lens = _lengths(rng, B, 400)
    real = np.maximum(lens - rng.integers(0, 3, size=B), 0)
    fp8 = bool(rng.random() < 0.5)
    P = int(rng.choice(PAGES))
    S = int(rng.choice([1, 2, 3, 4]))
    w = mla_workload(fixed_lens=lens, fixed_real=real, qlen=qlen, heads=H, page_size=P,
                     seed_offset=100 + seed)
    vals = w.values("cuda", poison=True, fp8=fp8)
    ks = torch.tensor([vals["k_scale"]], dtype=torch.float32, device="cuda") if fp8 else None
    out, lse = pd.paged_verify_mla(vals["q"], vals["kv"], torch.from_numpy(w.block_table).cuda(),
                                   torch.from_numpy(w.seq_lens).cuda(),
                                   torch.from_numpy(w.real_seq_lens).cuda(), w.qlen, w.sm_scale,
                                   head_dim_v=w.Lv, k_scale=ks, num_kv_splits=S)
    torch.cuda.synchronize()
    O, L = oracle_mla(w, vals, fp8=fp8)
    check_attention(out, lse, O.reshape(out.shape), L, o_atol=O_ATOL_FP8 if fp8 else 2e-2,
                    what=f"seed={seed} B={B} qlen={qlen} H={H} P={P} fp8={fp8} S={S} "
                         f"lens={list(lens)} real={list(real)}")

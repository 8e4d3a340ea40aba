"""GPU parity of the FP8 E4M3FN GQA cache (paged_verify_gqa with K and V
scales) against the fp64 oracle, and bitwise against the bf16 path.

With power-of-two scales, folding k_scale into the exp2 scale and v_scale
into the output rounds exactly like scaling the cache values first, so the
FP8 path must equal the bf16 path on the cache of the dequantised values bit
for bit.  The oracle checks use the FP8 tolerance, over decode and verify,
split counts, page sizes, windows, scalar and per-head scales, and the full
sinks configuration on sampled requests.
"""

import numpy as np
import pytest
import torch

from helpers import O_ATOL_FP8, check_attention, oracle_gqa
from synth import gqa_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _run(pd, w, vals, S, kv=None, k_scale="w", v_scale="w"):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    ks = vals.get("k_scale") if isinstance(k_scale, str) else k_scale
    vs = vals.get("v_scale") if isinstance(v_scale, str) else v_scale
    out, lse = pd.paged_verify_gqa(vals["q"], vals["kv"] if kv is None else kv,
                                   torch.from_numpy(w.block_table).cuda(),
                                   torch.from_numpy(w.seq_lens).cuda(), w.qlen, w.sm_scale,
                                   sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                                   num_kv_splits=S, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    ("decode", dict(batch=6, len_range=(1, 900))),
    ("verify2", dict(batch=6, len_range=(1, 900), qlen=2, real_drop=(0, 2))),
    ("verify4_g4", dict(batch=5, len_range=(1, 700), qlen=4, heads=(32, 8))),
    ("window", dict(batch=6, len_range=(1, 900), window=100)),
    ("page32", dict(batch=6, len_range=(1, 900), page_size=32)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("S", ["cap", 1, 3])
def test_fp8_reduced(pd, name, kw, S):
    w = gqa_workload("gqa_sinks", seed_offset=len(name), pool="tight", **kw)
    vals = w.values("cuda", poison=True, fp8=True)
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    O, L = oracle_gqa(w, vals)
    check_attention(out, lse, O, L, o_atol=O_ATOL_FP8, what=f"fp8 {name} S={S}")


@pytest.mark.parametrize("qlen", [1, 2])
@pytest.mark.parametrize("S", [1, 3])
def test_fp8_equals_bf16_of_dequantised_cache_bitwise(pd, qlen, S):
    w = gqa_workload("gqa_sinks", batch=6, len_range=(1, 800), qlen=qlen, seed_offset=7,
                     pool="tight")
    vals = w.values("cuda", poison=False)
    g = torch.Generator().manual_seed(3)
    codes = torch.randint(0, 256, vals["kv"].shape, generator=g, dtype=torch.int32).to(torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38              # no NaN codes
    ks = torch.tensor([2.0 ** (i % 5 - 3) for i in range(w.Hkv)])
    vs = torch.tensor([2.0 ** (2 - i % 4) for i in range(w.Hkv)])
    deq = codes.view(torch.float8_e4m3fn).to(torch.float32)
    deq[..., :w.D] *= ks[None, :, None, None]
    deq[..., w.D:] *= vs[None, :, None, None]
    kv_bf = deq.to(torch.bfloat16)
    assert torch.equal(kv_bf.float(), deq)            # exact in bf16
    fp8_vals = dict(vals, kv=codes.cuda(), k_scale=ks.cuda(), v_scale=vs.cuda())
    o8, l8 = _run(pd, w, fp8_vals, S)
    o16, l16 = _run(pd, w, dict(vals, kv=kv_bf.cuda()), S, k_scale=None, v_scale=None)
    assert torch.equal(o8.view(torch.int16), o16.view(torch.int16))
    assert torch.equal(l8, l16)


def test_fp8_scalar_scale_equals_per_head(pd):
    w = gqa_workload("gqa_sinks", batch=5, len_range=(1, 600), seed_offset=4, pool="tight")
    vals = w.values("cuda", poison=True, fp8=True)
    ks1 = torch.tensor([0.02], device="cuda")
    vs1 = torch.tensor([0.03], device="cuda")
    o1, l1 = _run(pd, w, vals, 2, k_scale=ks1, v_scale=vs1)
    o2, l2 = _run(pd, w, vals, 2, k_scale=ks1.repeat(w.Hkv), v_scale=vs1.repeat(w.Hkv))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    O, L = oracle_gqa(w, dict(vals, k_scale=ks1.repeat(w.Hkv), v_scale=vs1.repeat(w.Hkv)))
    check_attention(o1, l1, O, L, o_atol=O_ATOL_FP8, what="scalar scales")


def test_fp8_full_sinks_config_sampled(pd):
    """The full sinks configuration on an FP8 cache, in the launch
    configuration bench.py times, checked on sampled requests."""
    w = gqa_workload("gqa_sinks")
    vals = w.values("cuda", poison=True, fp8=True)
    S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out, lse = _run(pd, w, vals, S)
    sample = [0, int(np.argmax(w.seq_lens)), int(np.argmin(w.seq_lens)), w.B - 1]
    O, L = oracle_gqa(w, vals, sample)
    check_attention(out[sample], lse[sample], O, L, o_atol=O_ATOL_FP8, what="fp8 sinks full")

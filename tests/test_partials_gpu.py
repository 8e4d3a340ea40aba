"""GPU parity of the partials-only entry points (paged_decode_gqa_partials,
paged_verify_gqa_partials with and without cu_seqlens_q,
paged_verify_mla_partials): the per-shard half of split-KV.

Each call goes through the C ABI.  The partials are checked two ways:
  * merged on the host by the oracle's split merge (fp64) they must match
    the oracle's attention over the whole key range, sinks included, so the
    partials themselves are pinned to the oracle independently of the GPU
    merge;
  * merged by merge_splits on the GPU they must equal the full call
    bit for bit when S > 1 (the same kernel plan and the same merge), and
    match it to the parity tolerance when S = 1 (the full call then writes
    O directly, without the fp32 partial).
Every workspace and output starts NaN-filled: every slot's LSE must end
finite or -inf (unused slots), never NaN, and every used slot's O finite.
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import O_ATOL_FP8, check_attention, oracle_gqa, oracle_mla
from synth import gqa_workload, mla_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def pd():
    import paged_split_kv_decode_amd as m
    return m


def _dev(w):
    real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()
    return torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), real


def _sinks_np(vals):
    return None if vals["sinks"] is None else vals["sinks"].cpu().numpy().astype(np.float64)


def _nan_ws(rows, H, S, Dv):
    """A workspace that starts as NaN: a slot the plan fails to write stays NaN."""
    return torch.full((rows * H * max(S, 1) * (Dv + 1),), float("nan"), dtype=torch.float32,
                      device="cuda")


def _nan_out(rows, H, Dv):
    return (torch.full((rows, H, Dv), float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full((rows, H), float("nan"), dtype=torch.float32, device="cuda"))


def _full_kw(rows, H, S, Dv):
    """NaN-filled outputs (and workspace) for the full call."""
    out, lse = _nan_out(rows, H, Dv)
    kw = dict(out=out, lse=lse)
    if S > 1:
        kw["workspace"] = _nan_ws(rows, H, S, Dv)
    return kw


def _check_partials(pd, ws, S, Dv, sinks_t, O_ref, L_ref, full, o_atol, what):
    """ws: [rows, H, S, Dv + 1] partials; full: (out, lse) of the full call."""
    torch.cuda.synchronize()
    assert tuple(ws.shape[2:]) == (S, Dv + 1)
    wsn = ws.double().cpu().numpy()
    lse_p = wsn[..., Dv]
    assert not np.isnan(lse_p).any(), f"{what}: NaN split LSE (a slot never written?)"
    assert np.all(np.isfinite(lse_p) | np.isneginf(lse_p)), f"{what}: +inf split LSE"
    used = np.isfinite(lse_p)
    assert np.all(np.isfinite(wsn[..., :Dv][used])), f"{what}: used slot with unwritten O"
    sinks = None if sinks_t is None else sinks_t.double().cpu().numpy()
    O_h, L_h = oracle.merge_partials(wsn[..., :Dv], lse_p, sinks)
    check_attention(torch.from_numpy(O_h), torch.from_numpy(L_h), O_ref.reshape(O_h.shape),
                    L_ref.reshape(L_h.shape), o_atol=o_atol, what=f"{what} host merge")
    rows, H = ws.shape[0], ws.shape[1]
    out_m, lse_m = pd.merge_splits(ws.contiguous(), rows, H, S, Dv, sinks=sinks_t)
    torch.cuda.synchronize()
    out_f, lse_f = full
    if S > 1:
        assert torch.equal(out_m.view(torch.int16), out_f.view(torch.int16)), \
            f"{what}: merged partials differ from the full call"
        assert torch.equal(lse_m, lse_f), f"{what}: merged LSE differs from the full call"
    else:
        check_attention(out_m, lse_m, O_ref.reshape(out_m.shape), L_ref.reshape(lse_m.shape),
                        o_atol=o_atol, what=f"{what} S=1 merge")


@pytest.mark.parametrize("S", [1, 3, "cap"])
@pytest.mark.parametrize("window", [0, 37])
def test_decode_partials(pd, S, window):
    w = gqa_workload("gqa_sinks", batch=6, len_range=(1, 900), window=window, seed_offset=41)
    vals = w.values("cuda", poison=True)
    bt, sl, _ = _dev(w)
    if S == "cap":
        S = pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    ws = pd.paged_decode_gqa_partials(vals["q"], vals["kv"], bt, sl, w.sm_scale,
                                      window=w.window, num_kv_splits=S,
                                      workspace=_nan_ws(w.rows, w.Hq, S, w.D))
    full = pd.paged_decode_gqa(vals["q"], vals["kv"], bt, sl, w.sm_scale, sinks=vals["sinks"],
                               window=w.window, num_kv_splits=S,
                               **_full_kw(w.rows, w.Hq, S, w.D))
    O, L = oracle_gqa(w, vals)
    _check_partials(pd, ws, S, w.D, vals["sinks"], O, L, full, 2e-2,
                    f"decode S={S} window={window}")


VERIFY = [(4, (32, 8)), (2, (64, 8)), (16, (8, 8))]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S", [1, 2, 5])
@pytest.mark.parametrize("qlen,heads", VERIFY, ids=[f"q{q}" for q, _ in VERIFY])
def test_verify_partials(pd, qlen, heads, S, fp8):
    w = gqa_workload("gqa_verify", batch=5, len_range=(1, 700), qlen=qlen, heads=heads,
                     real_drop=(0, 3), window=29 if qlen == 2 else None, seed_offset=53 + qlen)
    vals = w.values("cuda", poison=True, fp8=fp8)
    bt, sl, real = _dev(w)
    scales = dict(k_scale=vals["k_scale"], v_scale=vals["v_scale"]) if fp8 else {}
    ws = pd.paged_verify_gqa_partials(vals["q"], vals["kv"], bt, sl, w.qlen, w.sm_scale,
                                      window=w.window, real_seq_lens=real, num_kv_splits=S,
                                      workspace=_nan_ws(w.rows, w.Hq, S, w.D), **scales)
    full = pd.paged_verify_gqa(vals["q"], vals["kv"], bt, sl, w.qlen, w.sm_scale,
                               sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                               num_kv_splits=S, **_full_kw(w.rows, w.Hq, S, w.D), **scales)
    O, L = oracle_gqa(w, vals)
    _check_partials(pd, ws, S, w.D, vals["sinks"], O, L, full, O_ATOL_FP8 if fp8 else 2e-2,
                    f"verify qlen={qlen} S={S} fp8={fp8}")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S", [1, 3])
def test_varlen_partials(pd, S, fp8):
    qlens = [2, 0, 1, 4, 1, 3]
    lens = [300, 50, 1, 2, 700, 33]
    real = [max(L - 1, 0) for L in lens]
    w = gqa_workload("gqa_verify", fixed_lens=lens, fixed_real=real, heads=(32, 8), qlen=4,
                     pool="tight", seed_offset=61)
    vals = w.values("cuda", poison=True, fp8=fp8)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    g = torch.Generator(device="cpu").manual_seed(61)
    q = torch.randn((int(cu[-1]), w.Hq, w.D), generator=g).to(torch.bfloat16).cuda()
    bt, sl, real_d = _dev(w)
    cu_d = torch.from_numpy(cu).cuda()
    scales = dict(k_scale=vals["k_scale"], v_scale=vals["v_scale"]) if fp8 else {}
    rows = int(cu[-1])
    ws = pd.paged_verify_gqa_partials(q, vals["kv"], bt, sl, max(qlens), w.sm_scale,
                                      real_seq_lens=real_d, cu_seqlens_q=cu_d, num_kv_splits=S,
                                      workspace=_nan_ws(rows, w.Hq, S, w.D), **scales)
    full = pd.paged_verify_gqa_varlen(q, vals["kv"], bt, sl, cu_d, max(qlens), w.sm_scale,
                                      sinks=vals["sinks"], real_seq_lens=real_d,
                                      num_kv_splits=S, **_full_kw(rows, w.Hq, S, w.D), **scales)
    kv = vals["kv"].cpu().numpy() if fp8 else vals["kv"].view(torch.int16).cpu().numpy().view(
        np.uint16)
    kw = {}
    if fp8:
        kw = dict(kv_dtype="fp8_e4m3fn", k_scale=vals["k_scale"].cpu().numpy().astype(np.float64),
                  v_scale=vals["v_scale"].cpu().numpy().astype(np.float64))
    O, L = oracle.gqa_verify_varlen(q.view(torch.int16).cpu().numpy().view(np.uint16), kv,
                                    w.block_table, w.seq_lens, cu.astype(np.int64), w.sm_scale,
                                    sinks=_sinks_np(vals), window=w.window,
                                    real_seq_lens=w.real_seq_lens, **kw)
    _check_partials(pd, ws, S, w.D, vals["sinks"], O, L, full, O_ATOL_FP8 if fp8 else 2e-2,
                    f"varlen S={S} fp8={fp8}")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S", [1, 2, 4])
def test_mla_partials(pd, S, fp8):
    w = mla_workload(fixed_lens=[2, 5, 40, 330, 0, 697], fixed_real=[2, 4, 39, 330, 0, 695],
                     heads=16)
    vals = w.values("cuda", poison=True, fp8=fp8)
    bt, sl, real = _dev(w)
    ks = torch.tensor([vals["k_scale"]], dtype=torch.float32, device="cuda") if fp8 else None
    ws = pd.paged_verify_mla_partials(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                                      head_dim_v=w.Lv, k_scale=ks, num_kv_splits=S,
                                      workspace=_nan_ws(w.rows, w.H, S, w.Lv))
    full = pd.paged_verify_mla(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                               head_dim_v=w.Lv, k_scale=ks, num_kv_splits=S,
                               **_full_kw(w.rows, w.H, S, w.Lv))
    O, L = oracle_mla(w, vals, fp8=fp8)
    _check_partials(pd, ws, S, w.Lv, None, O, L, full, O_ATOL_FP8 if fp8 else 2e-2,
                    f"mla S={S} fp8={fp8}")


def test_mla_partials_reduced_config(pd):
    """The verify configuration's shapes (qlen 4, 128 heads) with its split
    cap at oracle-sized lengths."""
    w = mla_workload(batch=3, len_range=(100, 700), seed_offset=5)
    vals = w.values("cuda", poison=True)
    bt, sl, real = _dev(w)
    S = pd.mla_split_cap(w.B, w.qlen, w.H, int(w.seq_lens.max()))
    ws = pd.paged_verify_mla_partials(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                                      head_dim_v=w.Lv, num_kv_splits=S,
                                      workspace=_nan_ws(w.rows, w.H, S, w.Lv))
    full = pd.paged_verify_mla(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                               head_dim_v=w.Lv, num_kv_splits=S, **_full_kw(w.rows, w.H, S, w.Lv))
    O, L = oracle_mla(w, vals)
    _check_partials(pd, ws, S, w.Lv, None, O, L, full, 2e-2, f"mla cap S={S}")

"""GPU test of paged_verify_gqa_noalloc, the entry point that allocates
nothing (split partials in the library's per-GPU scratch array).

Both entry points are called through the C ABI (ctypes) on the same seeded
inputs: the allocation-free call must give exactly the output of
paged_verify_gqa with a caller-owned workspace (same kernels, same plan),
and both must pass the oracle's parity gates.  Two calls follow each other,
the second with a smaller batch and fewer splits, so the second reads a
scratch array that still holds the first call's partials.  A call whose
partials would not fit the 64 MiB array is refused before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

from helpers import check_attention, oracle_gqa
from synth import gqa_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

SCRATCH_BYTES = 64 << 20


@pytest.fixture(scope="module")
def lib():
    from paged_split_kv_decode_amd._native import lib as L
    return L


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(lib, noalloc, w, vals, bt, sl, real, S, ws=None):
    out = torch.full((w.rows, w.Hq, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.rows, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    q, kv = vals["q"], vals["kv"]
    head = (_p(q), q.stride(0), q.stride(1), _p(kv), 0, None, None, 0,
            kv.stride(0), kv.stride(1), w.num_pages, _p(bt), bt.stride(0), w.max_blocks,
            _p(sl), _p(real), w.qlen, _p(vals["sinks"]), w.window, float(w.sm_scale),
            w.B, w.Hq, w.Hkv, w.D, w.P, S)
    tail = (_p(out), out.stride(0), out.stride(1), _p(lse), lse.stride(0),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if noalloc:
        st = lib.paged_verify_gqa_noalloc(*head, *tail)
    else:
        st = lib.paged_verify_gqa(*head, _p(ws), 0 if ws is None else ws.numel() * 4, *tail)
    return st, out, lse


def _case(batch, qlen, seed, len_range=(40, 1500)):
    w = gqa_workload("gqa_verify", batch=batch, len_range=len_range, qlen=qlen,
                     real_drop=(0, 1), seed_offset=seed)
    vals = w.values("cuda", poison=True)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    real = torch.from_numpy(w.real_seq_lens).cuda()
    return w, vals, bt, sl, real


def test_noalloc_matches_workspace_entry_on_two_calls_in_a_row(lib):
    # first call: 24 requests x 2 verify tokens, 8 splits; second: 7 requests
    # x 1 token, 3 splits (smaller partials, stale scratch from the first)
    for batch, qlen, S, seed in ((24, 2, 8, 311), (7, 1, 3, 312)):
        w, vals, bt, sl, real = _case(batch, qlen, seed)
        ws = torch.full((w.rows * w.Hq * S * (w.D + 1),), float("nan"), dtype=torch.float32,
                        device="cuda")
        st0, out0, lse0 = _call(lib, False, w, vals, bt, sl, real, S, ws)
        st1, out1, lse1 = _call(lib, True, w, vals, bt, sl, real, S)
        torch.cuda.synchronize()
        assert st0 == 0 and st1 == 0, (st0, st1)
        assert torch.equal(out0.view(torch.int16), out1.view(torch.int16)), \
            f"B={batch} S={S}: O differs from the workspace entry point"
        assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32)), \
            f"B={batch} S={S}: LSE differs from the workspace entry point"
        O_ref, L_ref = oracle_gqa(w, vals)
        check_attention(out1, lse1, O_ref.reshape(out1.shape), L_ref.reshape(lse1.shape),
                        what=f"noalloc B={batch} qlen={qlen} S={S}")


def test_noalloc_single_split_and_empty_batch(lib):
    w, vals, bt, sl, real = _case(5, 2, 313)
    st0, out0, lse0 = _call(lib, False, w, vals, bt, sl, real, 1)
    st1, out1, lse1 = _call(lib, True, w, vals, bt, sl, real, 1)
    torch.cuda.synchronize()
    assert st0 == 0 and st1 == 0
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32))


def test_noalloc_refuses_partials_beyond_the_scratch(lib):
    from paged_split_kv_decode_amd._native import PD_ERR_WORKSPACE

    w, vals, bt, sl, real = _case(64, 2, 314, len_range=(64, 256))
    # 128 rows x 64 heads x S x 129 x 4 bytes > 64 MiB from S = 16 on
    S = 1 + SCRATCH_BYTES // (w.rows * w.Hq * (w.D + 1) * 4)
    st, out, _ = _call(lib, True, w, vals, bt, sl, real, S)
    torch.cuda.synchronize()
    assert st == PD_ERR_WORKSPACE
    assert torch.isnan(out.float()).all(), "a refused call must enqueue nothing"

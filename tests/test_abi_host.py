"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/paged_decode.h
declares, compute the static split cap exactly as the oracle's restatement of
the pages' rule, and reject bad arguments with the documented status before
any HIP call (fake device addresses are never dereferenced on the host).
"""

import ctypes
import os
import random
import re

import pytest

import oracle
from paged_split_kv_decode_amd import _native
from paged_split_kv_decode_amd._native import (PD_ERR_ALIGN, PD_ERR_INVALID, PD_ERR_UNSUPPORTED,
                                               PD_ERR_WORKSPACE, PD_OK, lib)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_decode.h")
FAKE = 0x100000          # 16-byte aligned stand-in address, never dereferenced
NULL = None


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^PD_API\s+[\w\s\*]+?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = _declared_functions()
    for want in ("paged_decode_gqa", "paged_verify_mla", "num_kv_splits_cap", "merge_splits"):
        assert want in names


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(_native.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), f"{name} declared in paged_decode.h but not exported"
    assert set(_native.EXPORTS) <= set(_declared_functions())


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.pd_status_string(s)
    assert lib.pd_status_string(7) == b"unknown status"


def _cap(*a):
    return lib.pd_split_rule(*a)


@pytest.mark.parametrize("args,want", [
    ((70, 3, 1, 1, 1, 256, 1.0, 64, 8), 2),
    ((100000, 300, 1, 1, 1, 256, 1.0, 64, 8), 4),
    ((4096, 1, 1, 32, 32, 256, 1.0, 64, 8), 64),
    ((64, 1, 1, 32, 32, 256, 1.0, 64, 8), 1),
    ((16384, 4, 4, 128, 64, 256, 1.0, 64, 16), 8),
    ((16384, 32, 4, 128, 64, 256, 1.0, 64, 16), 1),
])
def test_split_cap_hand_values(args, want):
    assert _cap(*args, 0) == want


def test_split_cap_matches_oracle_rule_randomised():
    rng = random.Random(0)
    for _ in range(3000):
        msl = rng.choice([0, 1, 7, 64, 100, 1000, 4096, 16384, 131072, rng.randint(0, 200000)])
        batch = rng.choice([0, 1, 2, 3, 17, 64, 256, rng.randint(0, 5000)])
        qlen = rng.randint(1, 8)
        heads = rng.choice([1, 8, 16, 32, 64, 128])
        block_h = rng.choice([1, 16, 32, 64, 128])
        sm = rng.choice([1, 80, 256, 304])
        occ = rng.choice([1.0, 2.0, 4.0])
        mw = rng.choice([1, 16, 64, 256])
        ms = rng.choice([1, 2, 8, 16, 64])
        want = oracle.verify_num_kv_splits(msl, batch, qlen, heads, sm, block_h, occ, mw, ms)
        assert _cap(msl, batch, qlen, heads, block_h, sm, occ, mw, ms, 0) == want


def test_split_cap_balance_extension():
    # P1 rule alone returns 1 when programs exceed slots with equal rounds
    assert _cap(131072, 256, 1, 8, 1, 256, 1.0, 256, 64, 0) == 1
    # the skew bound raises it to ceil(max_len / chunk), capped by max_splits
    assert _cap(131072, 256, 1, 8, 1, 256, 1.0, 256, 64, 1024) == 64
    assert _cap(8192, 64, 1, 8, 1, 256, 1.0, 256, 64, 1024) == 8
    # and never above ideal = ceil(max_len / min_work)
    assert _cap(128, 64, 1, 8, 1, 256, 1.0, 256, 64, 16) == 1


def _cdiv(a, b):
    return -(-a // b)


def _policy_want(keys, programs_batch, qlen, heads, block_h, cus, min_work, max_splits, chunk):
    """The oracle's restated rule plus the documented skew bound."""
    base = oracle.verify_num_kv_splits(keys, programs_batch, qlen, heads, cus, block_h, 1.0,
                                       min_work, max_splits)
    ideal = _cdiv(max(keys, 1), min_work)
    return max(base, min(max_splits, ideal, _cdiv(max(keys, 1), chunk)))


def test_gqa_policy_cap_matches_oracle_rule_and_skew_bound():
    rng = random.Random(1)
    for _ in range(2000):
        msl = rng.choice([0, 1, 100, 1024, 8192, 32768, 131072, rng.randint(0, 300000)])
        batch = rng.choice([1, 3, 64, 256, rng.randint(0, 4000)])
        hkv = rng.choice([1, 2, 8, 16])
        window = rng.choice([0, 0, 128, 4096, rng.randint(-5, 70000)])
        cus = rng.choice([80, 256, 304])
        keys = min(msl, window) if window > 0 else msl
        want = _policy_want(keys, batch, 1, hkv, 1, cus, 256, 64, 1024)
        assert lib.pd_gqa_split_cap(batch, hkv, msl, window, cus) == want


def test_mla_policy_cap_matches_oracle_rule_and_skew_bound():
    rng = random.Random(2)
    for _ in range(2000):
        msl = rng.choice([0, 1, 2048, 16384, 65536, rng.randint(0, 200000)])
        batch = rng.choice([1, 4, 32, 128, rng.randint(0, 1000)])
        qlen = rng.randint(1, 8)
        heads = rng.choice([8, 16, 32, 128])
        cus = rng.choice([80, 256, 304])
        want = _policy_want(msl, batch, qlen, heads, 128, cus, 128, 16, 2048)
        assert lib.pd_mla_split_cap(batch, qlen, heads, msl, cus) == want


def test_policy_caps_at_the_configs():
    # GQA with sinks, window, skewed batch; MLA verify (256 compute units)
    assert lib.pd_gqa_split_cap(64, 8, 8192, 0, 256) == 8
    assert lib.pd_gqa_split_cap(64, 8, 32768, 128, 256) == 1
    assert lib.pd_gqa_split_cap(256, 8, 131072, 0, 256) == 64
    assert lib.pd_mla_split_cap(32, 4, 128, 16384, 256) == 8


def test_num_kv_splits_cap_checks_before_the_device_query():
    f = lib.num_kv_splits_cap
    assert f(-1, 1, 1, 8, 8, 128, 0, -1) == PD_ERR_INVALID
    assert f(10, 1, 0, 8, 8, 128, 0, -1) == PD_ERR_INVALID
    assert f(10, 1, 1, 12, 8, 128, 0, -1) == PD_ERR_INVALID        # Hq % Hkv
    assert f(10, 1, 1, 8, 8, 64, 0, -1) == PD_ERR_UNSUPPORTED      # no kernel for D = 64
    assert f(10, 1, 1, 8, 2, 576, 0, -1) == PD_ERR_UNSUPPORTED     # latent width needs one kv head


def test_split_cap_rejects_bad_arguments():
    assert _cap(-1, 1, 1, 1, 1, 256, 1.0, 64, 8, 0) == PD_ERR_INVALID
    assert _cap(10, 1, 0, 1, 1, 256, 1.0, 64, 8, 0) == PD_ERR_INVALID
    assert _cap(10, 1, 1, 1, 0, 256, 1.0, 64, 8, 0) == PD_ERR_INVALID
    assert _cap(10, 1, 1, 1, 1, 256, 0.0, 64, 8, 0) == PD_ERR_INVALID
    assert _cap(10, 1, 1, 1, 1, 256, 1.0, 64, 0, 0) == PD_ERR_INVALID


def test_workspace_bytes():
    assert lib.pd_workspace_bytes(64, 64, 8, 128) == 64 * 64 * 8 * 129 * 4
    assert lib.pd_workspace_bytes(128, 128, 16, 512) == 128 * 128 * 16 * 513 * 4
    assert lib.pd_workspace_bytes(64, 64, 1, 128) == 0
    assert lib.pd_workspace_bytes(0, 64, 4, 128) == 0


def _gqa(**kw):
    a = dict(q=FAKE, qsb=64 * 128, qsh=128, kv=FAKE, kvsp=8 * 16 * 256, kvsh=16 * 256, npages=10,
             bt=FAKE, btsb=4, maxb=4, sl=FAKE, sinks=NULL, window=0, scale=0.088, B=2, Hq=64,
             Hkv=8, D=128, P=16, S=1, ws=NULL, wsb=0, out=FAKE, osb=64 * 128, osh=128,
             lse=NULL, lsesb=64, stream=NULL)
    a.update(kw)
    return lib.paged_decode_gqa(*a.values())


def test_gqa_argument_checks_happen_before_any_hip_call():
    assert _gqa(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, out=NULL) == PD_OK
    assert _gqa(q=NULL) == PD_ERR_INVALID
    assert _gqa(sl=NULL) == PD_ERR_INVALID
    assert _gqa(Hq=60) == PD_ERR_INVALID                      # Hq % Hkv
    assert _gqa(B=-1) == PD_ERR_INVALID
    assert _gqa(scale=float("nan")) == PD_ERR_INVALID
    assert _gqa(scale=0.0) == PD_ERR_INVALID                  # softmax scale must be > 0
    assert _gqa(scale=-0.088) == PD_ERR_INVALID
    assert _gqa(D=64) == PD_ERR_UNSUPPORTED
    assert _gqa(P=1 << 17) == PD_ERR_UNSUPPORTED
    assert _gqa(P=(1 << 16) + 1) == PD_ERR_UNSUPPORTED
    assert _gqa(P=0) == PD_ERR_INVALID
    assert _gqa(q=FAKE + 8) == PD_ERR_ALIGN
    assert _gqa(kvsp=8 * 16 * 256 + 4) == PD_ERR_ALIGN
    assert _gqa(osh=132) == PD_ERR_ALIGN
    assert _gqa(S=4) == PD_ERR_WORKSPACE                       # no workspace
    need = lib.pd_workspace_bytes(2, 64, 4, 128)
    assert _gqa(S=4, ws=FAKE, wsb=need - 4) == PD_ERR_WORKSPACE
    assert _gqa(S=4, ws=FAKE + 4, wsb=need) == PD_ERR_ALIGN


def _gqav(**kw):
    a = dict(q=FAKE, qsr=64 * 128, qsh=128, kv=FAKE, dt=0, ks=NULL, vs=NULL, per=0,
             kvsp=8 * 16 * 256, kvsh=16 * 256,
             npages=10, bt=FAKE, btsb=4, maxb=4, sl=FAKE, real=NULL, qlen=2, sinks=NULL,
             window=0, scale=0.088, B=2, Hq=64, Hkv=8, D=128, P=16, S=1, ws=NULL, wsb=0,
             out=FAKE, osr=64 * 128, osh=128, lse=NULL, lser=64, stream=NULL)
    a.update(kw)
    return lib.paged_verify_gqa(*a.values())


def _gqavl(**kw):
    a = dict(q=FAKE, qsr=64 * 128, qsh=128, kv=FAKE, dt=0, ks=NULL, vs=NULL, per=0,
             kvsp=8 * 16 * 256, kvsh=16 * 256,
             npages=10, bt=FAKE, btsb=4, maxb=4, sl=FAKE, real=NULL, cu=FAKE, maxq=2, rows=3,
             sinks=NULL, window=0, scale=0.088, B=2, Hq=64, Hkv=8, D=128, P=16, S=1, ws=NULL,
             wsb=0, out=FAKE, osr=64 * 128, osh=128, lse=NULL, lser=64, stream=NULL)
    a.update(kw)
    return lib.paged_verify_gqa_varlen(*a.values())


def test_gqa_verify_varlen_argument_checks_happen_before_any_hip_call():
    assert _gqavl(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, out=NULL, cu=NULL) == PD_OK
    assert _gqavl(rows=0, q=NULL) == PD_OK                    # no query row at all
    assert _gqavl(cu=NULL) == PD_ERR_INVALID
    assert _gqavl(rows=-1) == PD_ERR_INVALID
    assert _gqavl(maxq=0) == PD_ERR_INVALID
    assert _gqavl(maxq=9) == PD_ERR_UNSUPPORTED                # max_qlen * G = 72 > 64
    assert _gqavl(S=4) == PD_ERR_WORKSPACE
    need = lib.pd_workspace_bytes(3, 64, 4, 128)               # rows = total_rows
    assert _gqavl(S=4, ws=FAKE, wsb=need - 4) == PD_ERR_WORKSPACE
    assert _gqavl(S=4, ws=FAKE + 4, wsb=need) == PD_ERR_ALIGN


def test_gqa_verify_argument_checks_happen_before_any_hip_call():
    assert _gqav(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, out=NULL) == PD_OK
    assert _gqav(qlen=0) == PD_ERR_INVALID
    assert _gqav(q=NULL) == PD_ERR_INVALID
    assert _gqav(scale=float("inf")) == PD_ERR_INVALID
    # qlen * G = 72 > 64: accepted (two launches of 5 and 4 tokens); the
    # missing workspace stops it before any HIP call
    assert _gqav(qlen=9, S=4) == PD_ERR_WORKSPACE
    assert _gqav(qlen=9, Hq=8 * 65, Hkv=8) == PD_ERR_UNSUPPORTED   # G = 65
    assert _gqa(Hq=8 * 65, Hkv=8) == PD_ERR_UNSUPPORTED       # G = 65
    assert _gqav(qlen=4, Hq=32, D=64) == PD_ERR_UNSUPPORTED
    assert _gqav(osr=64 * 128 + 4) == PD_ERR_ALIGN
    assert _gqav(S=4) == PD_ERR_WORKSPACE
    need = lib.pd_workspace_bytes(2 * 2, 64, 4, 128)           # rows = B * qlen
    assert _gqav(S=4, ws=FAKE, wsb=need - 4) == PD_ERR_WORKSPACE
    assert _gqav(S=4, ws=FAKE + 4, wsb=need) == PD_ERR_ALIGN
    # the query rows of a unit must be addressable with a 32-bit byte offset
    assert _gqav(qsr=(1 << 30)) == PD_ERR_UNSUPPORTED
    assert _gqav(dt=3) == PD_ERR_INVALID                      # unknown cache type
    assert _gqav(dt=1, per=2) == PD_ERR_INVALID
    assert _gqav(dt=1, kvsh=16 * 256 + 8) == PD_ERR_ALIGN     # FP8 rows: 16-byte strides
    assert _gqav(dt=1, S=4) == PD_ERR_WORKSPACE


def _app(**kw):
    a = dict(s0=FAKE, s0t=8 * 128, s0h=128, n0=128, s1=FAKE, s1t=8 * 128, s1h=128, n1=128, eb=2,
             cache=FAKE, csp=8 * 16 * 256, csh=16 * 256, cst=256, npages=10, bt=FAKE, btsb=4,
             maxb=4, sl=FAKE, qlen=1, B=2, H=8, P=16, stream=NULL)
    a.update(kw)
    return lib.paged_kv_append(*a.values())


def test_kv_append_argument_checks_happen_before_any_hip_call():
    assert _app(B=0, s0=NULL, s1=NULL, n1=0, cache=NULL, bt=NULL, sl=NULL) == PD_OK
    assert _app(qlen=0) == PD_ERR_INVALID
    assert _app(eb=4) == PD_ERR_INVALID
    assert _app(s1=NULL) == PD_ERR_INVALID                     # elements given, no source
    assert _app(n1=0) == PD_ERR_INVALID                        # source given, no elements
    assert _app(cache=NULL) == PD_ERR_INVALID
    assert _app(cst=200) == PD_ERR_INVALID                     # K | V do not fit a token row
    assert _app(n0=4, n1=4, cst=8) == PD_ERR_ALIGN             # 8-byte rows
    assert _app(s0=FAKE + 8) == PD_ERR_ALIGN
    assert _app(csh=16 * 256 + 4) == PD_ERR_ALIGN
    assert _app(eb=1, n0=8, n1=8, cst=16) == PD_ERR_ALIGN       # FP8: 8-byte rows


def _mla(**kw):
    a = dict(q=FAKE, qsr=128 * 576, qsh=576, kv=FAKE, dt=0, sp=16 * 576, st=576, npages=10,
             ks=NULL, bt=FAKE, btsb=4, maxb=4, sl=FAKE, real=NULL, qlen=4, scale=0.07, B=2,
             H=128, Lk=576, Lv=512, P=16, S=1, ws=NULL, wsb=0, out=FAKE, osr=128 * 512,
             osh=512, lse=FAKE, lser=128, stream=NULL)
    a.update(kw)
    return lib.paged_verify_mla(*a.values())


def test_mla_argument_checks_happen_before_any_hip_call():
    assert _mla(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, out=NULL) == PD_OK
    assert _mla(kv=NULL) == PD_ERR_INVALID
    assert _mla(qlen=0) == PD_ERR_INVALID
    assert _mla(dt=7) == PD_ERR_INVALID
    assert _mla(scale=-0.07) == PD_ERR_INVALID
    assert _mla(Lk=512) == PD_ERR_UNSUPPORTED
    assert _mla(Lv=256) == PD_ERR_UNSUPPORTED
    assert _mla(P=1 << 17) == PD_ERR_UNSUPPORTED
    assert _mla(P=0) == PD_ERR_INVALID
    assert _mla(out=FAKE + 2) == PD_ERR_ALIGN
    assert _mla(dt=1, st=576 + 8) == PD_ERR_ALIGN              # fp8 rows need 16 B
    assert _mla(S=2) == PD_ERR_WORKSPACE
    # page and token strides span under 4 GiB (32 x 32-bit offsets in the kernel)
    assert _mla(sp=1 << 31) == PD_ERR_UNSUPPORTED                # 4 GiB of bf16
    assert _mla(sp=(1 << 31) - 8, S=2) == PD_ERR_WORKSPACE     # passes the stride check, launches nothing
    assert _mla(dt=1, sp=1 << 32) == PD_ERR_UNSUPPORTED          # 4 GiB of fp8 codes
    assert _mla(st=1 << 31) == PD_ERR_UNSUPPORTED


def test_merge_argument_checks():
    f = lib.merge_splits
    assert f(FAKE, 0, 8, 2, 128, NULL, FAKE, 1024, 128, NULL, 8, NULL) == PD_OK
    assert f(NULL, 4, 8, 2, 128, NULL, FAKE, 1024, 128, NULL, 8, NULL) == PD_ERR_INVALID
    assert f(FAKE, 4, 8, 2, 96, NULL, FAKE, 1024, 128, NULL, 8, NULL) == PD_ERR_UNSUPPORTED
    assert f(FAKE, 4, 8, 0, 128, NULL, FAKE, 1024, 128, NULL, 8, NULL) == PD_ERR_INVALID
    assert f(FAKE, 4, 8, 2, 128, NULL, FAKE + 2, 1024, 128, NULL, 8, NULL) == PD_ERR_ALIGN


def _gqap(**kw):
    a = dict(q=FAKE, qsb=64 * 128, qsh=128, kv=FAKE, kvsp=8 * 16 * 256, kvsh=16 * 256, npages=10,
             bt=FAKE, btsb=4, maxb=4, sl=FAKE, window=0, scale=0.088, B=2, Hq=64, Hkv=8, D=128,
             P=16, S=1, ws=FAKE, wsb=2 * 64 * 129 * 4, stream=NULL)
    a.update(kw)
    return lib.paged_decode_gqa_partials(*a.values())


def test_gqa_partials_argument_checks_happen_before_any_hip_call():
    assert _gqap(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, ws=NULL, wsb=0) == PD_OK
    assert _gqap(q=NULL) == PD_ERR_INVALID
    assert _gqap(S=0) == PD_ERR_INVALID
    assert _gqap(D=64) == PD_ERR_UNSUPPORTED
    # a partial slot per (row, head, split) even with S = 1: no direct output
    assert _gqap(ws=NULL, wsb=0) == PD_ERR_WORKSPACE
    assert _gqap(wsb=2 * 64 * 129 * 4 - 4) == PD_ERR_WORKSPACE
    assert _gqap(ws=FAKE + 4) == PD_ERR_ALIGN
    assert _gqap(S=3, wsb=lib.pd_workspace_bytes(2, 64, 3, 128) - 4) == PD_ERR_WORKSPACE


def _gqavp(**kw):
    a = dict(q=FAKE, qsr=64 * 128, qsh=128, kv=FAKE, dt=0, ks=NULL, vs=NULL, per=0,
             kvsp=8 * 16 * 256, kvsh=16 * 256, npages=10, bt=FAKE, btsb=4, maxb=4, sl=FAKE,
             real=NULL, cu=NULL, qlen=2, rows=-1, window=0, scale=0.088, B=2, Hq=64, Hkv=8,
             D=128, P=16, S=1, ws=FAKE, wsb=4 * 64 * 129 * 4, stream=NULL)
    a.update(kw)
    return lib.paged_verify_gqa_partials(*a.values())


def test_gqa_verify_partials_argument_checks_happen_before_any_hip_call():
    assert _gqavp(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, ws=NULL, wsb=0) == PD_OK
    assert _gqavp(qlen=0) == PD_ERR_INVALID
    assert _gqavp(qlen=9) == PD_ERR_WORKSPACE                  # sliced; 18 rows need more
    assert _gqavp(dt=1, per=2) == PD_ERR_INVALID
    # fixed qlen: rows = B * qlen, total_rows ignored
    assert _gqavp(wsb=4 * 64 * 129 * 4 - 4) == PD_ERR_WORKSPACE
    assert _gqavp(ws=NULL, wsb=0) == PD_ERR_WORKSPACE
    # varlen: rows = total_rows
    assert _gqavp(cu=FAKE, rows=-1) == PD_ERR_INVALID
    assert _gqavp(cu=FAKE, rows=0, q=NULL, ws=NULL) == PD_OK   # no query row at all
    assert _gqavp(cu=FAKE, rows=3, wsb=3 * 64 * 129 * 4 - 4) == PD_ERR_WORKSPACE
    assert _gqavp(cu=FAKE, rows=3, ws=FAKE + 4, wsb=3 * 64 * 129 * 4) == PD_ERR_ALIGN


def _mlap(**kw):
    a = dict(q=FAKE, qsr=128 * 576, qsh=576, kv=FAKE, dt=0, sp=16 * 576, st=576, npages=10,
             ks=NULL, bt=FAKE, btsb=4, maxb=4, sl=FAKE, real=NULL, qlen=4, scale=0.07, B=2,
             H=128, Lk=576, Lv=512, P=16, S=1, ws=FAKE, wsb=8 * 128 * 513 * 4, stream=NULL)
    a.update(kw)
    return lib.paged_verify_mla_partials(*a.values())


def test_mla_partials_argument_checks_happen_before_any_hip_call():
    assert _mlap(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, ws=NULL, wsb=0) == PD_OK
    assert _mlap(kv=NULL) == PD_ERR_INVALID
    assert _mlap(qlen=0) == PD_ERR_INVALID
    assert _mlap(Lv=256) == PD_ERR_UNSUPPORTED
    assert _mlap(ws=NULL, wsb=0) == PD_ERR_WORKSPACE           # S = 1 still writes partials
    assert _mlap(wsb=8 * 128 * 513 * 4 - 4) == PD_ERR_WORKSPACE
    assert _mlap(ws=FAKE + 4) == PD_ERR_ALIGN
    assert _mlap(S=2, wsb=lib.pd_workspace_bytes(8, 128, 2, 512) - 4) == PD_ERR_WORKSPACE


def _noalloc(**kw):
    a = dict(q=FAKE, qsr=64 * 128, qsh=128, kv=FAKE, dt=0, ks=NULL, vs=NULL, ph=0,
             kvsp=8 * 16 * 256, kvsh=16 * 256, npages=10, bt=FAKE, btsb=4, maxb=4, sl=FAKE,
             real=NULL, qlen=2, sinks=NULL, window=0, scale=0.088, B=2, Hq=64, Hkv=8, D=128,
             P=16, S=1, out=FAKE, osr=64 * 128, osh=128, lse=NULL, lsesr=64, stream=NULL)
    a.update(kw)
    return lib.paged_verify_gqa_noalloc(*a.values())


def test_noalloc_checks_happen_before_the_scratch_lookup():
    # every refusal below comes from the host checks, before any HIP call
    assert _noalloc(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, out=NULL) == PD_OK
    assert _noalloc(q=NULL) == PD_ERR_INVALID
    assert _noalloc(Hq=60) == PD_ERR_INVALID
    assert _noalloc(scale=-1.0) == PD_ERR_INVALID
    assert _noalloc(P=0) == PD_ERR_INVALID
    assert _noalloc(D=64) == PD_ERR_UNSUPPORTED
    assert _noalloc(q=FAKE + 8) == PD_ERR_ALIGN
    # partials of 128 rows x 64 heads x 16 splits x 129 fp32 exceed the 64 MiB scratch
    assert _noalloc(B=64, S=16) == PD_ERR_WORKSPACE
    assert _noalloc(B=64 * 16, S=2, maxb=1) == PD_ERR_WORKSPACE


def _gqaa(**kw):
    a = dict(q=FAKE, qsr=64 * 128, qsh=128, kv=FAKE, dt=0, ks=NULL, vs=NULL, per=0,
             kvsp=8 * 16 * 256, kvsh=16 * 256,
             npages=10, bt=FAKE, btsb=4, maxb=4, sl=FAKE, real=NULL, qlen=2,
             kn=FAKE, knr=8 * 128, knh=128, vn=FAKE + 4096, vnr=8 * 128, vnh=128,
             sinks=NULL, window=0, scale=0.088, B=2, Hq=64, Hkv=8, D=128, P=16, S=1, ws=NULL,
             wsb=0, out=FAKE, osr=64 * 128, osh=128, lse=NULL, lser=64, stream=NULL)
    a.update(kw)
    return lib.paged_verify_gqa_append(*a.values())


def test_fused_append_argument_checks_happen_before_any_hip_call():
    assert _gqaa(B=0, q=NULL, kv=NULL, bt=NULL, sl=NULL, out=NULL, kn=NULL, vn=NULL) == PD_OK
    assert _gqaa(kn=NULL) == PD_ERR_INVALID
    assert _gqaa(vn=NULL) == PD_ERR_INVALID
    assert _gqaa(knr=-128) == PD_ERR_INVALID
    assert _gqaa(kn=FAKE + 8) == PD_ERR_ALIGN                 # rows in 16-byte chunks
    assert _gqaa(vnh=128 + 4) == PD_ERR_ALIGN
    assert _gqaa(dt=1, knr=8 * 128 + 8) == PD_ERR_ALIGN       # FP8: strides of 16 codes
    assert _gqaa(qlen=9, S=4) == PD_ERR_WORKSPACE              # qlen * G = 72: sliced, as verify
    assert _gqaa(knr=1 << 31) == PD_ERR_UNSUPPORTED
    assert _gqaa(S=4) == PD_ERR_WORKSPACE
    need = lib.pd_workspace_bytes(2 * 2, 64, 4, 128)
    assert _gqaa(S=4, ws=FAKE + 4, wsb=need) == PD_ERR_ALIGN

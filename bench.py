"""Benchmark of the paged split-KV decode hot path on one MI355X.

Default workload: the GQA decode-with-sinks configuration (B=64 requests,
Hq=64, Hkv=8, head_dim 128, 16-token HND pages in a 40000-page pool, seq_lens
uniform in [1024, 8192], per-head sinks), seeded synthetic bf16 data resident
in HBM.  One step is one full paged_decode_gqa call: the split decode kernel
plus the split merge.

Printed: ONE JSON line with KV-read GB/s (algorithmic K+V bytes of the
attended keys / time per call), the roofline of the dominant kernel measured
with HIP events on the launch stream, and the fp64 CPU oracle's rate on the
same inputs.  ``--config`` selects another workload (gqa_window, gqa_skewed,
tiny_gqa, gqa_verify, gqa_verify_varlen, gqa_sinks_fp8, kv_append, mla_verify,
mla_verify_fp8).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-read GB/s (% of HBM peak) and µs/call for paged decode, GQA and MLA verify"
HBM_PEAK_GBS = 8000.0
GRAPH_CALLS = 50      # calls per captured graph for launch-bound kernels
# The GPU clock climbs over the first ~100 ms of load after idle: the default
# warmup runs at least this long.
WARMUP_AUTO_S = 0.5
BF16_MFMA_PEAK_TFLOPS = 2500.0


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warmup steps; by default as many as run in %.1f s (at least "
                        "10), so the GPU clock has left its idle state before timing" % WARMUP_AUTO_S)
    p.add_argument("--config", default="gqa_sinks")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--splits", type=int, default=0, help="override the split cap")
    p.add_argument("--page-size", type=int, default=0,
                   help="decode / verify configs: store the same workload in pages of this many "
                        "tokens (a power of two; a GQA pool then holds exactly the pages in use)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run one plain device copy of this many MiB (a "
                        "known-size reference for hardware byte counters)")
    return p.parse_args()


def _kernel_split(S, step, partials, merge):
    """(kernel, rest) callables whose sequence is one step: with S > 1 the
    attention kernel alone (the partials-only entry) and then the merge; with
    S = 1 the step itself is the one kernel."""
    if S > 1:
        return partials, merge
    return step, (lambda: None)


def _gqa_case(name, torch, pd, splits, page_size=0):
    from synth import gqa_workload

    fp8 = name.endswith("_fp8")
    base = name[:-4] if fp8 else name
    w = gqa_workload(base, page_size=page_size, pool="tight") if page_size else gqa_workload(base)
    pool = f"{w.num_pages}-page pool" if page_size else "40000-page pool"
    vals = w.values("cuda", poison=False, fp8=fp8)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    S = splits or pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    out = torch.empty((w.rows, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.rows, w.Hq), dtype=torch.float32, device="cuda")
    ws = pd.alloc_workspace(w.rows, w.Hq, max(S, 2), w.D, "cuda")

    if w.qlen > 1 or w.real_seq_lens is not None or fp8:
        real = None if w.real_seq_lens is None else torch.from_numpy(w.real_seq_lens).cuda()

        def verify_step():
            pd.paged_verify_gqa(vals["q"], vals["kv"], bt, sl, w.qlen, w.sm_scale,
                                sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                                num_kv_splits=S, workspace=ws, out=out, lse=lse,
                                k_scale=vals.get("k_scale"), v_scale=vals.get("v_scale"))

        if fp8:
            desc = ("GQA decode with sinks on an FP8 E4M3FN cache (per-kv-head K and V "
                    f"scales): B=64, Hq=64, Hkv=8, D=128, page {w.P} HND, seq_lens U[1024,8192], "
                    f"{pool}")
        else:
            desc = (f"GQA causal verify with sinks: B={w.B}, qlen={w.qlen}, Hq={w.Hq}, "
                    f"Hkv={w.Hkv}, D={w.D}, page {w.P} HND bf16, seq_lens U[1024,8192], "
                    f"real length L - U{{0,1}}, {pool}")
        def verify_kernel():
            pd.paged_verify_gqa_partials(vals["q"], vals["kv"], bt, sl, w.qlen, w.sm_scale,
                                         window=w.window, real_seq_lens=real, num_kv_splits=S,
                                         workspace=ws, k_scale=vals.get("k_scale"),
                                         v_scale=vals.get("v_scale"))

        def verify_rest():
            pd.merge_splits(ws, w.rows, w.Hq, S, w.D, sinks=vals["sinks"], out=out, lse=lse)

        kernel, rest = _kernel_split(S, verify_step, verify_kernel, verify_rest)
        return dict(w=w, vals=vals, S=S, step=verify_step, kernel=kernel, rest=rest,
                    kv_bytes=w.kv_bytes() // (2 if fp8 else 1), flops=w.flops(), desc=desc,
                    kind="gqa_fp8" if fp8 else "gqa_verify", kernel_name="gqa_decode_kernel")

    def step():
        pd.paged_decode_gqa(vals["q"], vals["kv"], bt, sl, w.sm_scale, sinks=vals["sinks"],
                            window=w.window, num_kv_splits=S, workspace=ws, out=out, lse=lse)

    def kernel_only():
        pd.paged_decode_gqa_partials(vals["q"], vals["kv"], bt, sl, w.sm_scale, window=w.window,
                                     num_kv_splits=S, workspace=ws)

    def rest():
        pd.merge_splits(ws, w.B, w.Hq, S, w.D, sinks=vals["sinks"], out=out, lse=lse)

    desc = {
        "gqa_sinks": f"GQA decode with sinks: B=64, Hq=64, Hkv=8, D=128, page {w.P} HND bf16, "
                     f"seq_lens U[1024,8192], {pool}",
        "gqa_window": f"sliding-window GQA decode: B=64, Hq=64, Hkv=8, D=128, page {w.P}, "
                      "window 128, seq_lens U[4096,32768]",
        "gqa_skewed": f"skewed long-context GQA decode: B=256, Hq=32, Hkv=8, D=128, page {w.P}, "
                      "seq_lens log-uniform [16,131072] with 4 empty",
        "tiny_gqa": "tiny GQA decode: B=3, seq_lens [30,32,70], page 32",
    }[name]

    kernel, rest = _kernel_split(S, step, kernel_only, rest)
    return dict(w=w, vals=vals, S=S, step=step, kernel=kernel, rest=rest,
                kv_bytes=w.kv_bytes(), flops=w.flops(), desc=desc, kind="gqa",
                kernel_name="gqa_decode_kernel")


def _varlen_case(torch, pd, splits, page_size=0):
    """The GQA verify config with a query length per request, U{1, 2}
    (seeded), rows indexed by cumulative query lengths."""
    from synth import gqa_workload

    w = gqa_workload("gqa_verify", page_size=page_size, pool="tight") if page_size else \
        gqa_workload("gqa_verify")
    vals = w.values("cuda", poison=False)
    rng = np.random.default_rng(2016)
    qlens = rng.integers(1, w.qlen + 1, size=w.B)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    rows = np.concatenate([b * w.qlen + np.arange(n) for b, n in enumerate(qlens)])
    q = vals["q"][torch.from_numpy(rows).cuda()].contiguous()
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    real = torch.from_numpy(w.real_seq_lens).cuda()
    cu_d = torch.from_numpy(cu).cuda()
    S = splits or pd.gqa_split_cap(w.B, w.Hkv, int(w.seq_lens.max()), w.window)
    total = int(cu[-1])
    out = torch.empty((total, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((total, w.Hq), dtype=torch.float32, device="cuda")
    ws = pd.alloc_workspace(total, w.Hq, max(S, 2), w.D, "cuda")

    def step():
        pd.paged_verify_gqa_varlen(q, vals["kv"], bt, sl, cu_d, w.qlen, w.sm_scale,
                                   sinks=vals["sinks"], window=w.window, real_seq_lens=real,
                                   num_kv_splits=S, workspace=ws, out=out, lse=lse)

    def kernel_only():
        pd.paged_verify_gqa_partials(q, vals["kv"], bt, sl, w.qlen, w.sm_scale, window=w.window,
                                     real_seq_lens=real, cu_seqlens_q=cu_d, num_kv_splits=S,
                                     workspace=ws)

    def rest():
        pd.merge_splits(ws, total, w.Hq, S, w.D, sinks=vals["sinks"], out=out, lse=lse)

    kernel, rest = _kernel_split(S, step, kernel_only, rest)
    # keys of request b: rows t < n_b see [0, min(L, L_real)) at most (no window)
    keys = sum(max(min(int(L), int(Lr)), 0) for L, Lr in zip(w.seq_lens, w.real_seq_lens))
    desc = (f"GQA causal verify, variable query length U{{1,2}} per request (cumulative query "
            f"lengths, {total} rows): B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, page {w.P} HND "
            f"bf16, seq_lens U[1024,8192], real length L - U{{0,1}}")
    return dict(w=w, vals=vals, S=S, step=step, kernel=kernel, rest=rest,
                kv_bytes=keys * w.Hkv * 2 * w.D * 2, flops=w.flops(), desc=desc,
                kind="gqa_varlen", kernel_name="gqa_decode_kernel",
                extra=dict(q=q, cu=cu, qlens=qlens))


def _append_case(torch, pd):
    from synth import gqa_workload

    w = gqa_workload("gqa_sinks")
    vals = w.values("cuda", poison=False)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    g = torch.Generator(device="cuda").manual_seed(99)
    k = torch.randn((w.B, w.Hkv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((w.B, w.Hkv, w.D), generator=g, device="cuda").to(torch.bfloat16)

    def step():
        pd.paged_kv_append(vals["kv"], bt, sl, k, v)

    desc = ("KV append of the current token: B=64, Hkv=8, D=128, K and V into the 16-token "
            "HND pages of the 40000-page decode pool through the block table")
    moved = 2 * w.B * w.Hkv * 2 * w.D * 2          # read + write, K and V
    # The step loop is bound by the host-side binding, so the kernel's own
    # time comes from a HIP graph of GRAPH_CALLS appends replayed back to back.
    return dict(w=w, vals=vals, S=1, step=step, kernel=None, rest=None, kv_bytes=moved,
                graph_calls=GRAPH_CALLS,
                flops=0, desc=desc, kind="append", kernel_name="kv_append_kernel",
                extra=dict(k=k, v=v))


def _mla_case(fp8, torch, pd, splits, page_size=0):
    from synth import mla_workload

    w = mla_workload("mla_verify", page_size=page_size or None)
    vals = w.values("cuda", poison=False, fp8=fp8)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    real = torch.from_numpy(w.real_seq_lens).cuda()
    k_scale = torch.tensor([vals["k_scale"]], dtype=torch.float32, device="cuda")
    S = splits or pd.mla_split_cap(w.B, w.qlen, w.H, int(w.seq_lens.max()))
    out = torch.empty((w.rows, w.H, w.Lv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.rows, w.H), dtype=torch.float32, device="cuda")
    ws = pd.alloc_workspace(w.rows, w.H, max(S, 2), w.Lv, "cuda")

    def step():
        pd.paged_verify_mla(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                            head_dim_v=w.Lv, k_scale=k_scale if fp8 else None,
                            num_kv_splits=S, workspace=ws, out=out, lse=lse)

    def kernel_only():
        pd.paged_verify_mla_partials(vals["q"], vals["kv"], bt, sl, real, w.qlen, w.sm_scale,
                                     head_dim_v=w.Lv, k_scale=k_scale if fp8 else None,
                                     num_kv_splits=S, workspace=ws)

    def rest():
        pd.merge_splits(ws, w.rows, w.H, S, w.Lv, out=out, lse=lse)

    kernel, rest = _kernel_split(S, step, kernel_only, rest)
    desc = (f"MLA causal verify: B=32, qlen=4, H=128, Lk=576, Lv=512, page {w.P}, "
            f"seq_lens U[2048,16384], {'fp8 e4m3fn' if fp8 else 'bf16'} latent cache")
    return dict(w=w, vals=vals, S=S, step=step, kernel=kernel, rest=rest,
                kv_bytes=w.kv_bytes(1 if fp8 else 2), flops=w.flops(), desc=desc,
                kind="mla_fp8" if fp8 else "mla", kernel_name="mla_verify_kernel")


def _profiled_traffic(kernel, config):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>__<config>.md: calibrated FETCH_SIZE + WRITE_SIZE), or
    None when there is none or the kernel's sources changed since."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{kernel}__{config}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in (
                "traffic_bytes_per_launch", "kernel_source_sha256_16", "kernel_sources"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    try:
        h = hashlib.sha256()
        for f in fields["kernel_sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] != fields["kernel_source_sha256_16"]:
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, OSError, ValueError):
        return None


def _cpu_baseline(case, budget_s=20.0, min_s=10.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    inputs: whole requests in order, in repeated passes, for about min_s to
    budget_s of work."""
    import threadpoolctl
    import torch

    import oracle

    w, vals = case["w"], case["vals"]
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    if case["kind"] == "append":
        # the pages the appends write, as a compact pool
        pos = w.seq_lens.astype(np.int64) - 1
        pages = w.block_table[np.arange(w.B), pos // w.P]
        remap = {int(p): i for i, p in enumerate(np.unique(pages))}
        idx = torch.from_numpy(np.unique(pages)).cuda()
        cache = vals["kv"].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
        bt2 = np.full_like(w.block_table, -1)
        bt2[np.arange(w.B), pos // w.P] = [remap[int(p)] for p in pages]
        k = case["extra"]["k"].view(torch.int16).cpu().numpy().view(np.uint16)
        v = case["extra"]["v"].view(torch.int16).cpu().numpy().view(np.uint16)
        reps, t_total = 0, 0.0
        while t_total < min_s:
            t0 = time.perf_counter()
            oracle.kv_append(cache, bt2, w.seq_lens, 1, k, v)
            t_total += time.perf_counter() - t0
            reps += 1
        return {"value": round(case["kv_bytes"] * reps / t_total / 1e9, 4), "unit": "GB/s",
                "cores": 1, "kind": "oracle",
                "sample": f"all {w.B} requests' appends into a compact pool of their target "
                          f"pages, {reps} calls in {t_total:.1f} s, NumPy"}
    done_bytes = 0
    t_total = 0.0
    n_req = 0
    step = 0
    # whole requests in order, in repeated passes, until at least min_s of
    # oracle time (and at most budget_s, or 50 passes)
    while True:
        if t_total > budget_s or (step >= w.B and t_total >= min_s) or step >= 50 * w.B:
            break
        b = step % w.B
        step += 1
        bt = w.block_table[b:b + 1]
        used = np.unique(bt[bt >= 0])
        if used.size == 0:
            continue
        remap = np.full(w.num_pages, -1, np.int64)
        remap[used] = np.arange(used.size)
        idx = torch.from_numpy(used).cuda()
        kvt = vals["kv"].index_select(0, idx)
        kv = (kvt.cpu().numpy() if kvt.dtype == torch.uint8
              else kvt.view(torch.int16).cpu().numpy().view(np.uint16))
        bt2 = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
        if case["kind"] == "gqa":
            q = vals["q"][b:b + 1].view(torch.int16).cpu().numpy().view(np.uint16)
            sinks = None if vals["sinks"] is None else vals["sinks"].cpu().numpy()
            t0 = time.perf_counter()
            oracle.gqa_decode(q, kv, bt2, w.seq_lens[b:b + 1], w.sm_scale, sinks=sinks,
                              window=w.window)
            t_total += time.perf_counter() - t0
            lo = max(int(w.seq_lens[b]) - w.window, 0) if w.window > 0 else 0
            done_bytes += (int(w.seq_lens[b]) - lo) * w.Hkv * 2 * w.D * 2
        elif case["kind"] == "gqa_varlen":
            cu, qlens = case["extra"]["cu"], case["extra"]["qlens"]
            q = case["extra"]["q"][int(cu[b]):int(cu[b + 1])].view(torch.int16).cpu().numpy()
            sinks = None if vals["sinks"] is None else vals["sinks"].cpu().numpy()
            t0 = time.perf_counter()
            oracle.gqa_verify_varlen(q.view(np.uint16), kv, bt2, w.seq_lens[b:b + 1],
                                     np.array([0, int(qlens[b])]), w.sm_scale, sinks=sinks,
                                     window=w.window, real_seq_lens=w.real_seq_lens[b:b + 1])
            t_total += time.perf_counter() - t0
            done_bytes += max(min(int(w.seq_lens[b]), int(w.real_seq_lens[b])), 0) * w.Hkv * 2 * w.D * 2
        elif case["kind"] in ("gqa_verify", "gqa_fp8"):
            fp8 = case["kind"] == "gqa_fp8"
            rows = slice(b * w.qlen, (b + 1) * w.qlen)
            q = vals["q"][rows].view(torch.int16).cpu().numpy().view(np.uint16)
            sinks = None if vals["sinks"] is None else vals["sinks"].cpu().numpy()
            real = None if w.real_seq_lens is None else w.real_seq_lens[b:b + 1]
            scales = {}
            if fp8:
                scales = dict(kv_dtype="fp8_e4m3fn",
                              k_scale=vals["k_scale"].cpu().numpy().astype(np.float64),
                              v_scale=vals["v_scale"].cpu().numpy().astype(np.float64))
            t0 = time.perf_counter()
            oracle.gqa_verify(q, kv, bt2, w.seq_lens[b:b + 1], w.qlen, w.sm_scale,
                              sinks=sinks, window=w.window, real_seq_lens=real, **scales)
            t_total += time.perf_counter() - t0
            lo, hi = w.key_range(b)
            done_bytes += max(hi - lo, 0) * w.Hkv * 2 * w.D * (1 if fp8 else 2)
        else:
            rows = slice(b * w.qlen, (b + 1) * w.qlen)
            q = vals["q"][rows].view(torch.int16).cpu().numpy().view(np.uint16)
            fp8 = case["kind"] == "mla_fp8"
            t0 = time.perf_counter()
            oracle.mla_verify(q, kv, bt2, w.seq_lens[b:b + 1], w.real_seq_lens[b:b + 1],
                              w.qlen, w.sm_scale, w.Lv,
                              kv_dtype="fp8_e4m3fn" if fp8 else "bf16",
                              k_scale=vals["k_scale"])
            t_total += time.perf_counter() - t0
            done_bytes += w.request_keys(b) * w.Lk * (1 if fp8 else 2)
        n_req += 1
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_req} oracle calls, {n_req / w.B:.1f} passes over the {w.B} requests "
                      f"({done_bytes / 1e6:.1f} MB of KV) in {t_total:.1f} s, fp64 NumPy"}


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); multi-GPU sharding is a design note, not a code path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_split_kv_decode_amd as pd

    torch.cuda.init()
    name = args.config
    if args.page_size and name in ("kv_append", "tiny_gqa"):
        print("bench.py: --page-size applies to the decode and verify configs only",
              file=sys.stderr)
        sys.exit(2)
    if name in ("mla_verify", "mla_verify_fp8"):
        case = _mla_case(name.endswith("fp8"), torch, pd, args.splits, args.page_size)
        if args.page_size:
            name = f"{name}_p{args.page_size}"
    elif name == "kv_append":
        case = _append_case(torch, pd)
    elif name == "gqa_verify_varlen":
        case = _varlen_case(torch, pd, args.splits, args.page_size)
        if args.page_size:
            name = f"{name}_p{args.page_size}"
    else:
        case = _gqa_case(name, torch, pd, args.splits, args.page_size)
        if args.page_size:
            name = f"{name}_p{args.page_size}"
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    eager_step = case["step"]

    if args.warmup is not None:
        for _ in range(args.warmup):
            case["step"]()
    else:
        args.warmup = 0
        t_w = time.perf_counter()
        while args.warmup < 10 or time.perf_counter() - t_w < WARMUP_AUTO_S:
            for _ in range(10):
                case["step"]()
            args.warmup += 10
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        case["step"]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    print(f"# timed {args.steps} steps in {wall:.3f} s wall", file=sys.stderr)

    # dominant kernel alone: HIP events recorded on the launch stream right
    # around each launch of the split decode kernel
    kernel_ms = []
    if case.get("graph_calls"):
        n_calls = case["graph_calls"]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(n_calls):
                eager_step()
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, args.steps // n_calls)
        gstream = torch.cuda.current_stream()
        ev0.record(gstream)
        for _ in range(reps):
            graph.replay()
        ev1.record(gstream)
        torch.cuda.synchronize()
        kernel_ms = [ev0.elapsed_time(ev1) / (reps * n_calls)]
    elif case["kernel"] is not None:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            case["kernel"]()
            b.record(stream)
            case["rest"]()
        torch.cuda.synchronize()
        kernel_ms = [a.elapsed_time(b) for a, b in evs]
    else:
        kernel_ms = [ms_per_step]
    k_ms = float(np.mean(kernel_ms))

    kv = case["kv_bytes"]
    value = kv / (ms_per_step * 1e-3) / 1e9
    if case["kind"] in ("gqa", "gqa_verify", "gqa_fp8", "gqa_varlen", "append"):
        roof = {"bound": "hbm", "achieved": round(kv / (k_ms * 1e-3) / 1e9, 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(case["flops"] / (k_ms * 1e-3) / 1e12, 2),
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = _profiled_traffic(case["kernel_name"], name)
    roof["kernel"] = case["kernel_name"]
    roof["kernel_us"] = round(k_ms * 1e3, 2)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# calibration copy: {n} bytes read, {n} bytes written", file=sys.stderr)
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(case)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": case["desc"],
            "name": name,
            "num_kv_splits": case["S"],
            "kv_bytes_per_call": kv,
            "us_per_call": round(ms_per_step * 1e3, 2),
            "hbm_frac_per_call": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""Benchmark of the drafter block-attention hot path on one MI355X.

Default workload: 8 requests x 8 draft tokens, 24 query / 4 KV heads, head_dim 64,
context 32768 tokens per request (512 HND pages of 64 each, 4096 pages shuffled
across a 5000-page bf16 pool), per-head q/k RMSNorm + NeoX RoPE in the kernel.

A step is one call of drafter_attn_qknorm (one kernel launch).  The same run also
captures one call in a HIP graph and times its replays the same way
(``graph_us_per_call``); ``--graph`` makes the replays the headline instead.
Inputs are resident in HBM before timing starts.  Before every step (warm-up and
timed) an untimed kernel reads a 1 GiB buffer so that neither the L2 nor the 256 MB
Infinity Cache holds the 268 MB of K/V the call reads: each timed call streams its
pages from HBM.  (The flush only reads, so it leaves no dirty lines whose write-back
would compete with the timed call.)  Each call is bracketed by HIP events on the
stream it is launched on; ms_per_step is their mean (the median and p10/p90 are
reported too).  ``--hot`` times back-to-back calls without the flush instead
(reported, not the headline).

value = algorithmic K/V bytes per call / mean call time (GB/s): every context
K and V element is read exactly once, sum_r L_r * Hkv * 64 * 2 * 2 bytes.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 5])
    ap.add_argument("--hot", action="store_true", help="no cache flush between calls")
    ap.add_argument("--graph", action="store_true",
                    help="headline from replays of one call captured in a HIP graph instead of direct launches "
                         "(every run times both modes and reports the other beside the headline)")
    ap.add_argument("--yarn", action="store_true",
                    help="YaRN-scaled rotation (factor 4, 4096-token original context, ramp 1..32) in the qknorm "
                         "call; reported beside the headline, not instead of it")
    ap.add_argument("--large", action="store_true",
                    help="instead of the headline line: one line per large context (131k and 1M tokens, "
                         "24/4 and 96/16 heads; one request of 32k and 131k tokens), pools drawn on the device")
    ap.add_argument("--mixed", action="store_true",
                    help="instead of the headline line: the length-aware split schedule against the static plan "
                         "alone, on mixed-length workloads (one line per workload)")
    ap.add_argument("--phases", action="store_true",
                    help="instead of the headline line: phase timestamps of cold calls (measurement build with "
                         "DA_PHASE_TRACE), one line per workload")
    ap.add_argument("--ceiling", action="store_true",
                    help="instead of the headline line: the attention against the page-stream probe, which reads "
                         "the same tiles with the same grid and does no arithmetic (interleaved, cold)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (for counter calibration)")
    ap.add_argument("--ab-replaced", action="store_true",
                    help="instead of the headline line: A/B of the fused call against the path it replaces "
                         "(q/k norm + rotation, append to the pool, paged attention over L + b keys), "
                         "interleaved, cold")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calibrate-copy run into profiles/traffic.json")
    return ap.parse_args()


WORKLOADS = {
    1: "cfg1: 1 req x 8 tok, 6/1 heads, L=64 in a 4-page pool, plain path",
    2: "cfg2: 8 req x 8 tok, 6/1 heads, L~U[0,2041], 512-page pool, dense int32 rows, qknorm int32 pos",
    3: "cfg3: 8 req x 8 tok, 24/4 heads, L~U[0,2041], stride-40 rows, qknorm int64 pos",
    5: "drafter block attention qknorm, 8 req x 8 tok, 24/4 heads, L=32768/request, "
       "4096 of 5000 pages, dense int32 rows, int32 pos",
}


def _oracle_rate(case, budget_s: float):
    """K/V bytes per second of the fp64 oracle over whole requests, one at a time (cycling over
    the batch), until the budget is used: (GB/s, request-passes, seconds)."""
    import oracle

    a = case.np_args()
    R = case.R
    done_bytes = 0
    t0 = time.perf_counter()
    n_req = 0
    for it in range(1000 * R):
        r = it % R
        sub = dict(a)
        sub["qkv"] = a["qkv"][r * case.T:(r + 1) * case.T]
        sub["page_table"] = a["page_table"][r:r + 1]
        sub["context_lens"] = a["context_lens"][r:r + 1]
        sub["positions"] = None if a["positions"] is None else a["positions"][r * case.T:(r + 1) * case.T]
        if case.qknorm:
            oracle.drafter_attn_qknorm(**sub)
        else:
            oracle.drafter_attn(**sub)
        n_req += 1
        done_bytes += int(a["context_lens"][r]) * case.Hkv * 64 * 2 * 2
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return done_bytes / dt / 1e9, n_req, dt


def cpu_baseline(case, budget_s: float):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload: once with
    the BLAS pool at its default size (the headline figure, ``cores`` = its threads) and once
    with one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads, threadpool_limits = 1, None
    gbs, n_req, dt = _oracle_rate(case, budget_s)
    out = {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "host_cores": os.cpu_count(),
           "kind": "oracle",
           "sample": f"{n_req} request-passes over the {case.R} requests of the same workload "
                     f"(fp64 numpy oracle, {n_req / case.R:.2f} calls' worth), {dt:.1f} s"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            gbs1, n1, dt1 = _oracle_rate(case, budget_s / 2)
        out["one_thread"] = {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                             "sample": f"{n1} request-passes, {dt1:.1f} s"}
    return out


KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_drafter_amd", "csrc", "drafter_attn.hip")


def kernel_code_hash() -> str:
    """sha256 of what decides a launch's memory traffic -- the device code (the source above its
    host-side section) and the split plan (make_plan) -- with comments removed and whitespace
    collapsed: any change to that code changes it; an edit of a comment or of host-side
    validation does not."""
    import hashlib
    import re
    src = open(KERNEL_SRC).read()
    plan = re.search(r"\nPlan make_plan\(.*?\n}\n", src, flags=re.S)
    text = src.split("// host side", 1)[0] + (plan.group(0) if plan else "")
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic(workload: int):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (scaled by a plain copy's counters), or None when the kernel code has changed
    since those counters were taken or they cover another workload."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        sha = kernel_code_hash()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_code_sha256") != sha or rec.get("workload") != workload:
        return None
    return int(round(rec["traffic_bytes_per_launch"]))


COPY_BYTES = 1 << 29  # the --calibrate-copy buffer


def counter_means(path: str, counter: str):
    """Mean counter value (KiB) per dispatch, by kernel name, from a rocprofv3 counter CSV.
    The copy kernel is kept only for the dispatches of the 512 MiB calibration copy
    (the largest grid of that kernel)."""
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    copy = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
    big = max(int(r["Grid_Size"]) for r in copy) if copy else 0
    out = {}
    for r in rows:
        if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) != big:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in out.items()}


def write_traffic(fetch_csv: str, write_csv: str, workload: int, dest: str = None):
    fetch, write = counter_means(fetch_csv, "FETCH_SIZE"), counter_means(write_csv, "WRITE_SIZE")
    copy = next(k for k in fetch if "copyBuffer" in k)
    kern = next(k for k in fetch if "drafter_attn_kernel<" in k)
    fs = COPY_BYTES / 1024 / fetch[copy][0]
    ws = COPY_BYTES / 1024 / write[copy][0]
    rec = {"kernel_code_sha256": kernel_code_hash(), "workload": workload,
           "kernel": kern, "dispatches": fetch[kern][1],
           "fetch_kib": fetch[kern][0], "write_kib": write[kern][0],
           "copy_fetch_kib": fetch[copy][0], "copy_write_kib": write[copy][0],
           "fetch_scale": fs, "write_scale": ws,
           "traffic_bytes_per_launch": 1024 * (fetch[kern][0] * fs + write[kern][0] * ws)}
    with open(dest or os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return rec


LARGE = [(8, 24, 4, 2048), (8, 24, 4, 16384), (8, 96, 16, 16384),  # R, Hq, Hkv, pages per request
         (1, 24, 4, 512), (1, 24, 4, 2048)]                           # one request: 32k and 131k tokens


def large_contexts(args):
    """Context lengths beyond the headline workload (8 x 8 tokens, qknorm, every request at the
    same length): 131k tokens at 24/4 heads, 1M tokens at 24/4 and at 96/16 heads; and one
    request of 32k and of 131k tokens at 24/4 heads (plans of 64 splits).  The pools (67 MB to
    34 GB) are drawn on the device; one JSON line per size, mean of event-timed calls after
    warm-up, each after the untimed 1 GiB read (cold caches)."""
    import torch

    import drafter_synth as ds
    from speculative_decoding_drafter_amd import drafter_attn_qknorm, make_workspace, plan

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    for R, Hq, Hkv, pages in LARGE:
        pool = ds.device_normal_pool(R * pages, Hkv, seed=5, device="cuda")
        case = ds.make_case(R, 8, Hq, Hkv, [pages * 64] * R, seed=5, stride=pages, pool_pages=R * pages,
                            qknorm=True, pool_override=pool)
        g = ds.to_device(case, "cuda")
        ws = make_workspace(R, 8, Hq, Hkv, pages, "cuda")
        out = torch.empty(R * 8, Hq * 64, dtype=torch.bfloat16, device="cuda")

        def call():
            drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                g.q_norm_weight, g.k_norm_weight, num_q_heads=Hq, num_kv_heads=Hkv,
                                tokens_per_block=8, out=out, workspace=ws)
        for _ in range(args.warmup // 4 + 1):
            call()
        torch.cuda.synchronize()
        evs = []
        for _ in range(max(5, args.steps // 20)):
            torch.sum(flush, dim=0, out=flush_out)  # cold: the one-request pools fit the Infinity Cache
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        kv = R * pages * Hkv * 2 * 64 * 64 * 2
        print(json.dumps({"metric": "K/V-read HBM GB/s at large contexts", "requests": R, "tokens": 8,
                          "q_heads": Hq, "kv_heads": Hkv, "context_tokens": pages * 64, "kv_bytes_per_call": kv,
                          "us_per_call": round(ms * 1e3, 1), "GBs": round(kv / (ms * 1e-3) / 1e9, 1),
                          "pct_of_hbm_peak": round(100 * kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                          "splits": plan(R, Hkv, pages)[0], "cache": "cold (1 GiB read before each call)",
                          "calls_timed": len(evs)}), flush=True)
        del pool, case, g, ws, out
        torch.cuda.empty_cache()


def ab_replaced(args):
    """Fused op vs the path it replaces on the same workload (one fresh pool page per request
    for the appended slots).  Each step is timed alone after the cache flush; the two are
    interleaved in rounds so that both see the same machine state."""
    import numpy as np
    import torch

    import drafter_synth as ds
    from speculative_decoding_drafter_amd import (drafter_attn, drafter_attn_qknorm, kv_append, make_workspace,
                                                  paged_attn, qk_norm_rope)

    dev = torch.device("cuda:0")
    case = ds.with_append_room(ds.make_config(args.config), seed=1000 * args.config + 7)
    g = ds.to_device(case, dev)
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, dev)
    out = torch.empty(case.R * case.T, case.Hq * 64, dtype=torch.bfloat16, device=dev)
    rows = g.qkv.clone()
    b = g.block_lens if g.block_lens is not None else torch.full_like(g.context_lens, case.T)
    kv_lens = g.context_lens + b
    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T, block_lens=g.block_lens)

    def fused():
        if case.qknorm:
            drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                g.q_norm_weight, g.k_norm_weight, scale=case.scale, out=out, workspace=ws, **kw)
        else:
            drafter_attn(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, scale=case.scale, out=out,
                         workspace=ws, **kw)

    def stage_norm():
        if case.qknorm:
            qk_norm_rope(rows, g.positions, g.q_norm_weight, g.k_norm_weight, num_q_heads=case.Hq,
                         num_kv_heads=case.Hkv)

    def stage_append():
        kv_append(rows, g.k_pool, g.v_pool, g.page_table, g.context_lens, **kw)

    def stage_attn():
        paged_attn(rows, g.k_pool, g.v_pool, g.page_table, kv_lens, scale=case.scale, out=out, workspace=ws, **kw)

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    stages = [("append", stage_append), ("paged_attn", stage_attn)]
    if case.qknorm:
        stages.insert(0, ("norm", stage_norm))

    def replaced():
        for _, fn in stages:
            fn()

    # One event pair per timed interval (each pair adds its own overhead): the whole
    # replaced path in one interval, and each of its stages alone in separate steps
    # (the other stages run untimed around it).
    variants = {"fused": [("fused", fused)], "replaced": [("replaced", replaced)],
                "stages": [(name, fn) for name, fn in stages]}
    res = {"fused": [], "replaced": []}
    res.update({name: [] for name, _ in stages})
    rounds = max(1, args.steps // 20)
    for rnd in range(rounds + 1):              # round 0 is warm-up
        order = ("fused", "replaced", "stages") if rnd % 2 else ("stages", "replaced", "fused")
        for which in order:
            for i in range(20):
                if which == "stages":
                    timed = stages[i % len(stages)][0]
                    torch.sum(flush, dim=0, out=flush_out)
                    e0, e1 = ev(), ev()
                    for name, fn in stages:
                        if name == timed:
                            e0.record(); fn(); e1.record()
                        else:
                            fn()
                else:
                    timed, fn = variants[which][0]
                    torch.sum(flush, dim=0, out=flush_out)
                    e0, e1 = ev(), ev()
                    e0.record(); fn(); e1.record()
                torch.cuda.synchronize()
                if rnd:
                    res[timed].append(e0.elapsed_time(e1) * 1e3)
    mean = {k: round(float(np.mean(v)), 3) for k, v in res.items()}
    line = {"metric": "fused drafter attention vs the replaced path (us/call, cold)",
            "fused_us": mean["fused"], "replaced_us": mean["replaced"],
            "replaced_stages_us": {{"norm": "qk_norm_rope"}.get(k, "kv_append" if k == "append" else k): mean[k]
                                   for k, _ in stages},
            "replaced_over_fused": round(mean["replaced"] / mean["fused"], 4),
            "steps_each": len(res["fused"]), "launches": {"fused": 1, "replaced": len(stages)},
            "config": {"workload": WORKLOADS[args.config], "pool_pages": case.num_pages,
                       "page_table_stride": case.stride}}
    print(json.dumps(line), flush=True)


MIXED = [  # (name, R, Hq, Hkv, page-table stride, lengths: list or (seed, max))
    ("mixed lengths U[0, 32k], the 32k workload's stride", 8, 24, 4, 512, (11, 32768)),
    ("mixed lengths U[0, 64k]", 8, 24, 4, 1024, (12, 65536)),
    ("one 64k-token request among short ones", 8, 24, 4, 1024, [65536, 100, 0, 2000, 0, 1, 0, 64]),
    ("lengths U[0, 2041] under a padded stride of 1024 pages", 8, 24, 4, 1024, (13, 2041)),
    ("6/1 heads, mixed lengths U[0, 128k]", 8, 6, 1, 2048, (14, 131072)),
    ("equal 32k contexts (the headline workload's shape)", 8, 24, 4, 512, [32768] * 8),
]


def balanced_plan(R, Hkv, stride, lens):
    """(balanced?, pages per split) of the length-aware schedule for these lengths, as the
    header documents it (reported beside the timings)."""
    import math
    from speculative_decoding_drafter_amd import plan

    S, Ps = plan(R, Hkv, stride)
    npg = [math.ceil(min(max(L, 0), stride * 64) / 64) for L in lens]
    N, nmax = sum(npg), max(npg)
    if S > 1 and Ps >= 32 and N > 0:
        pb = max(math.ceil(N / (R * (S - 1))), math.ceil(nmax / 32))
        pb = max(8, math.ceil(pb / 8) * 8)
        if pb <= (3 * Ps // 4) // 8 * 8:
            return True, pb
    return False, Ps


def mixed_lengths(args):
    """The length-aware schedule against the static plan alone (the same source built with
    DA_STATIC_PLAN_ONLY), on mixed-length workloads: interleaved rounds, cold (1 GiB read
    before every call), one event pair per call; one JSON line per workload."""
    import ctypes

    import numpy as np
    import torch

    import drafter_synth as ds
    from speculative_decoding_drafter_amd import _lib, build

    libs = {}
    for name, path in (("length_aware", _lib.library_path()), ("static_plan", build.LIB_STATIC_PLAN)):
        lib = ctypes.CDLL(path)
        fn = lib.drafter_attn_qknorm
        fn.restype, fn.argtypes = _lib.SIGNATURES["drafter_attn_qknorm"]
        wsf = lib.drafter_attn_workspace_bytes
        wsf.restype, wsf.argtypes = _lib.SIGNATURES["drafter_attn_workspace_bytes"]
        libs[name] = (fn, wsf)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    for wname, R, Hq, Hkv, stride, lens in MIXED:
        if isinstance(lens, tuple):
            rng = np.random.default_rng(lens[0])
            lens = [int(x) for x in rng.integers(0, lens[1] + 1, R)]
        pages = sum(-(-L // 64) for L in lens) + 8
        pool = ds.device_normal_pool(pages, Hkv, seed=17, device="cuda")
        case = ds.make_case(R, 8, Hq, Hkv, lens, seed=17, stride=stride, pool_pages=pages, qknorm=True,
                            pool_override=pool)
        g = ds.to_device(case, "cuda")
        out = torch.empty(R * 8, Hq * 64, dtype=torch.bfloat16, device="cuda")
        ws = {k: torch.zeros(int(wsf(R, 8, Hq, Hkv, 64, stride)), dtype=torch.uint8, device="cuda")
              for k, (_, wsf) in libs.items()}

        def call(k):
            fn = libs[k][0]
            rc = fn(g.qkv.data_ptr(), g.qkv.stride(0), g.k_pool.data_ptr(), g.v_pool.data_ptr(), g.k_pool.stride(0),
                    g.k_pool.shape[0], g.page_table.data_ptr(), stride, g.context_lens.data_ptr(), None, R, 8, Hq,
                    Hkv, 64, 64, case.scale, g.positions.data_ptr(), 0, g.q_norm_weight.data_ptr(),
                    g.k_norm_weight.data_ptr(), 1e-5, 10000.0, ws[k].data_ptr(), ws[k].numel(), out.data_ptr(),
                    out.stride(0), None, torch.cuda.current_stream().cuda_stream)
            assert rc == 0, rc

        res = {k: [] for k in libs}
        rounds = max(2, args.steps // 25)
        for rnd in range(rounds + 1):             # round 0 is warm-up
            for k in (list(libs) if rnd % 2 else list(libs)[::-1]):
                evs = []
                for _ in range(25):
                    torch.sum(flush, dim=0, out=flush_out)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(); call(k); e1.record()
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                if rnd:
                    res[k] += [a.elapsed_time(b) * 1e3 for a, b in evs]
        kv = case.kv_bytes()
        us = {k: float(np.mean(v)) for k, v in res.items()}
        bal, ps = balanced_plan(R, Hkv, stride, lens)
        from speculative_decoding_drafter_amd import plan
        S, Ps = plan(R, Hkv, stride)
        print(json.dumps({"metric": "length-aware schedule vs static plan (us/call, cold)", "workload": wname,
                          "requests": R, "q_heads": Hq, "kv_heads": Hkv, "page_table_stride": stride,
                          "context_lens": lens, "kv_bytes_per_call": kv, "static_plan": {"splits": S, "pages": Ps},
                          "length_aware_plan": {"balanced": bal, "pages_per_split": ps},
                          "us_length_aware": round(us["length_aware"], 2), "us_static_plan": round(us["static_plan"], 2),
                          "speedup": round(us["static_plan"] / us["length_aware"], 3),
                          "GBs_length_aware": round(kv / (us["length_aware"] * 1e-6) / 1e9, 1),
                          "calls_each": len(res["length_aware"])}), flush=True)
        del pool, case, g, ws, out
        torch.cuda.empty_cache()


PROBE_MODES = {0: "LDS DMA, non-temporal (the attention's load path)", 1: "LDS DMA, default cache policy",
               2: "register loads, non-temporal, two pages in flight per wave",
               3: "contiguous read of the same byte count from the pool (no page table)"}


def ceiling(args):
    """The attention's time against the cost of its own access pattern: the page-stream
    probe (libpage_stream_probe.so) reads the same K/V tiles of the same workload with the
    attention's grid, LDS footprint and page-to-wave mapping and does no arithmetic
    (modes above).  Interleaved rounds, cold (1 GiB read before every call), one event
    pair per call; one JSON line."""
    import ctypes

    import numpy as np
    import torch

    import drafter_synth as ds
    from speculative_decoding_drafter_amd import build, drafter_attn, drafter_attn_qknorm, make_workspace, plan

    lib = ctypes.CDLL(build.LIB_PROBE)
    probe = lib.page_stream_probe
    probe.restype = ctypes.c_int
    probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    case = ds.make_config(args.config)
    g = ds.to_device(case, dev)
    assert case.stride > 0 and g.k_pool.stride(0) == g.v_pool.stride(0) and g.k_pool.stride(1) == 64 * 64
    S, Ps = plan(case.R, case.Hkv, case.stride)
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, dev)
    out = torch.empty(case.R * case.T, case.Hq * 64, dtype=torch.bfloat16, device=dev)
    words = torch.zeros(case.R * case.Hkv * S * 8, dtype=torch.int32, device=dev)
    kv = case.kv_bytes()
    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T, scale=case.scale, out=out,
              workspace=ws)

    def attention():
        if case.qknorm:
            drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                g.q_norm_weight, g.k_norm_weight, **kw)
        else:
            drafter_attn(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, **kw)

    def run_probe(mode):
        rc = probe(mode, g.k_pool.data_ptr(), g.v_pool.data_ptr(), g.k_pool.shape[0], 2 * g.k_pool.stride(0),
                   case.Hkv, g.page_table.data_ptr(), case.stride, g.context_lens.data_ptr(), case.R, S, Ps, kv,
                   words.data_ptr(), words.numel(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc

    variants = {"attention": attention}
    variants.update({f"probe{m}": (lambda m=m: run_probe(m)) for m in PROBE_MODES})
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)
    res = {k: [] for k in variants}
    rounds = max(2, args.steps // 25)
    for rnd in range(rounds + 1):                 # round 0 is warm-up
        for k in (list(variants) if rnd % 2 else list(variants)[::-1]):
            evs = []
            for _ in range(25):
                torch.sum(flush, dim=0, out=flush_out)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(); variants[k](); e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
            if rnd:
                res[k] += [a.elapsed_time(b) * 1e3 for a, b in evs]
    mean = {k: float(np.mean(v)) for k, v in res.items()}
    med = {k: float(np.median(v)) for k, v in res.items()}
    line = {"metric": "attention vs the cost of its access pattern (us/call, cold, event pair per call)",
            "workload": WORKLOADS[args.config], "kv_bytes_per_call": kv, "splits": S, "pages_per_split": Ps,
            "attention_us": round(mean["attention"], 2), "attention_median_us": round(med["attention"], 2),
            "probe_us": {PROBE_MODES[m]: round(mean[f"probe{m}"], 2) for m in PROBE_MODES},
            "probe_median_us": {PROBE_MODES[m]: round(med[f"probe{m}"], 2) for m in PROBE_MODES},
            "probe_GBs": {PROBE_MODES[m]: round(kv / (mean[f"probe{m}"] * 1e-6) / 1e9, 1) for m in PROBE_MODES},
            "attention_over_own_pattern": round(mean["attention"] / mean["probe0"], 4),
            "calls_each": len(res["attention"])}
    print(json.dumps(line), flush=True)


def phases(args):
    """Where a cold call's time goes: the phase timestamps of the measurement build
    (DA_PHASE_TRACE; per workgroup, see the kernel source), for the four configurations and
    two mixed-length workloads.  For each workload, five calls each after the 1 GiB read;
    every figure is the median over those calls of a per-call statistic, in us from the
    first wave's start (100 MHz counter)."""
    import ctypes

    import numpy as np
    import torch

    import drafter_synth as ds
    from speculative_decoding_drafter_amd import _lib, build, plan

    lib = ctypes.CDLL(build.LIB_PHASES)
    fns = {}
    for k in ("drafter_attn", "drafter_attn_qknorm"):
        fn = getattr(lib, k)
        fn.restype, fn.argtypes = _lib.SIGNATURES[k]
        fns[k] = fn
    wsf = lib.drafter_attn_workspace_bytes
    wsf.restype, wsf.argtypes = _lib.SIGNATURES["drafter_attn_workspace_bytes"]
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    work = [(WORKLOADS[n], ds.make_config(n)) for n in (1, 2, 3, 5)]
    for wname, R, Hq, Hkv, stride, lens in MIXED[1:3]:
        if isinstance(lens, tuple):
            lens = [int(x) for x in np.random.default_rng(lens[0]).integers(0, lens[1] + 1, R)]
        pages = sum(-(-L // 64) for L in lens) + 8
        work.append((wname, ds.make_case(R, 8, Hq, Hkv, lens, seed=17, stride=stride, pool_pages=pages, qknorm=True,
                                          pool_override=ds.device_normal_pool(pages, Hkv, seed=17, device="cuda"))))
    for wname, case in work:
        g = ds.to_device(case, "cuda")
        S, Ps = plan(case.R, case.Hkv, case.stride)
        ngroups = S * case.Hkv * case.R
        trace = torch.zeros(ngroups * 64, dtype=torch.int64, device="cuda")
        ws = torch.zeros(int(wsf(case.R, case.T, case.Hq, case.Hkv, 64, case.stride)), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty(case.R * case.T, case.Hq * 64, dtype=torch.bfloat16, device="cuda")

        def call():
            head = (g.qkv.data_ptr(), g.qkv.stride(0), g.k_pool.data_ptr(), g.v_pool.data_ptr(), g.k_pool.stride(0),
                    g.k_pool.shape[0], g.page_table.data_ptr() if case.stride else None, case.stride,
                    g.context_lens.data_ptr(), None, case.R, case.T, case.Hq, case.Hkv, 64, 64, case.scale)
            tail = (ws.data_ptr(), ws.numel(), out.data_ptr(), out.stride(0), trace.data_ptr(),
                    torch.cuda.current_stream().cuda_stream)
            if case.qknorm:
                mid = (g.positions.data_ptr(), 0 if g.positions.dtype == torch.int32 else 1,
                       g.q_norm_weight.data_ptr(), g.k_norm_weight.data_ptr(), case.eps, case.rope_base)
                assert fns["drafter_attn_qknorm"](*head, *mid, *tail) == 0
            else:
                assert fns["drafter_attn"](*head, *tail) == 0

        stats = []
        for it in range(8):
            trace.zero_()
            torch.sum(flush, dim=0, out=flush_out)
            call()
            torch.cuda.synchronize()
            if it < 3:  # warm-up calls
                continue
            d = trace.view(ngroups, 64).cpu().numpy().astype(np.int64)
            st = d[:, 0:8]
            t0 = st[st > 0].min()
            us = lambda x: (np.asarray(x, dtype=np.float64) - t0) / 100.0
            pos = lambda a: a[a > 0]
            ends = d[:, 46]
            last = int(np.argmax(ends))
            early = pos(d[:, 48:56])  # waves that issue their first page before the prologue
            row = {"prologue_loads_landed": np.median(us(pos(d[:, 8:16]))),
                   "first_dma_issued_early_waves": np.median(us(early)) if early.size else float("nan"),
                   "prologue_done_first_dma_issued_all_waves": np.median(us(pos(d[:, 16:24]))),
                   "prologue_barrier": np.median(us(pos(d[:, 47]))),
                   "first_k_tile_landed": np.median(us(pos(d[:, 24:32]))),
                   "loop_end_median": np.median(us(pos(d[:, 32:40]))),
                   "loop_end_last": us(pos(d[:, 32:40])).max(),
                   "end": us(ends[last])}
            for k, name in ((41, "last_group_merge_barrier"), (42, "last_group_merged"),
                            (43, "last_group_published"), (44, "last_group_counter"),
                            (45, "last_group_combine_loads_landed")):
                row[name] = us(d[last, k]) if d[last, k] > 0 else float("nan")
            stats.append(row)
        med = {k: round(float(np.median([r[k] for r in stats])), 2) for k in stats[0]}
        print(json.dumps({"metric": "phase timestamps of a cold call (us from the first wave's start, median of 5 "
                                    "calls)", "workload": wname, "splits": S, "pages_per_split": Ps,
                          "context_lens": case.context_lens.tolist(), "phases_us": med}), flush=True)


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.config)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this hot path is not sharded across GPUs "
              "(see the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.ab_replaced:
        ab_replaced(args)
        return
    if args.large:
        large_contexts(args)
        return
    if args.mixed:
        mixed_lengths(args)
        return
    if args.phases:
        phases(args)
        return
    if args.ceiling:
        ceiling(args)
        return
    import torch

    import drafter_synth as ds
    from speculative_decoding_drafter_amd import drafter_attn, drafter_attn_qknorm, make_workspace, plan

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    case = ds.make_config(args.config)
    g = ds.to_device(case, dev)
    ws = make_workspace(case.R, case.T, case.Hq, case.Hkv, case.stride, dev)
    out = torch.empty(case.R * case.T, case.Hq * 64, dtype=torch.bfloat16, device=dev)
    kw = dict(num_q_heads=case.Hq, num_kv_heads=case.Hkv, tokens_per_block=case.T, scale=case.scale,
              out=out, workspace=ws)
    yarn = dict(factor=4.0, original_max_position=4096, alpha=1.0, beta=32.0) if args.yarn else None
    assert yarn is None or case.qknorm, "--yarn needs a qknorm workload"
    if case.qknorm:
        call = lambda: drafter_attn_qknorm(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, g.positions,
                                           g.q_norm_weight, g.k_norm_weight, eps=case.eps,
                                           rope_base=case.rope_base, yarn=yarn, **kw)
    else:
        call = lambda: drafter_attn(g.qkv, g.k_pool, g.v_pool, g.page_table, g.context_lens, **kw)

    flush = None if args.hot else torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    # one call captured in a HIP graph (after an eager warm-up); replaying it is the other launch mode
    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    headline, other = (graph.replay, call) if args.graph else (call, graph.replay)

    def timed(step):
        """Warm-up, then each of args.steps calls alone between HIP events (after the flush):
        (sorted times in ms, wall seconds of the timed region)."""
        def one(timed_events=None):
            if flush is not None:
                torch.sum(flush, dim=0, out=flush_out)
            if timed_events is None:
                step()
            else:
                timed_events[0].record()
                step()
                timed_events[1].record()

        for _ in range(args.warmup):
            one()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for e in evs:
            one(e)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs), time.perf_counter() - t0

    pct = lambda ts: [round(ts[int(q * (len(ts) - 1))] * 1e3, 3) for q in (0.1, 0.5, 0.9)]
    times_ms, wall = timed(headline)
    mean_ms = sum(times_ms) / len(times_ms)
    p10, p50, p90 = (times_ms[int(q * (len(times_ms) - 1))] for q in (0.1, 0.5, 0.9))
    # the other launch mode on the same buffers, timed the same way (reported beside the headline)
    other_ms, _ = timed(other)
    other_mean = sum(other_ms) / len(other_ms)

    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    kv_bytes = case.kv_bytes()
    gbs = kv_bytes / (mean_ms * 1e-3) / 1e9
    S, Ps = plan(case.R, case.Hkv, case.stride)
    # every byte a call moves: K/V pages, the qkv rows it reads, the output, and the
    # split partials (written once, read back once by the combine)
    rows = case.R * case.T
    other_bytes = rows * (case.Hq + 2 * case.Hkv) * 64 * 2 + rows * case.Hq * 64 * 2
    if S > 1:
        other_bytes += 2 * case.R * case.Hkv * S * 48 * 66 * 4
    line = {
        "metric": "K/V-read HBM GB/s (% of MI355X peak) and us/call, 8 req x 8 tok, 24/4 heads",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 6),
        "us_per_call": round(mean_ms * 1e3, 3),
        "us_p10_p50_p90": [round(p10 * 1e3, 3), round(p50 * 1e3, 3), round(p90 * 1e3, 3)],
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "kv_GBs_at_median": round(kv_bytes / (p50 * 1e-3) / 1e9, 2),
        "all_bytes_GBs": round((kv_bytes + other_bytes) / (mean_ms * 1e-3) / 1e9, 2),
        "rope": "yarn factor 4, original context 4096, ramp 1..32" if yarn else "neox",
        "launch": ("HIP graph replay (DEBUG_CLR_GRAPH_PACKET_CAPTURE=%s)"
                   % os.environ.get("DEBUG_CLR_GRAPH_PACKET_CAPTURE", "unset")) if args.graph else "direct",
        ("direct_us_per_call" if args.graph else "graph_us_per_call"): round(other_mean * 1e3, 3),
        ("direct_us_p10_p50_p90" if args.graph else "graph_us_p10_p50_p90"): pct(other_ms),
        "graph_packet_capture_env": os.environ.get("DEBUG_CLR_GRAPH_PACKET_CAPTURE", "unset"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "cache": "hot (no flush)" if args.hot else "cold (1 GiB read before each call)",
        "wall_s_timed_region": round(wall, 4),
        "config": {"workload": WORKLOADS[args.config], "requests": case.R, "tokens": case.T,
                   "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": 64, "page": 64,
                   "context_lens_sum": int(case.context_lens.sum()), "pool_pages": case.num_pages,
                   "page_table_stride": case.stride, "splits": S, "pages_per_split": Ps,
                   "qknorm": case.qknorm, "kv_bytes_per_call": kv_bytes, "other_bytes_per_call": other_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if args.hot else measured_traffic(args.config),
                     "kernel": "drafter_attn_kernel<%d,%s,%s,true,%s,%s>" % (
                         (6 * case.T + 15) // 16, str(case.qknorm).lower(),
                         str(case.qknorm and case.positions.dtype == torch.int64).lower(),
                         str(S > 1 and Ps >= 32).lower(), str(S > 16).lower())},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

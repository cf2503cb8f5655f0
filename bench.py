"""Benchmark: paged GQA attention on one MI355X.

Headline workload: one Qwen3-8B layer decode step -- 8 sequences, 32 query /
8 KV heads, head_dim 128, bf16, 256-token blocks, cached context uniform in
[512, 2048]; a step appends one token per sequence (kv_append) and decodes
(paged_gqa_decode).  ``value`` is the decode KV-read rate: the unique K/V bytes
a step must read, divided by the wall time per step.  The step is captured in
a HIP graph and replayed, as a serving loop replays its decode step; the
step is one paged_gqa_decode_append launch (the append fused into the
decode), and the two-call step (kv_append, then paged_gqa_decode; graph and
eager) is reported beside it.  Pool copies are rotated
(>= 1 GiB in total) so that every step reads from HBM, not from the 256 MB
last-level cache.

The metric also names prefill: the Qwen3-8B causal prefill workload (4 prompts
of 1024..4096 tokens) is timed in the same run and reported as causal TFLOP/s
(4 * D * Hq flops per unmasked query/key pair) under ``prefill``.  Decode at a
bandwidth-bound scale (3.24 GB of unique K/V, shared prefixes and 32K-token
sequences) is reported under ``long_context_decode``, the mixed
continuous-batching step (64 decodes + two 512-row chunks, graphs of 8 steps)
under ``mixed_step``, and the INT8 KV cache (quantising append, decode over codes
and per-row scales) on the headline step and the long-context decode under
``int8_kv_cache``, and the fused QKV projection with its paged append
(prefill prompts and decode step shapes) under ``qkv_project_append``.

Kernel durations are measured with HIP events on the stream the kernels run
on; ``roofline`` relates the decode call to HBM peak, ``prefill.roofline`` the
prefill kernel to dense bf16 MFMA peak.  ``cpu_baseline`` times the fp64 CPU
oracle on the same decode step (all host cores and one thread) and on the
prefill workload, a reference point only.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context decode measurement")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed continuous-batching step")
    ap.add_argument("--no-append", action="store_true", help="skip the kv_append measurement")
    ap.add_argument("--no-int8", action="store_true", help="skip the INT8 KV cache measurements")
    ap.add_argument("--no-qkv", action="store_true", help="skip the fused QKV projection measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-pass", action="store_true",
                    help="for counter runs: a few untimed steps of each kernel plus a reference device copy, no JSON")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the reference copy in --profile-pass")
    ap.add_argument("--profile-warm-s", type=float, default=0.0,
                    help="--profile-pass: run each workload this long before its counted calls (steady clocks)")
    ap.add_argument("--profile-only", choices=("decode", "prefill", "long", "int8", "int8step", "qkv", "qkvdec",
                                               "copy"),
                    default=None,
                    help="--profile-pass: run only this workload (counter passes per workload)")
    return ap.parse_args()


def profile_pass(args):
    """A short program for rocprofv3 counter passes: the decode step (one
    decode_append launch), the prefill kernel and the long-context decode a
    few times each (the long one last, unless --no-long), and one plain
    device-to-device copy of --copy-mib MiB whose counter readings calibrate
    the byte counters.  --profile-only also offers the INT8 long-context
    decode (int8), the INT8 decode step (int8step, graphed as timed) and the
    fused QKV projection at the prefill-prompt (qkv) and decode-step (qkvdec)
    shapes."""
    import torch
    import paged_kv_gqa_scatter_amd as pkv
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import DeviceCase, Int8DeviceCase

    n = max(1, args.steps)
    only = args.profile_only
    done = []

    def warm(fn):
        t = time.perf_counter()
        while time.perf_counter() - t < args.profile_warm_s:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()

    if only in (None, "decode"):
        case = W.config2_decode()
        n_rot = max(1, -(-ROTATE_BYTES // case.pool_bytes))  # as timed: every step reads HBM
        dc = DeviceCase(case, pools=n_rot)
        dc.run_fills()
        st = dc.steps[0]
        # as timed: every pool copy's step in one HIP graph, replayed
        g = dc.capture(lambda: [dc.decode_append(st["append"], st["decode"], pool=r) for r in range(n_rot)])
        warm(g.replay)
        for _ in range(-(-n // n_rot)):
            g.replay()
        torch.cuda.synchronize()
        del g, dc
        done.append(f"{-(-n // n_rot) * n_rot} decode steps")
    if only in (None, "prefill"):
        pc = DeviceCase(W.config3_prefill())
        pc.run_fills()
        pc.append(pc.steps[0]["append"])
        warm(lambda: pc.prefill(pc.steps[0]["prefill"]))
        for _ in range(n):
            pc.prefill(pc.steps[0]["prefill"])
        torch.cuda.synchronize()
        del pc
        done.append(f"{n} prefills")
    if only == "long" or (only is None and not args.no_long):
        lc = DeviceCase(W.config5_prefix_long(draw_values=False))
        lc.run_fills()
        lc.append(lc.steps[0]["append"])
        warm(lambda: lc.decode(lc.steps[0]["decode"]))
        for _ in range(n):
            lc.decode(lc.steps[0]["decode"])
        torch.cuda.synchronize()
        del lc
        done.append(f"{n} long-context decodes")
    if only == "int8step":
        case = W.config2_decode()
        pool_bytes = case.pool_bytes * (case.head_dim + 4) // (2 * case.head_dim)
        n_rot = max(1, -(-ROTATE_BYTES // pool_bytes))  # as timed: every step reads HBM
        ic = Int8DeviceCase(case, pools=n_rot)
        ic.run_fills()
        st = ic.steps[0]
        g = ic.capture(lambda: [ic.decode_append(st["append"], st["decode"], pool=r) for r in range(n_rot)])
        warm(g.replay)
        for _ in range(-(-n // n_rot)):
            g.replay()
        torch.cuda.synchronize()
        del g, ic
        done.append(f"{-(-n // n_rot) * n_rot} INT8 decode steps")
    if only == "int8":
        ic = Int8DeviceCase(W.config5_prefix_long(draw_values=False))
        ic.run_fills()
        ic.append(ic.steps[0]["append"])
        warm(lambda: ic.decode(ic.steps[0]["decode"]))
        for _ in range(n):
            ic.decode(ic.steps[0]["decode"])
        torch.cuda.synchronize()
        del ic
        done.append(f"{n} INT8 long-context decodes")
    if only in ("qkv", "qkvdec"):
        case = W.config3_prefill(draw_values=False) if only == "qkv" else W.config2_decode(draw_values=False)
        a = case.steps[0].append
        T, dm, hq, hkv, d = int(a.cu_new_lens[-1]), 4096, 32, 8, 128
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0x9C7)
        w = (torch.randn(((hq + 2 * hkv) * d, dm), generator=gen, device="cuda") / 64).to(torch.bfloat16)
        x = torch.randn((T, dm), generator=gen, device="cuda").to(torch.bfloat16)
        kp = torch.zeros((case.num_blocks, hkv, case.block_size, d), dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        q = torch.empty((T, hq, d), dtype=torch.bfloat16, device="cuda")
        cu, ctx, tab = (torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in (a.cu_new_lens, a.ctx_lens,
                                                                                    a.block_table))
        call = lambda: pkv.qkv_project_append(x, w, kp, vp, cu, ctx, tab, hq, q_out=q)
        warm(call)
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        done.append(f"{n} QKV projections of {T} tokens")
    torch.cuda.empty_cache()
    if only in (None, "copy"):
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        done.append(f"a copy of {args.copy_mib} MiB")
    print("profile pass done: " + ", ".join(done), flush=True)


def library_source_hash() -> str:
    """sha256 over the HIP library's sources: a counter record is valid only
    for the kernels it was taken on."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "paged_kv_gqa_scatter_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def traffic_record(op: str):
    """HBM bytes per launch of `op` from the committed rocprofv3 --pmc
    summaries (lines `traffic-record: {json}` in profiles/*.md), or None when
    no record matches the current sources."""
    import glob
    want = library_source_hash()
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(f, encoding="utf-8"):
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("op") == op and rec.get("source_sha256") == want:
                    rec["file"] = os.path.relpath(f, ROOT)
                    return rec
    return None


def attach_traffic(roofline: dict, op: str) -> None:
    """roofline["traffic"]: HBM bytes per launch from the committed counter
    record for `op`, with where it came from; null (and why) when no record
    matches the current kernel sources -- the counters are not taken in
    this run."""
    rec = traffic_record(op)
    if rec is None:
        roofline["traffic"] = None
        roofline["traffic_source"] = "none: no counter record in profiles/ matches the current kernel sources"
    else:
        roofline["traffic"] = int(rec["hbm_bytes_per_launch"])
        roofline["traffic_source"] = (f"{rec['file']}: rocprofv3 --pmc FETCH_SIZE + WRITE_SIZE of an earlier run of "
                                      f"the same sources (SHA-256 matched), copy-calibrated; not measured in this run")


def _timed_replays(graphs, n, warmup):
    """Mean ms per replay of `n` graph replays (cycling over `graphs`),
    bracketed by events on the current stream after `warmup` replays."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(n):
        graphs[i % len(graphs)].replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


def _timed_steps(capture, call, n_rot, k, warmup):
    """Mean ms per step over exactly `k` steps, where step i is `call(i %
    n_rot)` (pool copy i % n_rot): one HIP graph holds the steps of all n_rot
    copies in order -- as a serving engine's per-token graph holds one
    attention step per layer, each over that layer's cache -- and is replayed
    k // n_rot times, then a graph of the k % n_rot steps left runs once;
    events on the current stream bracket the replays, after about `warmup`
    steps of the same graph."""
    import torch
    full = capture(lambda: [call(r) for r in range(n_rot)])
    part = capture(lambda: [call(r) for r in range(k % n_rot)]) if k % n_rot else None
    stream = torch.cuda.current_stream()
    for _ in range(max(1, warmup // n_rot)):
        full.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(k // n_rot):
        full.replay()
    if part is not None:
        part.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    del full, part
    return t0.elapsed_time(t1) / k


def time_decode_workload(args):
    """The headline step: kv_append of one row per sequence, then the decode,
    in one decode_append launch, timed over exactly args.steps steps rotating
    over the pool copies, all copies' steps in one HIP graph (_timed_steps).
    Returns the step time, the two-call step's and the decode call's (same
    graphs), the eagerly launched two-call step's, and the step's with one
    graph per step (each replay then pays a graph launch) for context."""
    import torch
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import DeviceCase

    case = W.config2_decode()
    dec = case.steps[0].decode
    kv_bytes = W.decode_unique_kv_bytes(case, dec)
    n_rot = max(1, -(-ROTATE_BYTES // case.pool_bytes))
    dc = DeviceCase(case, pools=n_rot)
    dc.run_fills()
    step = dc.steps[0]
    stream = torch.cuda.current_stream()

    def eager(i):
        r = i % n_rot
        dc.append(step["append"], pool=r)
        dc.decode(step["decode"], pool=r)

    for i in range(min(args.warmup, 200)):
        eager(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        eager(i)
    t1.record(stream)
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / args.steps

    # the step as one decode_append launch (append + decode fused), as
    # kv_append then paged_gqa_decode, and the decode call alone
    step_ms = _timed_steps(dc.capture, lambda r: dc.decode_append(step["append"], step["decode"], pool=r), n_rot,
                           args.steps, args.warmup)
    split_ms = _timed_steps(dc.capture, lambda r: dc.run_step(0, r), n_rot, args.steps, max(args.warmup // 2, 10))
    dec_ms = _timed_steps(dc.capture, lambda r: dc.decode(step["decode"], pool=r), n_rot, args.steps,
                          max(args.warmup // 2, 10))
    one = [dc.capture(lambda r=r: dc.decode_append(step["append"], step["decode"], pool=r)) for r in range(n_rot)]
    one_ms = _timed_replays(one, args.steps, max(args.warmup // 2, 10))
    del one
    return case, dec, kv_bytes, n_rot, step_ms, dec_ms, eager_ms, split_ms, one_ms


def time_kv_append(args):
    """kv_append alone: config 3's prompt rows (8130 tokens x 8 KV heads x
    128 dims, K and V) into 256-token blocks, bf16 and through the INT8 cache
    (quantising append), each over exactly args.steps calls rotating over
    pool copies and copies of the new rows (>= 1 GiB together) so that every
    call reads and writes HBM.  Bytes are the rows read plus the rows written:
    bf16 2 x T x Hkv x D x 2 x 2; INT8 T x Hkv x (2 D x 2 read + 2 (D + 4)
    written)."""
    import torch
    import paged_kv_gqa_scatter_amd as pkv
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import capture_graph

    case = W.config3_prefill(draw_values=False)
    a = case.steps[0].append
    T = int(a.cu_new_lens[-1])
    NB, Hkv, B, D = case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim
    dev = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    cu, ctx, tab = dev(a.cu_new_lens), dev(a.ctx_lens), dev(a.block_table)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0xA99)
    res = {"workload": f"qwen3-8b prefill prompts' rows appended: {T} tokens x {Hkv} KV heads x {D}, block {B}"}
    for name in ("bf16", "int8"):
        rows_bytes = T * Hkv * D * 2 * 2
        pool_bytes = case.pool_bytes if name == "bf16" else case.pool_bytes * (D + 4) // (2 * D)
        n_rot = max(1, -(-ROTATE_BYTES // (pool_bytes + rows_bytes)))
        rows = [(torch.randn((T, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16),
                 torch.randn((T, Hkv, D), generator=gen, device="cuda").to(torch.bfloat16)) for _ in range(n_rot)]
        if name == "bf16":
            caches = [(torch.empty((NB, Hkv, B, D), dtype=torch.bfloat16, device="cuda"),
                       torch.empty((NB, Hkv, B, D), dtype=torch.bfloat16, device="cuda")) for _ in range(n_rot)]
            call = lambda r: pkv.kv_append(*caches[r], *rows[r], cu, ctx, tab)
            nbytes = 2 * rows_bytes
        else:
            caches = [pkv.empty_int8_cache(NB, Hkv, B, D) for _ in range(n_rot)]
            call = lambda r: pkv.kv_append_int8(*caches[r], *rows[r], cu, ctx, tab)
            nbytes = rows_bytes + T * Hkv * 2 * (D + 4)
        ms = _timed_steps(capture_graph, call, n_rot, args.steps, max(args.warmup // 4, 10))
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 5), "bytes": int(nbytes), "copies_rotated": n_rot,
                     "roofline": {"bound": "hbm", "kernel": "kv_append" if name == "bf16" else "kv_append_int8",
                                  "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs / HBM_PEAK_GBS, 4)}}
        del rows, caches
        torch.cuda.empty_cache()
    return res


MIXED_STEPS_PER_GRAPH = 8


def time_mixed_step(args):
    """The mixed continuous-batching step (64 + 1024 new rows appended, a
    64-sequence decode, two 512-row chunks on 1024 cached tokens), captured
    in a HIP graph and replayed: the decode sequences' rows are appended by
    the decode launch itself, and the prefill rows' append and the prefill
    run beside it on a second stream (DeviceCase.run_step).  As for the
    headline step, a graph holds several steps (a decode iteration's graph
    holds every layer's step), MIXED_STEPS_PER_GRAPH of them here, so that
    the time per step is not one graph launch's overhead; the steps repeat
    the same work (their appends rewrite the same rows), and the decode's
    666 MB of K/V is read from HBM each time.  The time with one step per
    graph is reported beside it."""
    import torch
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import DeviceCase

    case = W.config4_mixed()
    st = case.steps[0]
    kv_bytes = W.decode_unique_kv_bytes(case, st.decode)
    flops = W.prefill_causal_flops(case, st.prefill)
    dc = DeviceCase(case)
    dc.run_fills()
    k = MIXED_STEPS_PER_GRAPH
    n = max(20, args.steps // 4)
    g1 = dc.capture_step(0)
    ms_one = _timed_replays([g1], n, 20)
    del g1
    g = dc.capture(lambda: [dc.run_step(0) for _ in range(k)])
    ms = _timed_replays([g], max(5, n // k), 3) / k
    del g
    # each branch on its own: the decode (decode_append of its 64 rows), and
    # the prefill (its 1024 rows appended once beforehand)
    dec, pre = dc._mixed_parts(0)
    step = dc.steps[0]
    gd = dc.capture(lambda: [dc.decode_append(dec, step["decode"]) for _ in range(k)])
    dms = _timed_replays([gd], max(5, n // k), 3) / k
    del gd
    dc.append(pre)
    gp = dc.capture(lambda: [dc.prefill(step["prefill"]) for _ in range(k)])
    pms = _timed_replays([gp], max(5, n // k), 3) / k
    del gp, dc
    torch.cuda.empty_cache()
    gbs = kv_bytes / (dms * 1e-3) / 1e9
    tfs = flops / (pms * 1e-3) / 1e12
    return {"workload": "qwen3-8b mixed step: 64 decode seqs (ctx log-uniform [128, 8192]) + 2 x 512-row chunks on "
                        "1024 cached; 32q/8kv, d128, block 256; HIP graphs of %d steps, decode_append and "
                        "kv_append + prefill as parallel branches" % k,
            "ms": round(ms, 5), "ms_one_graph_per_step": round(ms_one, 5), "steps_per_graph": k,
            "decode_unique_kv_bytes": int(kv_bytes), "prefill_causal_flops": int(flops),
            "decode_alone": {"ms": round(dms, 5), "what": "the decode branch alone (decode_append of the 64 "
                                                          "sequences' rows), %d per graph" % k,
                             "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode_append (decode_kernel)",
                                          "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": round(gbs / HBM_PEAK_GBS, 4)}},
            "prefill_alone": {"ms": round(pms, 5), "what": "the prefill branch's attention alone (two 512-row "
                                                           "chunks on 1024 cached keys), %d per graph" % k,
                              "roofline": {"bound": "mfma",
                                           "kernel": "paged_gqa_prefill (prefill_split_kernel: the launch "
                                                     "has fewer than two workgroups per CU)",
                                           "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                                           "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}},
            "overlap": round((dms + pms) / ms, 3)}


def time_prefill_workload(args):
    import torch
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import DeviceCase

    case = W.config3_prefill()
    pf = case.steps[0].prefill
    flops = W.prefill_causal_flops(case, pf)
    dc = DeviceCase(case)
    dc.run_fills()
    step = dc.steps[0]
    dc.append(step["append"])
    stream = torch.cuda.current_stream()
    t = time.perf_counter()
    while time.perf_counter() - t < 0.5:  # steady clocks
        for _ in range(10):
            dc.prefill(step["prefill"])
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.prefill_steps)]
    for a, b in evs:
        a.record(stream)
        dc.prefill(step["prefill"])
        b.record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    return case, flops, float(np.mean(times)), float(np.median(times)), float(np.min(times))


def device_context():
    """The device and practical ceilings: a 1 GiB device-to-device copy
    (read + write bytes over its median time, 10 timed copies), a 2 GiB plain
    read (pkv_read_probe, median of 10), a plain bf16 MFMA stream
    (pkv_mfma_probe, median of 10), and the engine clock the driver reports
    as current when there is one GPU to read it from."""
    import glob
    import torch
    n = 1 << 29  # int16 elements: 1 GiB
    src = torch.empty(n, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in evs:
        a.record(s)
        dst.copy_(src)
        b.record(s)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2]
    del src, dst
    # plain reads: 2 GiB streamed once per call by the library's read probe
    # (16-byte non-temporal loads, as the decode kernels stream K/V)
    import paged_kv_gqa_scatter_amd as pkv
    data = torch.zeros(1 << 30, dtype=torch.int16, device="cuda")
    sink = torch.empty(16 * pkv.READ_PROBE_WORKGROUPS, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        pkv.read_probe(data, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in evs:
        a.record(s)
        pkv.read_probe(data, sink)
        b.record(s)
    torch.cuda.synchronize()
    rms = sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2]
    read_bytes = data.numel() * data.element_size()
    del data, sink
    # the bf16 matrix cores' rate on a plain MFMA stream (pkv_mfma_probe:
    # the instruction of the prefill and the fused QKV projection)
    iters = 4096
    sink = torch.empty(4 * 256 * pkv.MFMA_PROBE_WORKGROUPS, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        pkv.mfma_probe(iters, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in evs:
        a.record(s)
        pkv.mfma_probe(iters, sink)
        b.record(s)
    torch.cuda.synchronize()
    mms = sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2]
    del sink
    props = torch.cuda.get_device_properties(0)
    ctx = {"name": props.name, "compute_units": props.multi_processor_count,
           "copy_GBps": round(2 * 2 * n / (ms * 1e-3) / 1e9, 1),
           "copy_note": "1 GiB device-to-device copy, read + write bytes",
           "read_GBps": round(read_bytes / (rms * 1e-3) / 1e9, 1),
           "read_note": "2 GiB read once by pkv_read_probe (16-byte non-temporal loads): the practical read "
                        "ceiling for the HBM-bound decode kernels",
           "mfma_bf16_TFLOPs": round(pkv.mfma_probe_flops(iters) / (mms * 1e-3) / 1e12, 1),
           "mfma_note": "pkv_mfma_probe: two chains of v_mfma_f32_32x32x16_bf16 per wave, two waves per SIMD, no "
                        "memory traffic (median of 10): the practical ceiling for the MFMA-bound prefill and "
                        "projection (the part runs below 2.4 GHz under this load)"}
    clocks = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                cur = [ln for ln in fh.read().split("\n") if ln.strip().endswith("*")]
            clocks += [c.split(":", 1)[1].strip(" *") for c in cur]
        except OSError:
            pass
    ctx["sclk_current"] = clocks[0] if len(clocks) == 1 else None
    return ctx


def time_long_decode(args):
    """Decode at a bandwidth-bound scale: 256 sequences sharing a 4096-token
    prefix (aliased blocks) plus 0..2048 private tokens, and 16 sequences of
    32768 cached tokens (3.24 GB of unique K/V, 7.5 GB logical).  Lengths and
    placement follow the seeded recipe; K/V/q values are drawn on the device
    (timing only, no parity claim)."""
    import torch
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import DeviceCase

    case = W.config5_prefix_long(draw_values=False)
    dec = case.steps[0].decode
    uniq = W.decode_unique_kv_bytes(case, dec)
    logical = W.decode_logical_kv_bytes(case, dec)
    dc = DeviceCase(case)
    dc.run_fills()
    step = dc.steps[0]
    dc.append(step["append"])
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dc.decode(step["decode"])
    torch.cuda.synchronize()
    n = max(5, args.prefill_steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        dc.decode(step["decode"])
        b.record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.mean(times))
    del dc
    torch.cuda.empty_cache()
    gbs = uniq / (ms * 1e-3) / 1e9
    res = {"workload": "qwen3-8b decode, 256 seqs sharing a 4096-token prefix + U[0,2048] private, 16 seqs x 32768; "
                        "32q/8kv, d128, block 256",
            "ms": round(ms, 5), "ms_median": round(float(np.median(times)), 5),
            "ms_min": round(float(np.min(times)), 5),
            "launches_timed": len(times), "unique_kv_bytes": int(uniq), "logical_kv_bytes": int(logical),
            "value": round(gbs, 2), "unit": "GB/s", "logical_gbs": round(logical / (ms * 1e-3) / 1e9, 2),
            "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode (decode_kernel + decode_merge_kernel)",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    attach_traffic(res["roofline"], "long_decode")
    return res


def _private_long_case():
    """16 sequences of 32768 cached tokens + 1 new, private blocks (seeded
    lengths and placement, values drawn on the device)."""
    from paged_kv_gqa_scatter_amd import workloads as W
    rng = np.random.default_rng(16)
    return W.build_case("qwen3_8b_16x32k_private", rng, hq=32, hkv=8, d=128, bs=256,
                        ctx_lens=np.full(16, 32768), new_lens=np.ones(16, np.int64), kinds="d" * 16,
                        draw_values=False)


def _time_decode_calls(dc, n):
    """Events around each of n decode calls of step 0 (after its append and
    3 untimed calls): the per-call times in ms."""
    import torch
    step = dc.steps[0]
    dc.append(step["append"])
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dc.decode(step["decode"])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        dc.decode(step["decode"])
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_private_long_decode(args):
    """Decode over private long contexts only: 16 sequences of 32768 cached
    tokens + 1 (2.15 GB of K/V, no block shared), the streaming rate of the
    split kernel without the shared prefix of the long-context workload.
    Lengths and placement seeded; values drawn on the device (timing only)."""
    import torch
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import DeviceCase

    case = _private_long_case()
    uniq = W.decode_unique_kv_bytes(case, case.steps[0].decode)
    dc = DeviceCase(case)
    dc.run_fills()
    times = _time_decode_calls(dc, max(5, args.prefill_steps))
    ms = float(np.mean(times))
    del dc
    torch.cuda.empty_cache()
    gbs = uniq / (ms * 1e-3) / 1e9
    return {"workload": "qwen3-8b decode, 16 seqs x 32769 keys, private blocks; 32q/8kv, d128, block 256",
            "ms": round(ms, 5), "ms_median": round(float(np.median(times)), 5),
            "ms_min": round(float(np.min(times)), 5), "launches_timed": len(times), "unique_kv_bytes": int(uniq),
            "value": round(gbs, 2), "unit": "GB/s",
            "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode (decode_kernel + decode_merge_kernel)",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def time_int8(args, bf16_step_ms, bf16_long_ms, bf16_private_ms=None):
    """The INT8 KV cache (quantising kv_append_int8, paged_gqa_decode_int8) on
    the headline decode step (both calls in one HIP graph per pool copy,
    rotated past the last-level cache), on the long-context decode and on
    the private long-context decode (16 x 32769 keys, no shared block: the
    streaming rate, where half the bytes should show as up to twice the
    speed); bytes are the unique code and scale bytes a call must read
    (D + 4 per row)."""
    import torch
    from paged_kv_gqa_scatter_amd import workloads as W
    from paged_kv_gqa_scatter_amd.runner import Int8DeviceCase

    res = {}
    case = W.config2_decode()
    dec = case.steps[0].decode
    nbytes = W.decode_unique_int8_kv_bytes(case, dec)
    pool_bytes = case.pool_bytes * (case.head_dim + 4) // (2 * case.head_dim)
    n_rot = max(1, -(-ROTATE_BYTES // pool_bytes))
    dc = Int8DeviceCase(case, pools=n_rot)
    dc.run_fills()
    step = dc.steps[0]
    ms = _timed_steps(dc.capture, lambda r: dc.decode_append(step["append"], step["decode"], pool=r), n_rot,
                      args.steps, max(args.warmup // 2, 10))
    sms = _timed_steps(dc.capture, lambda r: dc.run_step(0, r), n_rot, args.steps, max(args.warmup // 2, 10))
    dms = _timed_steps(dc.capture, lambda r: dc.decode(step["decode"], pool=r), n_rot, args.steps,
                       max(args.warmup // 2, 10))
    del dc
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    res["decode_step"] = {
        "workload": "the headline decode step over an INT8 cache: one paged_gqa_decode_append_int8 launch "
                    "(quantising append + decode), pool copies' steps in one HIP graph",
        "ms_per_step": round(ms, 5), "bf16_fused_step_ms": round(bf16_step_ms, 5),
        "ms_per_step_append_then_decode": round(sms, 5), "decode_only_ms": round(dms, 5),
        "unique_kv_bytes": int(nbytes),
        "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode_append_int8 (decode_int8_kernel, split "
                                                "sequences merged in the kernel)",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    attach_traffic(res["decode_step"]["roofline"], "int8_decode_append")
    if not args.no_long:
        case = W.config5_prefix_long(draw_values=False)
        dec = case.steps[0].decode
        nbytes = W.decode_unique_int8_kv_bytes(case, dec)
        dc = Int8DeviceCase(case)
        dc.run_fills()
        lms = float(np.mean(_time_decode_calls(dc, max(5, args.prefill_steps))))
        del dc
        torch.cuda.empty_cache()
        gbs = nbytes / (lms * 1e-3) / 1e9
        res["long_context_decode"] = {
            "workload": "the long-context decode (256 seqs on a shared 4096-token prefix + 16 x 32768) over an "
                        "INT8 cache",
            "ms": round(lms, 5), "unique_kv_bytes": int(nbytes),
            "speedup_vs_bf16": round(bf16_long_ms / lms, 3) if bf16_long_ms else None,
            "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode_int8 (decode_int8_kernel + decode_merge_kernel)",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}
        attach_traffic(res["long_context_decode"]["roofline"], "int8_long_decode")
        case = _private_long_case()
        nbytes = W.decode_unique_int8_kv_bytes(case, case.steps[0].decode)
        dc = Int8DeviceCase(case)
        dc.run_fills()
        pms = float(np.mean(_time_decode_calls(dc, max(5, args.prefill_steps))))
        del dc
        torch.cuda.empty_cache()
        gbs = nbytes / (pms * 1e-3) / 1e9
        res["private_long_decode"] = {
            "workload": "the private long-context decode (16 seqs x 32769 keys, no shared block) over an INT8 cache",
            "ms": round(pms, 5), "unique_kv_bytes": int(nbytes),
            "speedup_vs_bf16": round(bf16_private_ms / pms, 3) if bf16_private_ms else None,
            "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode_int8 (decode_int8_kernel + decode_merge_kernel)",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    return res


def time_qkv(args):
    """The fused QKV projection + paged append at Qwen3-8B layer shapes
    (d_model 4096, 32 / 8 heads of 128, merged weight 6144 x 4096): the
    prefill prompts (4 x U[1024, 4096] tokens; flops 2 T N d_model against
    the bf16 MFMA peak) and the decode step (8 tokens; the weight and input
    bytes it must read against HBM peak).  Inputs are N(0, 1) drawn on the
    device (timing only)."""
    import torch
    import paged_kv_gqa_scatter_amd as pkv
    from paged_kv_gqa_scatter_amd import workloads as W

    res = {}
    dm, hq, hkv, d = 4096, 32, 8, 128
    n_out = (hq + 2 * hkv) * d
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0x9C7)
    w = (torch.randn((n_out, dm), generator=gen, device="cuda") / 64).to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    for name, case in (("prefill_prompts", W.config3_prefill(draw_values=False)),
                       ("decode_step", W.config2_decode(draw_values=False))):
        a = case.steps[0].append
        T = int(a.cu_new_lens[-1])
        x = torch.randn((T, dm), generator=gen, device="cuda").to(torch.bfloat16)
        shape = (case.num_blocks, hkv, case.block_size, d)
        kp = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        q = torch.empty((T, hq, d), dtype=torch.bfloat16, device="cuda")
        cu, ctx, tab = (torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in (a.cu_new_lens, a.ctx_lens,
                                                                                    a.block_table))
        call = lambda: pkv.qkv_project_append(x, w, kp, vp, cu, ctx, tab, hq, q_out=q)
        t = time.perf_counter()
        while time.perf_counter() - t < 0.3:
            call()
            torch.cuda.synchronize()
        n = max(10, args.prefill_steps)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for e0, e1 in evs:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        flops = 2 * T * n_out * dm
        nbytes = (n_out * dm + T * dm + T * n_out) * 2
        r = {"tokens": T, "ms": round(ms, 5), "flops": int(flops), "bytes": int(nbytes)}
        if name == "prefill_prompts":
            tfs = flops / (ms * 1e-3) / 1e12
            r["roofline"] = {"bound": "mfma", "kernel": "qkv_project_append (qkv_append_kernel)",
                             "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                             "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
        else:
            gbs = nbytes / (ms * 1e-3) / 1e9
            r["roofline"] = {"bound": "hbm", "kernel": "qkv_project_append (qkv_append_skinny_kernel)",
                             "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}
        attach_traffic(r["roofline"], "qkv" if name == "prefill_prompts" else "qkv_decode")
        res[name] = r
        del x, kp, vp, q
        torch.cuda.empty_cache()
    res["workload"] = ("qwen3-8b fused QKV projection + paged append: x [T][4096] times the merged weight "
                       "[6144][4096], q to q_out, k/v rows into 256-token blocks")
    return res


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, dec, kv_bytes, seconds, pcase=None):
    """The fp64 oracle (plain C, OpenMP) on the host: the same decode step,
    repeated for about `seconds`, with all cores and with one thread; and the
    prefill workload, in full on all cores and on a sample of its rows (every
    8th row of each prompt, all heads) on one thread; and config 1 (_cpu_tiny).
    Reference points only."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from case_oracle import oracle_pools
    orc = oracle.get()
    cores = orc.max_threads()
    K, V = oracle_pools(case, orc)

    def decode_rate(threads, budget):
        reps, t = 0, time.perf_counter()
        while True:
            orc.decode(dec.q, K, V, dec.block_table, dec.seq_lens, case.scale, num_threads=threads)
            reps += 1
            el = time.perf_counter() - t
            if el >= budget:
                return kv_bytes * reps / el / 1e9, reps, el

    gbs, reps, el = decode_rate(cores, seconds)
    gbs1, reps1, el1 = decode_rate(1, seconds / 2)
    res = {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"the whole decode step ({dec.seq_lens.shape[0]} seqs, {int(dec.seq_lens.sum())} keys, "
                     f"32/8 heads, d128), fp64, repeated {reps}x over {el:.1f} s",
           "cpu_model": _cpu_model(),
           "one_thread": {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                          "sample": f"the same step repeated {reps1}x over {el1:.1f} s"}}
    if pcase is not None:
        p = pcase.steps[0].prefill
        PK, PV = oracle_pools(pcase, orc)
        D, Hq = pcase.head_dim, pcase.num_q_heads
        t = time.perf_counter()
        orc.attention(p.q, p.cu_q_lens, PK, PV, p.block_table, p.seq_lens, Hq, pcase.scale, num_threads=cores)
        el = time.perf_counter() - t
        S = p.seq_lens.shape[0]
        flops = 0
        items = []
        for s in range(S):
            n = int(p.cu_q_lens[s + 1] - p.cu_q_lens[s])
            ctx = int(p.seq_lens[s]) - n
            flops += 4 * D * Hq * (n * ctx + n * (n + 1) // 2)
        sflops = 0
        for s in range(S):
            n = int(p.cu_q_lens[s + 1] - p.cu_q_lens[s])
            ctx = int(p.seq_lens[s]) - n
            for r in range(0, n, 8):
                for h in range(Hq):
                    items.append((s, r, h))
                sflops += 4 * D * Hq * (ctx + r + 1)
        t = time.perf_counter()
        orc.attention_rows(np.array(items, np.int32), p.q, p.cu_q_lens, PK, PV, p.block_table, p.seq_lens, Hq,
                           pcase.scale, num_threads=1)
        el1 = time.perf_counter() - t
        res["prefill"] = {"value": round(flops / el / 1e9, 3), "unit": "GFLOP/s", "cores": cores,
                          "sample": f"the whole prefill workload ({int(p.cu_q_lens[-1])} rows x {Hq} heads, "
                                    f"{flops / 1e9:.1f} GFLOP causal), fp64, once in {el:.1f} s",
                          "one_thread": {"value": round(sflops / el1 / 1e9, 3), "unit": "GFLOP/s", "cores": 1,
                                         "sample": f"every 8th row of each prompt, all heads ({len(items)} rows, "
                                                   f"{sflops / 1e9:.1f} GFLOP) in {el1:.1f} s"}}
    res["tiny"] = _cpu_tiny(orc, cores)
    return res


def _cpu_tiny(orc, cores):
    """Config 1 on the oracle: its 300-row prefill (4 query heads, d64) and a
    decode step (301 keys), each repeated for about a second, on all cores and
    on one thread."""
    from case_oracle import oracle_pools
    from paged_kv_gqa_scatter_amd import workloads as W
    case = W.config1_tiny()
    K, V = oracle_pools(case, orc)  # every step's rows; each call reads only its own positions
    p, d = case.steps[0].prefill, case.steps[1].decode
    D, Hq = case.head_dim, case.num_q_heads
    n = int(p.cu_q_lens[1])
    flops = 4 * D * Hq * (n * (int(p.seq_lens[0]) - n) + n * (n + 1) // 2)
    kv = int(d.seq_lens.sum()) * case.num_kv_heads * D * 2 * 2

    def rate(fn, threads, amount):
        reps, t = 0, time.perf_counter()
        while True:
            fn(threads)
            reps += 1
            el = time.perf_counter() - t
            if el >= 1.0:
                return amount * reps / el / 1e9

    pre = lambda th: orc.attention(p.q, p.cu_q_lens, K, V, p.block_table, p.seq_lens, Hq, case.scale,
                                   num_threads=th)
    dec = lambda th: orc.decode(d.q, K, V, d.block_table, d.seq_lens, case.scale, num_threads=th)
    return {"workload": f"config 1: causal prefill of {n} rows ({Hq} query heads / 1 KV head, d{D}; "
                        f"{flops / 1e6:.1f} MFLOP) and a decode step over {int(d.seq_lens.sum())} keys, fp64, "
                        "each repeated for about 1 s",
            "prefill": {"value": round(rate(pre, cores, flops), 3), "unit": "GFLOP/s", "cores": cores,
                        "one_thread": round(rate(pre, 1, flops), 3)},
            "decode": {"value": round(rate(dec, cores, kv), 4), "unit": "GB/s", "cores": cores,
                       "one_thread": round(rate(dec, 1, kv), 4)}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.profile_pass:
        profile_pass(args)
        return

    case, dec, kv_bytes, n_rot, step_ms, dec_ms, eager_ms, split_ms, one_ms = time_decode_workload(args)
    gbs = kv_bytes / (step_ms * 1e-3) / 1e9
    line = {
        "metric": "paged GQA attn: decode KV-read GB/s + prefill causal TFLOP/s (bf16, 1 GPU)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b one-layer decode step: kv_append + paged_gqa_decode (one decode_append "
                               "launch), 8 seqs, ctx U[512,2048], 32q/8kv heads, d128, block 256",
                   "seqs": int(dec.seq_lens.shape[0]), "keys": int(dec.seq_lens.sum()),
                   "unique_kv_bytes": int(kv_bytes), "pool_copies_rotated": n_rot,
                   "hip_graph": f"the {n_rot} pool copies' steps in one graph (one step per layer of a decode "
                                f"iteration), replayed",
                   "ms_per_step_append_then_decode": round(split_ms, 5),
                   "eager_ms_per_step_append_then_decode": round(eager_ms, 5),
                   "ms_per_step_one_graph_per_step": round(one_ms, 5)},
        "roofline": {"bound": "hbm", "kernel": "paged_gqa_decode_append (decode_kernel, split sequences merged "
                                                "in the kernel), launches back to back in HIP graphs",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": int(kv_bytes),
                     "ms": round(step_ms, 5), "decode_only_ms": round(dec_ms, 5)},
    }
    attach_traffic(line["roofline"], "decode_append")
    if not args.no_prefill:
        pcase, flops, pms, pmed, pmin = time_prefill_workload(args)
        tfs = flops / (pms * 1e-3) / 1e12
        line["prefill"] = {
            "workload": "qwen3-8b one-layer causal prefill: 4 prompts U[1024,4096], 32q/8kv, d128, block 256",
            "value": round(tfs, 2), "unit": "TFLOP/s", "causal_flops": int(flops), "ms": round(pms, 5),
            "ms_median": round(pmed, 5), "ms_min": round(pmin, 5), "launches_timed": args.prefill_steps,
            "roofline": {"bound": "mfma", "kernel": "paged_gqa_prefill (prefill_kernel)", "achieved": round(tfs, 2),
                         "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                         "traffic": None}}
        attach_traffic(line["prefill"]["roofline"], "prefill")
    if not args.no_long:
        line["long_context_decode"] = time_long_decode(args)
        line["private_long_decode"] = time_private_long_decode(args)
    if not args.no_qkv:
        line["qkv_project_append"] = time_qkv(args)
    if not args.no_int8:
        line["int8_kv_cache"] = time_int8(args, step_ms, line.get("long_context_decode", {}).get("ms"),
                                          line.get("private_long_decode", {}).get("ms"))
    if not args.no_mixed:
        line["mixed_step"] = time_mixed_step(args)
    if not args.no_append:
        line["kv_append"] = time_kv_append(args)
    line["device"] = device_context()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, dec, kv_bytes, args.cpu_seconds,
                                            None if args.no_prefill else pcase)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

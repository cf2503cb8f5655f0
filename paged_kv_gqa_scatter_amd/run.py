"""Run one of the named workloads through the library on cuda:0.

    python -m paged_kv_gqa_scatter_amd.run --config N [--seed S] [--repeat R] [--int8]

Configs (``workloads.py``): 1 a tiny GQA prefill then 8 decode steps, 2 the
Qwen3-8B decode step (8 sequences), 3 the causal prefill of 4 prompts,
4 the mixed step (64 decodes beside two 512-row chunks), 5 the long-context
decode (256 sequences on a shared 4096-token prefix plus 16 of 32768 tokens).
``--seed`` replaces the config's default seed (lengths, placement and, where
the config draws them on the host, the values).  Each step of the config is
run ``--repeat`` times after the cache fills; one JSON line per step gives its
calls, shapes and the mean, median and minimum time of the repeats (HIP
events on the current stream, eager calls, after one untimed run).
``--int8`` runs the steps over an INT8 cache (configs 2 and 5: the INT8
cache has decode steps only).

Plumbing only, like ``runner``: every step is the library's kernels.
Results are not checked here; the tests compare them with the oracle.
"""
from __future__ import annotations

import argparse
import json
import sys

CONFIGS = {1: "config1_tiny", 2: "config2_decode", 3: "config3_prefill", 4: "config4_mixed",
           5: "config5_prefix_long"}


def parse_args(argv=None) -> argparse.Namespace:
    ap = argparse.ArgumentParser(prog="python -m paged_kv_gqa_scatter_amd.run",
                                 description="run a named workload through libpkv on cuda:0")
    ap.add_argument("--config", type=int, required=True, choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=None, help="seed of the workload (default: the config's own)")
    ap.add_argument("--repeat", type=int, default=10, help="timed runs of each step (>= 1)")
    ap.add_argument("--int8", action="store_true", help="an INT8 KV cache instead of bf16")
    args = ap.parse_args(argv)
    if args.repeat < 1:
        ap.error("--repeat must be >= 1")
    if args.int8 and args.config not in (2, 5):
        ap.error("--int8 runs configs 2 and 5 only (the INT8 cache has decode steps only)")
    return args


def build_case(config: int, seed=None):
    """The named workload, with ``seed`` in place of its default when given;
    K/V and q values are drawn on the device where the config allows it (the
    large configs)."""
    import inspect
    from . import workloads as W
    fn = getattr(W, CONFIGS[config])
    kw = {} if seed is None else {"seed": seed}
    params = inspect.signature(fn).parameters
    if "draw_values" in params:
        kw["draw_values"] = False
    return fn(**kw)


def main(argv=None) -> int:
    args = parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU: the library runs on cuda:0 only"}), flush=True)
        return 2
    from .runner import DeviceCase, Int8DeviceCase

    case = build_case(args.config, args.seed)
    dc = (Int8DeviceCase if args.int8 else DeviceCase)(case)
    dc.run_fills()
    stream = torch.cuda.current_stream()
    for i, st in enumerate(case.steps):
        calls = [k for k in ("append", "decode", "prefill") if getattr(st, k) is not None]
        dc.run_step(i)  # untimed: first calls (stream, workspace) and the step's rows written once
        times = []
        for r in range(args.repeat):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dc.run_step(i)  # rewrites the same rows, then decodes / prefills as the first run did
            b.record(stream)
            times.append((a, b))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in times]
        line = {"config": case.name, "step": i, "calls": calls, "cache": "int8" if args.int8 else "bf16",
                "repeats": args.repeat, "ms_mean": round(sum(ms) / len(ms), 5),
                "ms_median": round(sorted(ms)[len(ms) // 2], 5), "ms_min": round(min(ms), 5)}
        if st.decode is not None:
            line["decode_seqs"] = int(len(st.decode.seq_lens))
            line["decode_keys"] = int(st.decode.seq_lens.sum())
        if st.prefill is not None:
            line["prefill_rows"] = int(st.prefill.cu_q_lens[-1])
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Run a seeded workload (``workloads.Case``) through the HIP library.

Plumbing only: it copies the generated inputs to the GPU, creates the pools
filled with the NaN sentinel, and calls ``kv_append`` / ``paged_gqa_decode`` /
``paged_gqa_prefill`` in the order the case lists them.  All arithmetic
happens in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import (decode_int8_workspace_bytes, decode_workspace_bytes, kv_append, kv_append_int8, paged_gqa_decode,
               paged_gqa_decode_append, paged_gqa_decode_append_int8, paged_gqa_decode_int8, paged_gqa_prefill)
from .workloads import INT8_CODE_SENTINEL, NAN_SENTINEL, AppendBatch, Case, DecodeBatch, Deferred, PrefillBatch


_device_gen = {}


def _bits(a, device) -> torch.Tensor:
    """uint16 bf16 bits -> a CUDA bf16 tensor with the same bits; a Deferred
    array is drawn here as N(0,1) with torch's seeded device generator."""
    if isinstance(a, Deferred):
        gen = _device_gen.get(str(device))
        if gen is None:
            gen = _device_gen[str(device)] = torch.Generator(device=device)
            gen.manual_seed(0x5EED)
        return torch.randn(a.shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def _i32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


@dataclass
class DevAppend:
    k_new: torch.Tensor
    v_new: torch.Tensor
    cu_new_lens: torch.Tensor
    ctx_lens: torch.Tensor
    block_table: torch.Tensor


@dataclass
class DevDecode:
    q: torch.Tensor
    seq_lens: torch.Tensor
    block_table: torch.Tensor
    max_seq_len: int
    total_kv_tokens: int
    out: torch.Tensor
    workspace: torch.Tensor


@dataclass
class DevPrefill:
    q: torch.Tensor
    cu_q_lens: torch.Tensor
    seq_lens: torch.Tensor
    block_table: torch.Tensor
    max_q_len: int
    max_seq_len: int
    out: torch.Tensor


def capture_graph(fn) -> "torch.cuda.CUDAGraph":
    """Record what ``fn()`` launches on the current stream into a HIP graph
    (torch.cuda.CUDAGraph); ``replay()`` reruns it with the same buffers.  The
    library's calls allocate nothing, synchronise nothing and clear nothing
    with memset, so a whole step can be captured; ``fn`` runs once eagerly
    first, on a side stream, as torch's capture requires."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        fn()
    cur.wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


class DeviceCase:
    """A case resident on one GPU: pools, and every batch's inputs and outputs
    preallocated, so that running a step allocates nothing."""

    def __init__(self, case: Case, device: str = "cuda", pools: int = 1):
        self.case = case
        self.device = torch.device(device)
        self._side = None  # second stream of a step with both decode and prefill
        self._mixed = {}   # such steps' append batches split into decode and prefill rows
        shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
        self.pools = []
        for _ in range(pools):  # several copies let a timing loop rotate past the caches
            k = torch.full(shape, NAN_SENTINEL, dtype=torch.int16, device=self.device).view(torch.bfloat16)
            v = torch.full(shape, NAN_SENTINEL, dtype=torch.int16, device=self.device).view(torch.bfloat16)
            self.pools.append((k, v))
        self.fills = [self._append(b) for b in case.fills]
        self.steps = []
        for st in case.steps:
            self.steps.append({
                "append": self._append(st.append) if st.append is not None else None,
                "decode": self._decode(st.decode) if st.decode is not None else None,
                "prefill": self._prefill(st.prefill) if st.prefill is not None else None,
            })

    @property
    def k_pool(self):
        return self.pools[0][0]

    @property
    def v_pool(self):
        return self.pools[0][1]

    def _append(self, b: AppendBatch) -> DevAppend:
        d = self.device
        return DevAppend(_bits(b.k_new, d), _bits(b.v_new, d), _i32(b.cu_new_lens, d), _i32(b.ctx_lens, d),
                         _i32(b.block_table, d))

    def _decode(self, b: DecodeBatch) -> DevDecode:
        d = self.device
        c = self.case
        S = b.seq_lens.shape[0]
        max_len = int(b.seq_lens.max()) if S else 0
        total = int(b.seq_lens.astype(np.int64).sum())
        ws = decode_workspace_bytes(S, c.num_q_heads, c.num_kv_heads, c.head_dim, max_len, total) if S else 16
        return DevDecode(_bits(b.q, d), _i32(b.seq_lens, d), _i32(b.block_table, d), max_len, total,
                         torch.empty((S, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device=d),
                         torch.zeros(max(ws, 16), dtype=torch.uint8, device=d))

    def _prefill(self, b: PrefillBatch) -> DevPrefill:
        d = self.device
        c = self.case
        T = int(b.cu_q_lens[-1])
        return DevPrefill(_bits(b.q, d), _i32(b.cu_q_lens, d), _i32(b.seq_lens, d), _i32(b.block_table, d),
                          b.max_q_len, int(b.seq_lens.max()) if b.seq_lens.size else 0,
                          torch.empty((T, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device=d))

    # ------------------------------------------------------------------ calls
    def append(self, a: DevAppend, pool: int = 0):
        k, v = self.pools[pool]
        kv_append(k, v, a.k_new, a.v_new, a.cu_new_lens, a.ctx_lens, a.block_table)

    def decode(self, dd: DevDecode, pool: int = 0):
        k, v = self.pools[pool]
        return paged_gqa_decode(dd.q, k, v, dd.block_table, dd.seq_lens, float(self.case.scale),
                                max_seq_len=dd.max_seq_len, total_kv_tokens=dd.total_kv_tokens, out=dd.out,
                                workspace=dd.workspace)

    def decode_append(self, a: DevAppend, dd: DevDecode, pool: int = 0):
        """The step's append and decode in one launch; `a` must add exactly
        one row per sequence of `dd`, in the same order (a decode step)."""
        k, v = self.pools[pool]
        S = dd.q.shape[0]
        return paged_gqa_decode_append(dd.q, a.k_new.view(S, *a.k_new.shape[1:]), a.v_new.view(S, *a.v_new.shape[1:]),
                                       k, v, dd.block_table, dd.seq_lens, float(self.case.scale),
                                       max_seq_len=dd.max_seq_len, total_kv_tokens=dd.total_kv_tokens, out=dd.out,
                                       workspace=dd.workspace)

    def prefill(self, pp: DevPrefill, pool: int = 0):
        k, v = self.pools[pool]
        return paged_gqa_prefill(pp.q, pp.cu_q_lens, k, v, pp.block_table, pp.seq_lens, float(self.case.scale),
                                 max_q_len=pp.max_q_len, max_seq_len=pp.max_seq_len, out=pp.out)

    def run_fills(self, pool: Optional[int] = None):
        for p in (range(len(self.pools)) if pool is None else [pool]):
            for f in self.fills:
                self.append(f, p)

    def _mixed_parts(self, i: int):
        """The append batch of step i split into its decode rows (one per
        decode sequence, first in the batch) and its prefill rows."""
        if i not in self._mixed:
            a, nd = self.steps[i]["append"], self.steps[i]["decode"].q.shape[0]
            dec = DevAppend(a.k_new[:nd], a.v_new[:nd], a.cu_new_lens[:nd + 1], a.ctx_lens[:nd], a.block_table[:nd])
            pre = DevAppend(a.k_new[nd:], a.v_new[nd:], (a.cu_new_lens[nd:] - nd).contiguous(), a.ctx_lens[nd:],
                            a.block_table[nd:])
            self._mixed[i] = (dec, pre)
        return self._mixed[i]

    def run_step(self, i: int, pool: int = 0) -> Dict[str, torch.Tensor]:
        """Step i: its append, then its decode and prefill.  A step with both
        runs them side by side: the decode sequences' rows are appended by the
        decode itself (decode_append) on the current stream, while a second
        stream appends the prefill rows and runs the prefill -- the decode
        streams HBM while the prefill keeps the matrix cores busy.  Captured
        in a graph, the two are parallel branches."""
        st = self.steps[i]
        res = {}
        if st["append"] is not None and st["decode"] is not None and st["prefill"] is not None:
            dec, pre = self._mixed_parts(i)
            cur = torch.cuda.current_stream(self.device)
            if self._side is None:
                self._side = torch.cuda.Stream(self.device)  # default priority
            self._side.wait_stream(cur)
            with torch.cuda.stream(self._side):
                self.append(pre, pool)
                res["prefill"] = self.prefill(st["prefill"], pool)
            res["decode"] = self.decode_append(dec, st["decode"], pool)
            cur.wait_stream(self._side)
            return res
        if st["append"] is not None:
            self.append(st["append"], pool)
        if st["decode"] is not None:
            res["decode"] = self.decode(st["decode"], pool)
        if st["prefill"] is not None:
            res["prefill"] = self.prefill(st["prefill"], pool)
        return res

    def capture(self, fn) -> "torch.cuda.CUDAGraph":
        """``capture_graph(fn)``."""
        return capture_graph(fn)

    def capture_step(self, i: int, pool: int = 0) -> "torch.cuda.CUDAGraph":
        """A HIP graph of step ``i`` (append, then decode and/or prefill)."""
        return self.capture(lambda: self.run_step(i, pool))

    def run_all(self) -> list:
        """Fills, then every step in order; returns each step's outputs as fp64 numpy."""
        self.run_fills(0)
        outs = []
        for i in range(len(self.steps)):
            r = self.run_step(i)
            outs.append({k: v.float().cpu().numpy().astype(np.float64) for k, v in r.items()})
        return outs

    def pools_numpy(self, pool: int = 0):
        k, v = self.pools[pool]
        return (k.view(torch.int16).cpu().numpy().view(np.uint16), v.view(torch.int16).cpu().numpy().view(np.uint16))


class Int8DeviceCase(DeviceCase):
    """The same case over an INT8 KV cache (include/pkv_int8.h): appends
    quantise, decodes read codes and scales.  Pools are (k_codes, v_codes,
    k_scales, v_scales); unwritten codes hold -128 and unwritten scales NaN.
    Decode steps only (there is no INT8 prefill)."""

    def __init__(self, case: Case, device: str = "cuda", pools: int = 1):
        if any(st.prefill is not None for st in case.steps):
            raise ValueError("the INT8 cache has decode steps only")
        super().__init__(case, device, pools=0)
        shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
        for _ in range(pools):
            codes = [torch.full(shape, INT8_CODE_SENTINEL, dtype=torch.int8, device=self.device) for _ in range(2)]
            scales = [torch.full(shape[:3], float("nan"), dtype=torch.float32, device=self.device) for _ in range(2)]
            self.pools.append((codes[0], codes[1], scales[0], scales[1]))

    def _decode(self, b: DecodeBatch) -> DevDecode:
        dd = super()._decode(b)
        c = self.case
        S = b.seq_lens.shape[0]
        ws = decode_int8_workspace_bytes(S, c.num_q_heads, c.num_kv_heads, c.head_dim, dd.max_seq_len,
                                         dd.total_kv_tokens) if S else 16
        dd.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=self.device)
        return dd

    def append(self, a: DevAppend, pool: int = 0):
        kv_append_int8(*self.pools[pool], a.k_new, a.v_new, a.cu_new_lens, a.ctx_lens, a.block_table)

    def decode(self, dd: DevDecode, pool: int = 0):
        return paged_gqa_decode_int8(dd.q, *self.pools[pool], dd.block_table, dd.seq_lens, float(self.case.scale),
                                     max_seq_len=dd.max_seq_len, total_kv_tokens=dd.total_kv_tokens, out=dd.out,
                                     workspace=dd.workspace)

    def decode_append(self, a: DevAppend, dd: DevDecode, pool: int = 0):
        """The step's quantising append and decode in one launch; `a` must add
        exactly one row per sequence of `dd`, in the same order."""
        S = dd.q.shape[0]
        return paged_gqa_decode_append_int8(dd.q, a.k_new.view(S, *a.k_new.shape[1:]),
                                            a.v_new.view(S, *a.v_new.shape[1:]), *self.pools[pool], dd.block_table,
                                            dd.seq_lens, float(self.case.scale), max_seq_len=dd.max_seq_len,
                                            total_kv_tokens=dd.total_kv_tokens, out=dd.out, workspace=dd.workspace)

    def prefill(self, pp: DevPrefill, pool: int = 0):
        raise NotImplementedError("the INT8 cache has decode steps only")

    def pools_numpy(self, pool: int = 0):
        return tuple(t.cpu().numpy() for t in self.pools[pool])

"""Seeded synthetic inputs for paged-KV causal GQA attention.

This module only *generates inputs*: sequence lengths, the physical placement
of KV blocks (block tables), and bf16 samples of N(0, 1).  It holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method's code.

Shapes follow the Qwen3-8B engine described on the page "扔掉 vLLM！从零构建
Qwen3-8B 推理引擎" (section 4.3.1: KV cut into fixed 256-token blocks handed out
from a pool of free blocks; section 4.4.2: several query heads share one KV
head).  Head counts (32 query / 8 KV heads, head_dim 128) are Qwen3-8B's.

Recipe (the same for every case):
  1. lengths are drawn first (config-specific, below);
  2. one permutation of the whole pool of ``num_blocks`` physical blocks is
     drawn, and logical blocks take physical ids from it in order: a shared
     prefix first (if any), then each sequence's private blocks in sequence
     order;
  3. K rows for every token ever written (context fills first, then the
     step's new tokens), as fp32 N(0,1) rounded to bf16 (round-to-nearest-even);
  4. V rows, the same way;
  5. q rows for the step (one per decode sequence, ``new_len`` per prefill
     sequence), the same way.
Unwritten pool slots hold the quiet-NaN bf16 pattern ``NAN_SENTINEL`` so that a
kernel reading a slot it must not read shows up as NaN.

Pool layout (both K and V): ``[num_blocks][num_kv_heads][block_size][head_dim]``
bf16, stored as uint16 bit patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NAN_SENTINEL = 0x7FC1  # a quiet-NaN bf16 bit pattern
INT8_CODE_SENTINEL = -128  # never produced by the symmetric INT8 quantiser (codes are in [-127, 127])
_DRAW_CHUNK = 1 << 25  # fp32 samples drawn per numpy call


def bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) fp32 samples rounded to bf16 (RNE); returned as uint16 bits.

    Drawn in chunks of ``_DRAW_CHUNK`` values in C order, so peak host memory
    stays bounded for the multi-GB pools of the long-context case.
    """
    import torch

    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _DRAW_CHUNK):
        hi = min(n, lo + _DRAW_CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out.reshape(shape)


class Deferred:
    """Stands for a bf16 N(0,1) array that is drawn later, on the device.
    Slicing keeps track of the shape only."""

    def __init__(self, shape):
        self.shape = tuple(int(x) for x in shape)

    def __getitem__(self, key):
        if isinstance(key, slice):
            n = len(range(*key.indices(self.shape[0])))
            return Deferred((n,) + self.shape[1:])
        raise TypeError("Deferred arrays only support row slices")


@dataclass
class AppendBatch:
    """New K/V rows for ``kv_append``: rows of sequence s go to positions
    ``ctx_lens[s] .. ctx_lens[s] + new_len_s - 1`` of that sequence."""
    k_new: np.ndarray        # uint16 [T_new][Hkv][D]
    v_new: np.ndarray        # uint16 [T_new][Hkv][D]
    cu_new_lens: np.ndarray  # int32 [S+1]
    ctx_lens: np.ndarray     # int32 [S]
    block_table: np.ndarray  # int32 [S][MBS]

    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def total_new(self) -> int:
        return int(self.cu_new_lens[-1])


@dataclass
class DecodeBatch:
    """One query row per sequence, attending to keys ``0 .. seq_len-1``."""
    q: np.ndarray            # uint16 [S][Hq][D]
    seq_lens: np.ndarray     # int32 [S]
    block_table: np.ndarray  # int32 [S][MBS]


@dataclass
class PrefillBatch:
    """``q_len_s`` query rows per sequence; row r sits at absolute position
    ``seq_len_s - q_len_s + r`` and attends to keys ``0 ..`` that position."""
    q: np.ndarray            # uint16 [T_q][Hq][D]
    cu_q_lens: np.ndarray    # int32 [S+1]
    seq_lens: np.ndarray     # int32 [S]
    block_table: np.ndarray  # int32 [S][MBS]

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.cu_q_lens).max()) if self.seq_lens.size else 0


@dataclass
class Step:
    append: Optional[AppendBatch] = None
    decode: Optional[DecodeBatch] = None
    prefill: Optional[PrefillBatch] = None


@dataclass
class Case:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: np.float32
    fills: List[AppendBatch] = field(default_factory=list)  # context, written before the steps
    steps: List[Step] = field(default_factory=list)

    def empty_pool(self) -> np.ndarray:
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        return np.full(shape, NAN_SENTINEL, dtype=np.uint16)

    @property
    def pool_bytes(self) -> int:
        return 2 * self.num_blocks * self.num_kv_heads * self.block_size * self.head_dim * 2


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def build_case(name: str, rng: np.random.Generator, *, hq: int, hkv: int, d: int, bs: int,
               ctx_lens, new_lens, kinds, spare: float = 0.25, num_blocks: Optional[int] = None,
               shared_prefix: int = 0, shared_seqs=None, scale: Optional[float] = None,
               placement_seed: Optional[int] = None, draw_values: bool = True) -> Case:
    """One batch of sequences: ``ctx_lens[s]`` tokens already cached (written
    by the fills), then a step that appends ``new_lens[s]`` tokens and runs
    decode (``kinds[s] == 'd'``, needs new_len 1) or chunked prefill
    (``kinds[s] == 'p'``).  Decode sequences must come before prefill ones so
    that each attention call sees a contiguous slice of the table.

    ``shared_prefix`` tokens (a whole number of blocks) are aliased: the
    sequences listed in ``shared_seqs`` all map their first blocks to the same
    physical blocks, which are written once by a fill of their own.

    ``placement_seed`` replaces the drawn block permutation by one from another
    generator (the draw still happens, so the samples do not change): the same
    data at a different physical placement.

    ``draw_values=False`` skips steps (3)-(5): K/V/q arrays are left as None
    (with their shapes recorded) for timing runs that draw N(0,1) values on the
    device instead; lengths and placement are unchanged.
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    new_lens = np.asarray(new_lens, dtype=np.int64)
    kinds = list(kinds)
    S = len(ctx_lens)
    assert len(new_lens) == S and len(kinds) == S
    nd = sum(1 for k in kinds if k == "d")
    assert all(k == "d" for k in kinds[:nd]) and all(k == "p" for k in kinds[nd:])
    assert all(new_lens[s] == 1 for s in range(nd))
    shared_seqs = set(range(S) if shared_seqs is None else shared_seqs) if shared_prefix else set()
    assert shared_prefix % bs == 0
    n_pref_blocks = shared_prefix // bs
    for s in shared_seqs:
        assert ctx_lens[s] >= shared_prefix

    final = ctx_lens + new_lens
    nblk = [_ceil_div(int(x), bs) for x in final]
    mbs = max(1, max(nblk) if nblk else 1)
    needed = n_pref_blocks + sum(nblk[s] - (n_pref_blocks if s in shared_seqs else 0) for s in range(S))
    if num_blocks is None:
        num_blocks = needed + int(math.ceil(spare * needed))
    assert num_blocks >= needed

    # (2) physical placement
    perm = rng.permutation(num_blocks).astype(np.int32)
    if placement_seed is not None:
        perm = np.random.default_rng(placement_seed).permutation(num_blocks).astype(np.int32)
    table = np.full((S, mbs), -1, dtype=np.int32)
    nxt = n_pref_blocks
    pref_ids = perm[:n_pref_blocks]
    for s in range(S):
        start = 0
        if s in shared_seqs:
            table[s, :n_pref_blocks] = pref_ids
            start = n_pref_blocks
        cnt = nblk[s] - start
        table[s, start:nblk[s]] = perm[nxt:nxt + cnt]
        nxt += cnt

    # token accounting: context fills (prefix once, then private context), then the step
    fill_ctx = np.array([shared_prefix if s in shared_seqs else 0 for s in range(S)], dtype=np.int64)
    fill_new = ctx_lens - fill_ctx
    n_fill = shared_prefix + int(fill_new.sum())
    n_step = int(new_lens.sum())

    # (3) K rows, (4) V rows: fills first, then the step; (5) q rows of the step
    if draw_values:
        k_all = bf16_normal(rng, (n_fill + n_step, hkv, d))
        v_all = bf16_normal(rng, (n_fill + n_step, hkv, d))
        q_all = bf16_normal(rng, (n_step, hq, d))
    else:
        k_all = v_all = Deferred((n_fill + n_step, hkv, d))
        q_all = Deferred((n_step, hq, d))

    def cu(lens):
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

    fills: List[AppendBatch] = []
    off = 0
    if shared_prefix:
        ptab = np.full((1, mbs), -1, dtype=np.int32)
        ptab[0, :n_pref_blocks] = pref_ids
        fills.append(AppendBatch(k_all[:shared_prefix], v_all[:shared_prefix], cu([shared_prefix]),
                                 np.zeros(1, np.int32), ptab))
        off = shared_prefix
    if fill_new.sum() > 0:
        n = int(fill_new.sum())
        fills.append(AppendBatch(k_all[off:off + n], v_all[off:off + n], cu(fill_new),
                                 fill_ctx.astype(np.int32), table.copy()))
        off += n
    assert off == n_fill

    step = Step()
    step.append = AppendBatch(k_all[n_fill:], v_all[n_fill:], cu(new_lens), ctx_lens.astype(np.int32),
                              table.copy())
    keep = (lambda a: a) if not draw_values else np.ascontiguousarray
    if nd:
        step.decode = DecodeBatch(keep(q_all[:nd]), final[:nd].astype(np.int32), np.ascontiguousarray(table[:nd]))
    if nd < S:
        step.prefill = PrefillBatch(keep(q_all[nd:]), cu(new_lens[nd:]), final[nd:].astype(np.int32),
                                    np.ascontiguousarray(table[nd:]))
    sc = np.float32(1.0 / math.sqrt(d)) if scale is None else np.float32(scale)
    return Case(name, hq, hkv, d, bs, int(num_blocks), int(mbs), sc, fills, [step])


# --------------------------------------------------------------------------
# The five workloads.  Config k draws from numpy.random.default_rng(k).
# --------------------------------------------------------------------------

def config1_tiny(seed: int = 1, block_size: int = 16, num_blocks: int = 32, perm_blocks: Optional[np.ndarray] = None) -> Case:
    """Tiny single-layer case: 1 sequence, 4 query heads sharing 1 KV head,
    head_dim 64, block 16.  A causal prefill over a 300-token prompt, then 8
    decode steps (each appends one token and attends over 301..308 tokens).
    Blocks sit at a random permutation of a 32-block pool."""
    rng = np.random.default_rng(seed)
    hq, hkv, d = 4, 1, 64
    n_prompt, n_dec = 300, 8
    total = n_prompt + n_dec
    nblk = _ceil_div(total, block_size)
    perm = rng.permutation(num_blocks).astype(np.int32)
    if perm_blocks is not None:
        perm = np.asarray(perm_blocks, dtype=np.int32)
    table = np.full((1, nblk), -1, dtype=np.int32)
    table[0, :] = perm[:nblk]
    k_all = bf16_normal(rng, (total, hkv, d))
    v_all = bf16_normal(rng, (total, hkv, d))
    q_all = bf16_normal(rng, (total, hq, d))
    steps = [Step(append=AppendBatch(k_all[:n_prompt], v_all[:n_prompt], np.array([0, n_prompt], np.int32),
                                     np.zeros(1, np.int32), table.copy()),
                  prefill=PrefillBatch(q_all[:n_prompt], np.array([0, n_prompt], np.int32),
                                       np.array([n_prompt], np.int32), table.copy()))]
    for t in range(n_dec):
        pos = n_prompt + t
        steps.append(Step(append=AppendBatch(k_all[pos:pos + 1], v_all[pos:pos + 1], np.array([0, 1], np.int32),
                                             np.array([pos], np.int32), table.copy()),
                          decode=DecodeBatch(q_all[pos:pos + 1], np.array([pos + 1], np.int32), table.copy())))
    return Case("tiny_gqa4_d64_b16_prefill300_decode8", hq, hkv, d, block_size, num_blocks, nblk,
                np.float32(0.125), [], steps)


def config2_decode(seed: int = 2, draw_values: bool = True) -> Case:
    """Qwen3-8B one-layer decode step: 8 sequences, 32/8 heads, d 128,
    block 256, cached context uniform in [512, 2048]; the step appends one
    token per sequence and decodes over ctx+1 keys."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 2048, size=8, endpoint=True)
    return build_case("qwen3_8b_decode_8seq_ctx512_2048", rng, hq=32, hkv=8, d=128, bs=256,
                      ctx_lens=ctx, new_lens=np.ones(8, np.int64), kinds="d" * 8, draw_values=draw_values)


def config3_prefill(seed: int = 3, draw_values: bool = True) -> Case:
    """Qwen3-8B one-layer causal prefill: 4 prompts of length uniform in
    [1024, 4096], 32/8 heads, d 128, block 256; K/V are written by kv_append
    first, then the prefill attends causally over each whole prompt."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 4096, size=4, endpoint=True)
    return build_case("qwen3_8b_prefill_4x1024_4096", rng, hq=32, hkv=8, d=128, bs=256,
                      ctx_lens=np.zeros(4, np.int64), new_lens=lens, kinds="pppp", draw_values=draw_values)


def config4_mixed(seed: int = 4) -> Case:
    """Mixed continuous-batching step: 64 decode sequences with cached context
    log-uniform in [128, 8192], plus 2 chunked-prefill requests that each add
    a 512-token chunk on top of 1024 cached tokens; one step."""
    rng = np.random.default_rng(seed)
    ctx_d = np.rint(np.exp(rng.uniform(math.log(128), math.log(8192), size=64))).astype(np.int64)
    ctx = np.concatenate([ctx_d, [1024, 1024]])
    new = np.concatenate([np.ones(64, np.int64), [512, 512]])
    return build_case("qwen3_8b_mixed_64decode_2x512chunk", rng, hq=32, hkv=8, d=128, bs=256,
                      ctx_lens=ctx, new_lens=new, kinds="d" * 64 + "pp")


def config5_prefix_long(seed: int = 5, n_share: int = 256, n_long: int = 16, long_ctx: int = 32768,
                        prefix: int = 4096, private_max: int = 2048, draw_values: bool = True) -> Case:
    """Prefix-sharing long-context decode: 256 sequences whose first 4096
    tokens alias the same 16 physical blocks, plus 0..2048 private cached
    tokens each; and 16 sequences with 32768 cached tokens.  The step appends
    one token per sequence and decodes."""
    rng = np.random.default_rng(seed)
    priv = rng.integers(0, private_max, size=n_share, endpoint=True)
    ctx = np.concatenate([prefix + priv, np.full(n_long, long_ctx)])
    S = n_share + n_long
    return build_case("qwen3_8b_prefix4096x256_plus_16x32k", rng, hq=32, hkv=8, d=128, bs=256,
                      ctx_lens=ctx, new_lens=np.ones(S, np.int64), kinds="d" * S,
                      shared_prefix=prefix, shared_seqs=range(n_share), draw_values=draw_values)


CONFIGS = {1: config1_tiny, 2: config2_decode, 3: config3_prefill, 4: config4_mixed, 5: config5_prefix_long}


# --------------------------------------------------------------------------
# Algorithmic work units (what the method itself must move or compute).
# --------------------------------------------------------------------------

def decode_unique_kv_bytes(case: Case, batch: DecodeBatch) -> int:
    """Bytes of K and V a decode must read: each distinct physical
    (block, kv_head, slot) row that some sequence attends to, counted once."""
    B = case.block_size
    rows_read = {}  # physical block -> rows of it that some sequence attends to
    for s in range(batch.seq_lens.shape[0]):
        L = int(batch.seq_lens[s])
        for lb in range(_ceil_div(L, B)):
            blk = int(batch.block_table[s, lb])
            rows_read[blk] = max(rows_read.get(blk, 0), min(B, L - lb * B))
    return sum(rows_read.values()) * case.num_kv_heads * case.head_dim * 2 * 2


def decode_unique_int8_kv_bytes(case: Case, batch: DecodeBatch) -> int:
    """The same rows over an INT8 cache: D code bytes plus one fp32 scale per
    row, for K and for V."""
    rows = decode_unique_kv_bytes(case, batch) // (case.head_dim * 2 * 2)
    return rows * (case.head_dim + 4) * 2


def decode_logical_kv_bytes(case: Case, batch: DecodeBatch) -> int:
    return int(batch.seq_lens.astype(np.int64).sum()) * case.num_kv_heads * case.head_dim * 2 * 2


def prefill_causal_flops(case: Case, batch: PrefillBatch) -> int:
    """4 * D * Hq flops (QK^T and PV, multiply-add = 2) per unmasked
    (query, key) pair: row r of a chunk of n rows on ctx cached keys sees
    ctx + r + 1 keys."""
    tot = 0
    for s in range(batch.seq_lens.shape[0]):
        n = int(batch.cu_q_lens[s + 1] - batch.cu_q_lens[s])
        ctx = int(batch.seq_lens[s]) - n
        tot += n * ctx + n * (n + 1) // 2
    return 4 * case.head_dim * case.num_q_heads * tot


def append_bytes(case: Case, batch: AppendBatch) -> int:
    """New rows read plus written, K and V."""
    return 2 * batch.total_new * case.num_kv_heads * case.head_dim * 2 * 2

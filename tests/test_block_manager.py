"""The host block manager and prefix cache (C++, include/pkv_blocks.h), on
the CPU.

The main check drives random operation sequences (append, fork from the
prefix cache, cache a prefix, free) against a plain model of the device
pools: every append writes its token ids into the slots the manager's block
table names (after performing the manager's copy-on-write copies), and after
every operation each live sequence must read back exactly its own token
history through its block table.  That holds only if no two sequences ever
write one slot, shared blocks are copied before being diverged from, and
forks share only blocks holding the right tokens.  Block conservation is
checked alongside: blocks held by live sequences plus the available ones
(free, or cached and held by nobody) are all the blocks.
"""
import numpy as np
import pytest

import paged_kv_gqa_scatter_amd as pkv
from paged_kv_gqa_scatter_amd.blocks import BlockManager


class PoolModel:
    """Token id stored in each (block, slot); None = never written."""

    def __init__(self, num_blocks, block_size):
        self.B = block_size
        self.slots = [[None] * block_size for _ in range(num_blocks)]

    def copy(self, src, dst):
        self.slots[dst] = list(self.slots[src])

    def write(self, table_row, pos, token):
        self.slots[table_row[pos // self.B]][pos % self.B] = token

    def read(self, table_row, n):
        return [self.slots[table_row[p // self.B]][p % self.B] for p in range(n)]


def append_tokens(bm, pool, seq, hist, toks, mbs):
    cow = bm.append(seq, len(toks))
    if cow is not None:
        pool.copy(*cow)
    row = bm.block_table([seq], mbs)[0]
    start = len(hist)
    for i, t in enumerate(toks):
        pool.write(row, start + i, t)
    hist.extend(toks)


def check_all(bm, pool, hists, mbs, num_blocks):
    held = set()
    for s, h in hists.items():
        assert bm.seq_len(s) == len(h)
        row = bm.block_table([s], mbs)[0]
        assert pool.read(row, len(h)) == h, f"sequence {s} reads back wrong tokens"
        nb = -(-len(h) // pool.B)
        assert (row[:nb] >= 0).all() and (row[nb:] == -1).all()
        held.update(int(b) for b in row[:nb])
    assert bm.available() + len(held) == num_blocks, "blocks lost or double counted"


@pytest.mark.parametrize("seed,block_size,num_blocks", [(1, 16, 48), (2, 16, 200), (3, 32, 64), (4, 256, 24)])
def test_random_operations_keep_every_history(seed, block_size, num_blocks):
    rng = np.random.default_rng(seed)
    B, mbs = block_size, 64
    bm = BlockManager(num_blocks, B)
    pool = PoolModel(num_blocks, B)
    hists = {}
    next_id = 0
    vocab = 6  # few distinct ids, so that forks find shared prefixes
    for step in range(400):
        op = rng.integers(5)
        live = list(hists)
        if op == 0 or not live:  # new sequence from the cache (or empty)
            base = hists[live[rng.integers(len(live))]] if live and rng.random() < 0.7 else []
            cut = int(rng.integers(len(base) + 1)) if base else 0
            toks = list(base[:cut]) + [int(x) for x in rng.integers(vocab, size=int(rng.integers(1, 3 * B)))]
            seq = next_id
            next_id += 1
            m = bm.fork(seq, toks)
            assert 0 <= m <= len(toks)
            hists[seq] = list(toks[:m])
            try:
                append_tokens(bm, pool, seq, hists[seq], toks[m:], mbs)
            except pkv.PkvError as e:
                assert e.status == 6  # out of blocks: the sequence keeps its shared prefix only
        elif op == 1:  # decode-like append of a few tokens
            seq = live[rng.integers(len(live))]
            n = int(rng.integers(1, B + 2))
            if len(hists[seq]) + n > mbs * B:
                continue
            before = (bm.available(), bm.seq_len(seq))
            try:
                append_tokens(bm, pool, seq, hists[seq], [int(x) for x in rng.integers(vocab, size=n)], mbs)
            except pkv.PkvError as e:
                assert e.status == 6
                assert (bm.available(), bm.seq_len(seq)) == before, "a failed append changed state"
        elif op == 2:  # cache a prefix of a sequence
            seq = live[rng.integers(len(live))]
            h = hists[seq]
            bm.cache_prefix(seq, h[: int(rng.integers(len(h) + 1))])
        elif op == 3:  # finish a sequence
            seq = live[rng.integers(len(live))]
            bm.free(seq)
            del hists[seq]
        else:  # cache the whole history, then fork an exact copy: all of it must be shared
            seq = live[rng.integers(len(live))]
            h = hists[seq]
            bm.cache_prefix(seq, h)
            twin = next_id
            next_id += 1
            assert bm.fork(twin, h) == len(h)
            hists[twin] = list(h)
        check_all(bm, pool, hists, mbs, num_blocks)
    bm.close()


def test_longest_prefix_whole_blocks_then_partial():
    B = 256
    bm = BlockManager(40, B)
    rng = np.random.default_rng(7)
    p = [int(x) for x in rng.integers(1000, size=600)]  # 2 whole blocks + 88 tokens
    assert bm.append(0, 600) is None
    bm.cache_prefix(0, p)
    assert bm.fork(1, p) == 600                      # the whole prompt
    assert bm.fork(2, p + [5] * 100) == 600          # longer prompt: all cached tokens
    assert bm.fork(3, p[:599]) == 512                # the 87-token tail is not a cached partial block
    assert bm.fork(4, p[:300]) == 256
    assert bm.fork(5, [p[0] + 1] + p[1:]) == 0       # differs in the first token
    t = bm.block_table([0, 1, 2, 3, 4], 4)
    assert (t[1:3, :3] == t[0, :3]).all() and (t[3, :2] == t[0, :2]).all() and t[4, 0] == t[0, 0]
    assert (t[3, 2:] == -1).all() and (t[4, 1:] == -1).all()


def test_copy_on_write_of_a_shared_partial_block():
    B = 16
    bm = BlockManager(8, B)
    toks = list(range(20))                 # one whole block + 4 tokens
    bm.append(0, 20)
    bm.cache_prefix(0, toks)
    assert bm.fork(1, toks) == 20          # shares both blocks
    assert bm.append(0, 1) is None          # the owner writes at the block's frontier in place
    src, dst = bm.append(1, 1)              # the fork must diverge on a private copy
    t = bm.block_table([0, 1], 2)
    assert t[0, 1] == src and t[1, 1] == dst and t[0, 0] == t[1, 0] and src != dst
    assert bm.append(1, 1) is None          # its own block now


def test_cached_blocks_are_evicted_least_recently_used_first():
    B = 16
    bm = BlockManager(4, B)
    a, b = list(range(16)), list(range(100, 116))
    bm.append(0, 16)
    bm.cache_prefix(0, a)
    bm.append(1, 16)
    bm.cache_prefix(1, b)
    bm.free(0)
    bm.free(1)
    assert bm.available() == 4
    assert bm.fork(2, b) == 16             # touches b: a is now the least recently used
    bm.free(2)
    bm.append(3, 48)                       # needs 3 blocks: the 2 free ones and a's
    assert bm.fork(4, b) == 16 and bm.fork(5, a) == 0
    with pytest.raises(pkv.PkvError) as e:
        bm.append(6, 17)                   # b's block is held by sequence 4 now
    assert e.value.status == 6


def test_errors():
    assert not pkv.lib().pkv_bm_create(0, 16)
    assert not pkv.lib().pkv_bm_create(8, 24)
    bm = BlockManager(2, 16)
    with pytest.raises(pkv.PkvError) as e:
        bm.free(9)
    assert e.value.status == 7
    with pytest.raises(pkv.PkvError) as e:
        bm.append(0, 33)                   # needs 3 of 2 blocks
    assert e.value.status == 6 and bm.seq_len(0) == -1 and bm.available() == 2
    bm.append(0, 32)
    with pytest.raises(pkv.PkvError) as e:
        bm.block_table([0], 1)             # 2 blocks do not fit one column
    assert e.value.status == 2
    with pytest.raises(pkv.PkvError) as e:
        bm.cache_prefix(0, list(range(33)))  # longer than the sequence
    assert e.value.status == 2
    with pytest.raises(pkv.PkvError):
        bm.fork(0, [1, 2])                 # sequence 0 exists

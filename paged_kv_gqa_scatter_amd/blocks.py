"""Host block manager and prefix cache (ctypes over ``include/pkv_blocks.h``).

Marshalling only: every decision (free pool, reference counts, copy-on-write,
prefix lookup, eviction) is made by the C++ manager in ``libpkv.so``.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import PkvError, lib


class BlockManager:
    """Physical block ids ``[0, num_blocks)`` of blocks of ``block_size``
    tokens, handed to sequences (see ``pkv_bm_*`` in ``pkv_blocks.h``)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._h = lib().pkv_bm_create(num_blocks, block_size)
        if not self._h:
            raise ValueError("bad block manager sizes")
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            lib().pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _check(st: int, what: str):
        if st != 0:
            raise PkvError(st, what)

    def available(self) -> int:
        return int(lib().pkv_bm_available(self._h))

    def seq_len(self, seq_id: int) -> int:
        return int(lib().pkv_bm_seq_len(self._h, seq_id))

    def append(self, seq_id: int, n_tokens: int) -> Optional[Tuple[int, int]]:
        """Reserve n_tokens positions; returns the (src, dst) block pair to
        copy on the device first (copy-on-write), or None."""
        src, dst = ctypes.c_int32(-1), ctypes.c_int32(-1)
        self._check(lib().pkv_bm_append(self._h, seq_id, n_tokens, ctypes.byref(src), ctypes.byref(dst)), "append")
        return (src.value, dst.value) if src.value >= 0 else None

    def free(self, seq_id: int):
        self._check(lib().pkv_bm_free_sequence(self._h, seq_id), "free_sequence")

    def block_table(self, seq_ids: Sequence[int], max_blocks_per_seq: int) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        out = np.empty((ids.size, max_blocks_per_seq), dtype=np.int32)
        self._check(lib().pkv_bm_block_table(self._h, ids.ctypes.data, ids.size, max_blocks_per_seq,
                                             out.ctypes.data), "block_table")
        return out

    def cache_prefix(self, seq_id: int, tokens: Sequence[int]):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        self._check(lib().pkv_bm_cache_prefix(self._h, seq_id, t.ctypes.data, t.size), "cache_prefix")

    def fork(self, new_seq_id: int, tokens: Sequence[int]) -> int:
        """New sequence on the longest cached prefix of tokens; returns the
        number of tokens whose K/V it shares."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        m = ctypes.c_int32(0)
        self._check(lib().pkv_bm_fork(self._h, new_seq_id, t.ctypes.data, t.size, ctypes.byref(m)), "fork")
        return m.value

"""CPU oracle for paged-KV causal GQA attention (fp64, plain C).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
It shares no code with the HIP library.  See ``pkv_oracle.c`` for what it
computes and which passage of the pages each step follows.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` (hand-worked golden cases, closed forms, a library
routine on special cases, brute force on tiny inputs, invariants, and planted
mistakes that the pins must catch).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

ERRORS = {0: "ok", -1: "bad arguments", -2: "invalid block id or position", -3: "two rows target one slot",
          -4: "out of memory"}


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (C99, -O2, OpenMP)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class OracleError(RuntimeError):
    pass


_I32P = ctypes.POINTER(ctypes.c_int32)
_U16P = ctypes.POINTER(ctypes.c_uint16)
_F64P = ctypes.POINTER(ctypes.c_double)
_I8P = ctypes.POINTER(ctypes.c_int8)
_F32P = ctypes.POINTER(ctypes.c_float)


def _p(a, typ):
    return a.ctypes.data_as(typ)


class Oracle:
    """Thin ctypes front of one compiled oracle library."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            build(out=path) if path == LIB_PATH else None
        self.lib = ctypes.CDLL(path)
        self.lib.oracle_kv_append.restype = ctypes.c_int
        self.lib.oracle_attention.restype = ctypes.c_int
        self.lib.oracle_attention_rows.restype = ctypes.c_int
        self.lib.oracle_max_threads.restype = ctypes.c_int
        self.lib.oracle_quantize_int8.restype = None
        self.lib.oracle_kv_append_int8.restype = ctypes.c_int
        self.lib.oracle_attention_rows_int8.restype = ctypes.c_int
        self.lib.oracle_qkv_project_append.restype = ctypes.c_int

    @staticmethod
    def _check(rc):
        if rc != 0:
            raise OracleError(f"oracle error {rc}: {ERRORS.get(rc, '?')}")

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def kv_append(self, k_pool, v_pool, k_new, v_new, cu_new_lens, ctx_lens, block_table):
        """In place on host pools ``[NB][Hkv][B][D]`` (uint16)."""
        NB, Hkv, B, D = k_pool.shape
        for a in (k_pool, v_pool, k_new, v_new):
            assert a.dtype == np.uint16 and a.flags.c_contiguous
        cu = np.ascontiguousarray(cu_new_lens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        tab = np.ascontiguousarray(block_table, dtype=np.int32)
        assert k_new.shape[1:] == (Hkv, D) and k_new.shape[0] >= cu[-1]
        rc = self.lib.oracle_kv_append(_p(k_pool, _U16P), _p(v_pool, _U16P), _p(k_new, _U16P), _p(v_new, _U16P),
                                       _p(cu, _I32P), _p(ctx, _I32P), _p(tab, _I32P), tab.shape[1],
                                       ctx.shape[0], Hkv, D, B, NB)
        self._check(rc)

    def attention(self, q, cu_q_lens, k_pool, v_pool, block_table, seq_lens, num_q_heads, scale,
                  num_threads: int = 0):
        """All rows: returns fp64 ``[T_q][Hq][D]``; q is packed ``[T_q][Hq][D]`` uint16."""
        NB, Hkv, B, D = k_pool.shape
        q = np.ascontiguousarray(q)
        cu = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
        tab = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        out = np.zeros((int(cu[-1]), num_q_heads, D), dtype=np.float64)
        rc = self.lib.oracle_attention(_p(out, _F64P), _p(q, _U16P), _p(cu, _I32P), _p(k_pool, _U16P),
                                       _p(v_pool, _U16P), _p(tab, _I32P), tab.shape[1], _p(sl, _I32P),
                                       sl.shape[0], num_q_heads, Hkv, D, B, NB, ctypes.c_float(scale),
                                       num_threads)
        self._check(rc)
        return out

    def attention_rows(self, items, q, cu_q_lens, k_pool, v_pool, block_table, seq_lens, num_q_heads, scale,
                       num_threads: int = 0):
        """Selected rows: ``items`` is int [n][3] of (seq, row within the
        sequence's chunk, q head); returns fp64 ``[n][D]``."""
        NB, Hkv, B, D = k_pool.shape
        items = np.asarray(items, dtype=np.int32).reshape(-1, 3)
        s_, r_, h_ = (np.ascontiguousarray(items[:, i]) for i in range(3))
        q = np.ascontiguousarray(q)
        cu = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
        tab = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        out = np.zeros((items.shape[0], D), dtype=np.float64)
        rc = self.lib.oracle_attention_rows(_p(out, _F64P), items.shape[0], _p(s_, _I32P), _p(r_, _I32P),
                                            _p(h_, _I32P), _p(q, _U16P), _p(cu, _I32P), _p(k_pool, _U16P),
                                            _p(v_pool, _U16P), _p(tab, _I32P), tab.shape[1], _p(sl, _I32P),
                                            sl.shape[0], num_q_heads, Hkv, D, B, NB, ctypes.c_float(scale),
                                            num_threads)
        self._check(rc)
        return out

    # ---- INT8 KV cache: codes [NB][Hkv][B][D] int8, scales [NB][Hkv][B] fp32

    def quantize_int8(self, rows):
        """Quantise bf16 rows ``[..., D]`` (uint16): returns (codes int8 of the
        same shape, scales fp32 ``[...]``)."""
        rows = np.ascontiguousarray(rows, dtype=np.uint16)
        D = rows.shape[-1]
        flat = rows.reshape(-1, D)
        codes = np.zeros(flat.shape, np.int8)
        scales = np.zeros(flat.shape[0], np.float32)
        for i in range(flat.shape[0]):
            self.lib.oracle_quantize_int8(_p(codes[i], _I8P), _p(scales[i:i + 1], _F32P), _p(flat[i], _U16P), D)
        return codes.reshape(rows.shape), scales.reshape(rows.shape[:-1])

    def kv_append_int8(self, k_codes, v_codes, k_scales, v_scales, k_new, v_new, cu_new_lens, ctx_lens,
                       block_table):
        """In place on host INT8 pools."""
        NB, Hkv, B, D = k_codes.shape
        for a in (k_codes, v_codes):
            assert a.dtype == np.int8 and a.flags.c_contiguous
        for a in (k_scales, v_scales):
            assert a.dtype == np.float32 and a.flags.c_contiguous and a.shape == (NB, Hkv, B)
        for a in (k_new, v_new):
            assert a.dtype == np.uint16 and a.flags.c_contiguous
        cu = np.ascontiguousarray(cu_new_lens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        tab = np.ascontiguousarray(block_table, dtype=np.int32)
        assert k_new.shape[1:] == (Hkv, D) and k_new.shape[0] >= cu[-1]
        rc = self.lib.oracle_kv_append_int8(_p(k_codes, _I8P), _p(v_codes, _I8P), _p(k_scales, _F32P),
                                            _p(v_scales, _F32P), _p(k_new, _U16P), _p(v_new, _U16P),
                                            _p(cu, _I32P), _p(ctx, _I32P), _p(tab, _I32P), tab.shape[1],
                                            ctx.shape[0], Hkv, D, B, NB)
        self._check(rc)

    def attention_rows_int8(self, items, q, cu_q_lens, k_codes, v_codes, k_scales, v_scales, block_table,
                            seq_lens, num_q_heads, scale, num_threads: int = 0):
        """Selected rows over an INT8 cache (dequantised keys and values)."""
        NB, Hkv, B, D = k_codes.shape
        items = np.asarray(items, dtype=np.int32).reshape(-1, 3)
        s_, r_, h_ = (np.ascontiguousarray(items[:, i]) for i in range(3))
        q = np.ascontiguousarray(q)
        cu = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
        tab = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        kc, vc = np.ascontiguousarray(k_codes, np.int8), np.ascontiguousarray(v_codes, np.int8)
        ks, vs = np.ascontiguousarray(k_scales, np.float32), np.ascontiguousarray(v_scales, np.float32)
        out = np.zeros((items.shape[0], D), dtype=np.float64)
        rc = self.lib.oracle_attention_rows_int8(_p(out, _F64P), items.shape[0], _p(s_, _I32P), _p(r_, _I32P),
                                                 _p(h_, _I32P), _p(q, _U16P), _p(cu, _I32P), _p(kc, _I8P),
                                                 _p(vc, _I8P), _p(ks, _F32P), _p(vs, _F32P), _p(tab, _I32P),
                                                 tab.shape[1], _p(sl, _I32P), sl.shape[0], num_q_heads, Hkv, D,
                                                 B, NB, ctypes.c_float(scale), num_threads)
        self._check(rc)
        return out

    def decode_int8(self, q, k_codes, v_codes, k_scales, v_scales, block_table, seq_lens, scale,
                    num_threads: int = 0):
        """Decode over an INT8 cache: fp64 ``[S][Hq][D]``."""
        S, Hq, D = q.shape
        items = np.array([(s, 0, h) for s in range(S) for h in range(Hq)], np.int32).reshape(-1, 3)
        cu = np.arange(S + 1, dtype=np.int32)
        out = self.attention_rows_int8(items, q.reshape(S, Hq, D), cu, k_codes, v_codes, k_scales, v_scales,
                                       block_table, seq_lens, Hq, scale, num_threads)
        return out.reshape(S, Hq, D)

    # ---- fused QKV projection with the paged append of k and v

    def qkv_project_append(self, k_pool, v_pool, x, w, cu_new_lens, ctx_lens, block_table, num_q_heads):
        """``x [T][d_model]`` and the merged weight ``w [(Hq + 2 Hkv) D][d_model]``
        (uint16 bf16 bits): returns q ``[T][Hq][D]`` and writes the k and v rows
        into the host pools (in place)."""
        NB, Hkv, B, D = k_pool.shape
        for a in (k_pool, v_pool, x, w):
            assert a.dtype == np.uint16 and a.flags.c_contiguous
        T, dm = x.shape
        assert w.shape == ((num_q_heads + 2 * Hkv) * D, dm)
        cu = np.ascontiguousarray(cu_new_lens, dtype=np.int32)
        ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        tab = np.ascontiguousarray(block_table, dtype=np.int32)
        assert T >= cu[-1]
        q = np.zeros((T, num_q_heads, D), np.uint16)
        rc = self.lib.oracle_qkv_project_append(_p(q, _U16P), _p(k_pool, _U16P), _p(v_pool, _U16P), _p(x, _U16P),
                                                _p(w, _U16P), _p(cu, _I32P), _p(ctx, _I32P), _p(tab, _I32P),
                                                tab.shape[1], ctx.shape[0], dm, num_q_heads, Hkv, D, B, NB)
        self._check(rc)
        return q

    # decode is the one-row-per-sequence case of the same definition
    def decode(self, q, k_pool, v_pool, block_table, seq_lens, scale, num_threads: int = 0):
        S, Hq, D = q.shape
        cu = np.arange(S + 1, dtype=np.int32)
        return self.attention(q.reshape(S, Hq, D), cu, k_pool, v_pool, block_table, seq_lens, Hq, scale,
                              num_threads)


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default

"""paged_kv_gqa_scatter_amd: paged-KV causal GQA attention on AMD MI355X.

A thin ctypes binding over ``libpkv.so`` (HIP kernels for gfx950 behind the C
ABI declared in ``include/pkv.h``).  It only marshals arguments: it checks
dtypes, shapes and devices, passes ``data_ptr()`` values and the current
torch stream, and raises on a non-zero status.  Every step of the attention
runs in the library's kernels; there is no fallback of any kind: the first
call raises ImportError when the library has not been built.

Tensors: bf16 tensors may be ``torch.bfloat16`` (or 16-bit integer views of the
same bits); index tensors are ``torch.int32``; all on the same CUDA device.
Host-side size bounds (``max_seq_len``, ``max_q_len``, ``total_kv_tokens``)
are explicit arguments, so no call reads anything back from the device.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

STATUS = {0: "PKV_OK", 1: "PKV_ERR_NULL_POINTER", 2: "PKV_ERR_BAD_SHAPE", 3: "PKV_ERR_MISALIGNED",
          4: "PKV_ERR_WORKSPACE", 5: "PKV_ERR_HIP", 6: "PKV_ERR_NO_BLOCKS", 7: "PKV_ERR_UNKNOWN_SEQ",
          8: "PKV_ERR_SCRATCH_LIMIT"}
EXPORTS = ("pkv_abi_version", "pkv_status_string", "pkv_kv_append", "pkv_decode_workspace_bytes",
           "pkv_decode_workspace_reset", "pkv_paged_gqa_decode", "pkv_paged_gqa_decode_append",
           "pkv_paged_gqa_decode_append_static", "pkv_paged_gqa_prefill")
BLOCK_EXPORTS = ("pkv_bm_create", "pkv_bm_destroy", "pkv_bm_available", "pkv_bm_seq_len", "pkv_bm_append",
                 "pkv_bm_free_sequence", "pkv_bm_block_table", "pkv_bm_cache_prefix", "pkv_bm_fork",
                 "pkv_copy_blocks")
INT8_EXPORTS = ("pkv_kv_append_int8", "pkv_decode_int8_workspace_bytes", "pkv_paged_gqa_decode_int8",
                "pkv_paged_gqa_decode_append_int8")
QKV_EXPORTS = ("pkv_qkv_project_append",)
DIAG_EXPORTS = ("pkv_read_probe", "pkv_mfma_probe")
READ_PROBE_WORKGROUPS = 8192  # PKV_READ_PROBE_WORKGROUPS
MFMA_PROBE_WORKGROUPS = 512  # PKV_MFMA_PROBE_WORKGROUPS
MFMA_PROBE_MAX_ITERS = 1 << 20  # PKV_MFMA_PROBE_MAX_ITERS


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({lib().pkv_status_string(status).decode()})")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libpkv.so is not built ({path}); run `python __graft_entry__.py build` "
                          f"or `python -m paged_kv_gqa_scatter_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pkv_abi_version.restype = I32
    lib.pkv_abi_version.argtypes = []
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [I32]
    lib.pkv_kv_append.restype = I32
    lib.pkv_kv_append.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P]
    lib.pkv_decode_workspace_bytes.restype = SZ
    lib.pkv_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I64]
    lib.pkv_decode_workspace_reset.restype = I32
    lib.pkv_decode_workspace_reset.argtypes = [P, SZ, P]
    lib.pkv_paged_gqa_decode.restype = I32
    lib.pkv_paged_gqa_decode.argtypes = [P, P, P, P, P, I32, P, I32, I64, I32, I32, I32, I32, I32, I32, F32, P, SZ, P]
    lib.pkv_paged_gqa_decode_append.restype = I32
    lib.pkv_paged_gqa_decode_append.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I64, I32, I32, I32, I32, I32, I32,
                                                F32, P, SZ, P]
    lib.pkv_paged_gqa_decode_append_static.restype = I32
    lib.pkv_paged_gqa_decode_append_static.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I64, I32, I32, I32, I32,
                                                       I32, I32, F32, P]
    lib.pkv_bm_create.restype = P
    lib.pkv_bm_create.argtypes = [I32, I32]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_destroy.argtypes = [P]
    lib.pkv_bm_available.restype = I32
    lib.pkv_bm_available.argtypes = [P]
    lib.pkv_bm_seq_len.restype = I32
    lib.pkv_bm_seq_len.argtypes = [P, I64]
    lib.pkv_bm_append.restype = I32
    lib.pkv_bm_append.argtypes = [P, I64, I32, P, P]
    lib.pkv_bm_free_sequence.restype = I32
    lib.pkv_bm_free_sequence.argtypes = [P, I64]
    lib.pkv_bm_block_table.restype = I32
    lib.pkv_bm_block_table.argtypes = [P, P, I32, I32, P]
    lib.pkv_bm_cache_prefix.restype = I32
    lib.pkv_bm_cache_prefix.argtypes = [P, I64, P, I32]
    lib.pkv_bm_fork.restype = I32
    lib.pkv_bm_fork.argtypes = [P, I64, P, I32, P]
    lib.pkv_copy_blocks.restype = I32
    lib.pkv_copy_blocks.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P]
    lib.pkv_kv_append_int8.restype = I32
    lib.pkv_kv_append_int8.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P]
    lib.pkv_decode_int8_workspace_bytes.restype = SZ
    lib.pkv_decode_int8_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I64]
    lib.pkv_paged_gqa_decode_int8.restype = I32
    lib.pkv_paged_gqa_decode_int8.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I64, I32, I32, I32, I32, I32, I32,
                                              F32, P, SZ, P]
    lib.pkv_paged_gqa_decode_append_int8.restype = I32
    lib.pkv_paged_gqa_decode_append_int8.argtypes = [P, P, P, P, P, P, P, P, P, I32, P, I32, I64, I32, I32, I32, I32,
                                                     I32, I32, F32, P, SZ, P]
    lib.pkv_qkv_project_append.restype = I32
    lib.pkv_qkv_project_append.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32, P]
    lib.pkv_read_probe.restype = I32
    lib.pkv_read_probe.argtypes = [P, SZ, P, SZ, P]
    lib.pkv_mfma_probe.restype = I32
    lib.pkv_mfma_probe.argtypes = [I32, P, SZ, P]
    lib.pkv_paged_gqa_prefill.restype = I32
    lib.pkv_paged_gqa_prefill.argtypes = [P, P, P, I32, I32, P, P, P, I32, P, I32, I32, I32, I32, I32, I32, I32,
                                          F32, P]
    return lib


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpkv.so (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _bf16(t: torch.Tensor, name: str, ndim: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype not in _BF16_LIKE:
        raise TypeError(f"{name} must be a bf16 tensor")
    if t.dim() != ndim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {ndim}-d CUDA tensor")
    return t


def _i32(t: torch.Tensor, name: str, ndim: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32:
        raise TypeError(f"{name} must be an int32 tensor")
    if t.dim() != ndim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {ndim}-d CUDA tensor")
    return t


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _pool_shape(k_pool, v_pool):
    _bf16(k_pool, "k_pool", 4)
    _bf16(v_pool, "v_pool", 4)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    return tuple(k_pool.shape)  # (num_blocks, num_kv_heads, block_size, head_dim)


def _check(st: int, what: str):
    if st != 0:
        raise PkvError(st, what)


def kv_append(k_pool, v_pool, k_new, v_new, cu_new_lens, ctx_lens, block_table) -> None:
    """Scatter rows ``k_new/v_new [T][Hkv][D]`` into the pools at positions
    ``ctx_lens[s] ..`` of each sequence (see ``pkv_kv_append``)."""
    NB, Hkv, B, D = _pool_shape(k_pool, v_pool)
    _bf16(k_new, "k_new", 3)
    _bf16(v_new, "v_new", 3)
    if k_new.shape != v_new.shape or tuple(k_new.shape[1:]) != (Hkv, D):
        raise ValueError("k_new/v_new must be [T][num_kv_heads][head_dim]")
    _i32(cu_new_lens, "cu_new_lens", 1)
    _i32(ctx_lens, "ctx_lens", 1)
    _i32(block_table, "block_table", 2)
    S = ctx_lens.shape[0]
    if cu_new_lens.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("cu_new_lens must have num_seqs+1 entries and block_table num_seqs rows")
    st = lib().pkv_kv_append(k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                            cu_new_lens.data_ptr(), ctx_lens.data_ptr(), block_table.data_ptr(),
                            block_table.shape[1], S, k_new.shape[0], Hkv, D, B, NB, _stream())
    _check(st, "kv_append")


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_seq_len: int,
                           total_kv_tokens: int = 0) -> int:
    n = lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                        total_kv_tokens)
    if n == 0 and num_seqs > 0:
        raise PkvError(2, "decode_workspace_bytes")
    return int(n)


def decode_workspace_reset(workspace) -> None:
    """Zero the chunk counters of a decode workspace (uint8 CUDA tensor) on the
    current stream: needed before the first use of a workspace that was not
    zero-filled, or after a call on it that did not complete."""
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    _check(lib().pkv_decode_workspace_reset(workspace.data_ptr(), workspace.numel(), _stream()),
           "decode_workspace_reset")


def paged_gqa_decode(q, k_pool, v_pool, block_table, seq_lens, scale: float, *, max_seq_len: int,
                     total_kv_tokens: int = 0, out=None, workspace=None):
    """One query row per sequence: ``q [S][Hq][D]`` -> ``out [S][Hq][D]`` bf16.
    ``workspace`` (uint8 CUDA tensor, zero-filled before its first use; every
    call leaves its counters at zero) is allocated zero-filled if not given."""
    NB, Hkv, B, D = _pool_shape(k_pool, v_pool)
    _bf16(q, "q", 3)
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim differs from the pools'")
    _i32(block_table, "block_table", 2)
    _i32(seq_lens, "seq_lens", 1)
    if block_table.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_table and seq_lens need one row per sequence")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q.device)
    _bf16(out, "out", 3)
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [S][Hq][D]")
    need = decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, total_kv_tokens) if S > 0 else 0
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    st = lib().pkv_paged_gqa_decode(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                   block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(), max_seq_len,
                                   total_kv_tokens, S, Hq, Hkv, D, B, NB, float(scale), workspace.data_ptr(),
                                   workspace.numel(), _stream())
    _check(st, "paged_gqa_decode")
    return out


def paged_gqa_decode_append(q, k_new, v_new, k_pool, v_pool, block_table, seq_lens, scale: float, *,
                            max_seq_len: int, total_kv_tokens: int = 0, out=None, workspace=None):
    """One decode step in one launch: append ``k_new/v_new [S][Hkv][D]`` at
    position ``seq_lens[s] - 1`` of each sequence (the pools are written),
    then decode ``q [S][Hq][D]`` over all ``seq_lens[s]`` keys -> ``out``."""
    NB, Hkv, B, D = _pool_shape(k_pool, v_pool)
    _bf16(q, "q", 3)
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim differs from the pools'")
    _bf16(k_new, "k_new", 3)
    _bf16(v_new, "v_new", 3)
    if tuple(k_new.shape) != (S, Hkv, D) or tuple(v_new.shape) != (S, Hkv, D):
        raise ValueError("k_new/v_new must be [S][num_kv_heads][head_dim]")
    _i32(block_table, "block_table", 2)
    _i32(seq_lens, "seq_lens", 1)
    if block_table.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_table and seq_lens need one row per sequence")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q.device)
    _bf16(out, "out", 3)
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [S][Hq][D]")
    need = decode_workspace_bytes(S, Hq, Hkv, D, max_seq_len, total_kv_tokens) if S > 0 else 0
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    st = lib().pkv_paged_gqa_decode_append(out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                          k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                                          block_table.shape[1], seq_lens.data_ptr(), max_seq_len, total_kv_tokens,
                                          S, Hq, Hkv, D, B, NB, float(scale), workspace.data_ptr(),
                                          workspace.numel(), _stream())
    _check(st, "paged_gqa_decode_append")
    return out


# ---- INT8 KV cache (include/pkv_int8.h): codes [NB][Hkv][B][D] int8, one
# fp32 scale per slot [NB][Hkv][B] for K and for V

def _int8_cache(k_codes, v_codes, k_scales, v_scales):
    for t, name in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int8:
            raise TypeError(f"{name} must be an int8 tensor")
        if t.dim() != 4 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous 4-d CUDA tensor")
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
            raise TypeError(f"{name} must be a float32 tensor")
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
    if k_codes.shape != v_codes.shape:
        raise ValueError("k_codes and v_codes must have the same shape")
    NB, Hkv, B, D = k_codes.shape
    if tuple(k_scales.shape) != (NB, Hkv, B) or tuple(v_scales.shape) != (NB, Hkv, B):
        raise ValueError("scales must be [num_blocks][num_kv_heads][block_size]")
    return NB, Hkv, B, D


def empty_int8_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, device="cuda"):
    """Uninitialised INT8 cache tensors (k_codes, v_codes, k_scales, v_scales)."""
    codes = (num_blocks, num_kv_heads, block_size, head_dim)
    return (torch.empty(codes, dtype=torch.int8, device=device), torch.empty(codes, dtype=torch.int8, device=device),
            torch.empty(codes[:3], dtype=torch.float32, device=device),
            torch.empty(codes[:3], dtype=torch.float32, device=device))


def kv_append_int8(k_codes, v_codes, k_scales, v_scales, k_new, v_new, cu_new_lens, ctx_lens, block_table) -> None:
    """Quantise rows ``k_new/v_new [T][Hkv][D]`` (bf16) into the INT8 cache at
    positions ``ctx_lens[s] ..`` of each sequence (see ``pkv_kv_append_int8``)."""
    NB, Hkv, B, D = _int8_cache(k_codes, v_codes, k_scales, v_scales)
    _bf16(k_new, "k_new", 3)
    _bf16(v_new, "v_new", 3)
    if k_new.shape != v_new.shape or tuple(k_new.shape[1:]) != (Hkv, D):
        raise ValueError("k_new/v_new must be [T][num_kv_heads][head_dim]")
    _i32(cu_new_lens, "cu_new_lens", 1)
    _i32(ctx_lens, "ctx_lens", 1)
    _i32(block_table, "block_table", 2)
    S = ctx_lens.shape[0]
    if cu_new_lens.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("cu_new_lens must have num_seqs+1 entries and block_table num_seqs rows")
    st = lib().pkv_kv_append_int8(k_codes.data_ptr(), v_codes.data_ptr(), k_scales.data_ptr(),
                                 v_scales.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), cu_new_lens.data_ptr(),
                                 ctx_lens.data_ptr(), block_table.data_ptr(), block_table.shape[1], S,
                                 k_new.shape[0], Hkv, D, B, NB, _stream())
    _check(st, "kv_append_int8")


def decode_int8_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                max_seq_len: int, total_kv_tokens: int = 0) -> int:
    n = lib().pkv_decode_int8_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                             total_kv_tokens)
    if n == 0 and num_seqs > 0:
        raise PkvError(2, "decode_int8_workspace_bytes")
    return int(n)


def paged_gqa_decode_int8(q, k_codes, v_codes, k_scales, v_scales, block_table, seq_lens, scale: float, *,
                          max_seq_len: int, total_kv_tokens: int = 0, out=None, workspace=None):
    """Decode over the INT8 cache: ``q [S][Hq][D]`` -> ``out [S][Hq][D]`` bf16."""
    NB, Hkv, B, D = _int8_cache(k_codes, v_codes, k_scales, v_scales)
    _bf16(q, "q", 3)
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim differs from the cache's")
    _i32(block_table, "block_table", 2)
    _i32(seq_lens, "seq_lens", 1)
    if block_table.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_table and seq_lens need one row per sequence")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q.device)
    _bf16(out, "out", 3)
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [S][Hq][D]")
    need = decode_int8_workspace_bytes(S, Hq, Hkv, D, max_seq_len, total_kv_tokens) if S > 0 else 0
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    st = lib().pkv_paged_gqa_decode_int8(out.data_ptr(), q.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
                                        k_scales.data_ptr(), v_scales.data_ptr(), block_table.data_ptr(),
                                        block_table.shape[1], seq_lens.data_ptr(), max_seq_len, total_kv_tokens, S,
                                        Hq, Hkv, D, B, NB, float(scale), workspace.data_ptr(), workspace.numel(),
                                        _stream())
    _check(st, "paged_gqa_decode_int8")
    return out


def qkv_project_append(x, w_qkv, k_pool, v_pool, cu_new_lens, ctx_lens, block_table, num_q_heads: int, *,
                       q_out=None):
    """The fused QKV projection (see ``pkv_qkv_project_append``): ``x [T][d_model]``
    times the merged weight ``w_qkv [(Hq + 2 Hkv) D][d_model]``; returns
    ``q_out [T][Hq][D]`` and writes the k / v rows into the pools."""
    NB, Hkv, B, D = _pool_shape(k_pool, v_pool)
    _bf16(x, "x", 2)
    _bf16(w_qkv, "w_qkv", 2)
    T, dm = x.shape
    if tuple(w_qkv.shape) != ((num_q_heads + 2 * Hkv) * D, dm):
        raise ValueError("w_qkv must be [(num_q_heads + 2 num_kv_heads) head_dim][d_model]")
    _i32(cu_new_lens, "cu_new_lens", 1)
    _i32(ctx_lens, "ctx_lens", 1)
    _i32(block_table, "block_table", 2)
    S = ctx_lens.shape[0]
    if cu_new_lens.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("cu_new_lens must have num_seqs+1 entries and block_table num_seqs rows")
    if q_out is None:
        q_out = torch.empty((T, num_q_heads, D), dtype=torch.bfloat16, device=x.device)
    _bf16(q_out, "q_out", 3)
    if tuple(q_out.shape) != (T, num_q_heads, D):
        raise ValueError("q_out must be [T][num_q_heads][head_dim]")
    st = lib().pkv_qkv_project_append(q_out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), x.data_ptr(),
                                     w_qkv.data_ptr(), cu_new_lens.data_ptr(), ctx_lens.data_ptr(),
                                     block_table.data_ptr(), block_table.shape[1], S, T, dm, num_q_heads, Hkv, D, B,
                                     NB, _stream())
    _check(st, "qkv_project_append")
    return q_out


def paged_gqa_decode_append_int8(q, k_new, v_new, k_codes, v_codes, k_scales, v_scales, block_table, seq_lens,
                                 scale: float, *, max_seq_len: int, total_kv_tokens: int = 0, out=None,
                                 workspace=None):
    """One INT8 decode step in one launch: quantise ``k_new/v_new [S][Hkv][D]``
    into position ``seq_lens[s] - 1`` of each sequence, then decode
    ``q [S][Hq][D]`` over the INT8 cache -> ``out``."""
    NB, Hkv, B, D = _int8_cache(k_codes, v_codes, k_scales, v_scales)
    _bf16(q, "q", 3)
    S, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim differs from the cache's")
    _bf16(k_new, "k_new", 3)
    _bf16(v_new, "v_new", 3)
    if tuple(k_new.shape) != (S, Hkv, D) or tuple(v_new.shape) != (S, Hkv, D):
        raise ValueError("k_new/v_new must be [S][num_kv_heads][head_dim]")
    _i32(block_table, "block_table", 2)
    _i32(seq_lens, "seq_lens", 1)
    if block_table.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_table and seq_lens need one row per sequence")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q.device)
    _bf16(out, "out", 3)
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [S][Hq][D]")
    need = decode_int8_workspace_bytes(S, Hq, Hkv, D, max_seq_len, total_kv_tokens) if S > 0 else 0
    if workspace is None:
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    st = lib().pkv_paged_gqa_decode_append_int8(out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                               k_codes.data_ptr(), v_codes.data_ptr(), k_scales.data_ptr(),
                                               v_scales.data_ptr(), block_table.data_ptr(), block_table.shape[1],
                                               seq_lens.data_ptr(), max_seq_len, total_kv_tokens, S, Hq, Hkv, D, B,
                                               NB, float(scale), workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "paged_gqa_decode_append_int8")
    return out


def copy_blocks(k_pool, v_pool, src_ids, dst_ids) -> None:
    """Copy whole blocks src_ids[i] -> dst_ids[i] of both pools (the device
    side of the block manager's copy-on-write)."""
    import numpy as np
    NB, Hkv, B, D = _pool_shape(k_pool, v_pool)
    src = np.ascontiguousarray(src_ids, dtype=np.int32)
    dst = np.ascontiguousarray(dst_ids, dtype=np.int32)
    if src.shape != dst.shape or src.ndim != 1:
        raise ValueError("src_ids and dst_ids must be 1-d and of one length")
    st = lib().pkv_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), src.ctypes.data, dst.ctypes.data, src.size,
                              Hkv, D, B, NB, _stream())
    _check(st, "copy_blocks")


def paged_gqa_prefill(q, cu_q_lens, k_pool, v_pool, block_table, seq_lens, scale: float, *, max_q_len: int,
                      max_seq_len: int, out=None):
    """Causal attention of packed chunk rows ``q [T][Hq][D]`` (see
    ``pkv_paged_gqa_prefill``) -> ``out [T][Hq][D]`` bf16."""
    NB, Hkv, B, D = _pool_shape(k_pool, v_pool)
    _bf16(q, "q", 3)
    T, Hq, Dq = q.shape
    if Dq != D:
        raise ValueError("q head_dim differs from the pools'")
    _i32(cu_q_lens, "cu_q_lens", 1)
    _i32(block_table, "block_table", 2)
    _i32(seq_lens, "seq_lens", 1)
    S = seq_lens.shape[0]
    if cu_q_lens.shape[0] != S + 1 or block_table.shape[0] != S:
        raise ValueError("cu_q_lens must have num_seqs+1 entries and block_table num_seqs rows")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=q.device)
    _bf16(out, "out", 3)
    if tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must be [T][Hq][D]")
    st = lib().pkv_paged_gqa_prefill(out.data_ptr(), q.data_ptr(), cu_q_lens.data_ptr(), T, max_q_len,
                                    k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                                    block_table.shape[1], seq_lens.data_ptr(), max_seq_len, S, Hq, Hkv, D, B, NB,
                                    float(scale), _stream())
    _check(st, "paged_gqa_prefill")
    return out


def read_probe(data: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of ``data`` once on the current stream (see
    ``pkv_read_probe`` in include/pkv_diag.h): the device's plain read rate.
    ``sink`` is a device buffer of at least 16 * READ_PROBE_WORKGROUPS bytes
    whose contents are unspecified afterwards."""
    if not (data.is_cuda and sink.is_cuda and data.is_contiguous() and sink.is_contiguous()):
        raise ValueError("data and sink must be contiguous device tensors")
    st = lib().pkv_read_probe(data.data_ptr(), data.numel() * data.element_size(), sink.data_ptr(),
                              sink.numel() * sink.element_size(), _stream())
    _check(st, "read_probe")


def mfma_probe_flops(iters: int) -> int:
    """Flops of one pkv_mfma_probe launch of ``iters`` rounds."""
    return MFMA_PROBE_WORKGROUPS * 4 * 8 * iters * 2 * 32 * 32 * 16


def mfma_probe(iters: int, sink: torch.Tensor) -> None:
    """Run the bf16 MFMA stream of ``pkv_mfma_probe`` (include/pkv_diag.h)
    on the current stream: ``mfma_probe_flops(iters)`` flop, no memory reads.
    ``sink`` is a device buffer of at least 4 * 256 * MFMA_PROBE_WORKGROUPS
    bytes whose contents are unspecified afterwards."""
    if not (sink.is_cuda and sink.is_contiguous()):
        raise ValueError("sink must be a contiguous device tensor")
    st = lib().pkv_mfma_probe(int(iters), sink.data_ptr(), sink.numel() * sink.element_size(), _stream())
    _check(st, "mfma_probe")

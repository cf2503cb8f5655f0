"""The C-ABI library on the host (no GPU): it loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_gqa_scatter_amd as pkv
from paged_kv_gqa_scatter_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")
BLOCKS_HEADER = os.path.join(ROOT, "include", "pkv_blocks.h")
INT8_HEADER = os.path.join(ROOT, "include", "pkv_int8.h")
QKV_HEADER = os.path.join(ROOT, "include", "pkv_qkv.h")
DIAG_HEADER = os.path.join(ROOT, "include", "pkv_diag.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_gqa_scatter_amd import build
        build.build()
    return pkv.lib()


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(pkv_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("pkv_kv_append", "pkv_paged_gqa_decode", "pkv_paged_gqa_prefill"):
        assert n in names
    assert set(names) == set(pkv.EXPORTS)


def test_block_header_declares_its_functions():
    assert set(declared_functions(BLOCKS_HEADER)) == set(pkv.BLOCK_EXPORTS)


def test_int8_header_declares_its_functions():
    assert set(declared_functions(INT8_HEADER)) == set(pkv.INT8_EXPORTS)


def test_qkv_header_declares_its_functions():
    assert set(declared_functions(QKV_HEADER)) == set(pkv.QKV_EXPORTS)


def test_diag_header_declares_its_functions():
    assert set(declared_functions(DIAG_HEADER)) == set(pkv.DIAG_EXPORTS)
    text = open(DIAG_HEADER).read()
    assert f"#define PKV_READ_PROBE_WORKGROUPS {pkv.READ_PROBE_WORKGROUPS}" in text
    assert f"#define PKV_MFMA_PROBE_WORKGROUPS {pkv.MFMA_PROBE_WORKGROUPS}" in text
    assert "#define PKV_MFMA_PROBE_MAX_ITERS (1 << 20)" in text and pkv.MFMA_PROBE_MAX_ITERS == 1 << 20


def test_mfma_probe_rejects(lib):
    sink_bytes = 4 * 256 * pkv.MFMA_PROBE_WORKGROUPS
    assert lib.pkv_mfma_probe(16, None, sink_bytes, None) == 1
    assert lib.pkv_mfma_probe(16, A16 + 2, sink_bytes, None) == 3
    assert lib.pkv_mfma_probe(0, A16, sink_bytes, None) == 2
    assert lib.pkv_mfma_probe(-5, A16, sink_bytes, None) == 2
    assert lib.pkv_mfma_probe(pkv.MFMA_PROBE_MAX_ITERS + 1, A16, sink_bytes, None) == 2
    assert lib.pkv_mfma_probe(16, A16, sink_bytes - 4, None) == 4
    assert pkv.mfma_probe_flops(1) == pkv.MFMA_PROBE_WORKGROUPS * 4 * 8 * 32768


def test_read_probe_rejects(lib):
    sink_bytes = 16 * pkv.READ_PROBE_WORKGROUPS
    assert lib.pkv_read_probe(None, 1 << 20, A16, sink_bytes, None) == 1
    assert lib.pkv_read_probe(A16, 1 << 20, None, sink_bytes, None) == 1
    assert lib.pkv_read_probe(A16 + 8, 1 << 20, A16, sink_bytes, None) == 3
    assert lib.pkv_read_probe(A16, 1 << 20, A16 + 4, sink_bytes, None) == 3
    assert lib.pkv_read_probe(A16, 0, A16, sink_bytes, None) == 2
    assert lib.pkv_read_probe(A16, (1 << 20) + 8, A16, sink_bytes, None) == 2
    assert lib.pkv_read_probe(A16, 1 << 20, A16, sink_bytes - 16, None) == 4


def test_every_declared_symbol_is_exported(lib):
    for header in (HEADER, BLOCKS_HEADER, INT8_HEADER, QKV_HEADER, DIAG_HEADER):
        for name in declared_functions(header):
            assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.pkv_abi_version() == 1
    for code in range(9):
        assert lib.pkv_status_string(code)
    assert lib.pkv_status_string(99) == b"unknown status"


A16 = 1 << 12  # any 16-byte aligned non-null address: these calls must be rejected before touching it


def append_args(**kw):
    a = dict(k_pool=A16, v_pool=A16, k_new=A16, v_new=A16, cu=A16, ctx=A16, table=A16, mbs=4, S=2, T=3, hkv=8,
             d=128, bs=256, nb=10, stream=None)
    a.update(kw)
    return (a["k_pool"], a["v_pool"], a["k_new"], a["v_new"], a["cu"], a["ctx"], a["table"], a["mbs"], a["S"],
            a["T"], a["hkv"], a["d"], a["bs"], a["nb"], a["stream"])


def test_append_rejects(lib):
    f = lib.pkv_kv_append
    assert f(*append_args(d=96)) == 2
    assert f(*append_args(bs=48)) == 2
    assert f(*append_args(bs=512)) == 2
    assert f(*append_args(bs=8)) == 2
    assert f(*append_args(S=0)) == 2
    assert f(*append_args(T=-1)) == 2
    assert f(*append_args(k_new=None)) == 1
    assert f(*append_args(table=None)) == 1
    assert f(*append_args(v_pool=A16 + 2)) == 3
    assert f(*append_args(T=0, k_new=None)) == 0  # nothing to do, nothing touched


def decode_args(**kw):
    a = dict(out=A16, q=A16, kp=A16, vp=A16, table=A16, mbs=9, lens=A16, maxlen=2049, total=0, S=8, hq=32, hkv=8,
             d=128, bs=256, nb=50, scale=0.088, ws=A16, wsb=1 << 30, stream=None)
    a.update(kw)
    return tuple(a[k] for k in ("out", "q", "kp", "vp", "table", "mbs", "lens", "maxlen", "total", "S", "hq", "hkv",
                                "d", "bs", "nb", "scale", "ws", "wsb", "stream"))


def test_decode_rejects(lib):
    f = lib.pkv_paged_gqa_decode
    assert f(*decode_args(hq=30)) == 2          # Hq % Hkv
    assert f(*decode_args(hq=128, hkv=8)) == 2  # group of 16 unsupported
    assert f(*decode_args(d=256)) == 2
    assert f(*decode_args(maxlen=9 * 256 + 1)) == 2  # longer than the table can hold
    assert f(*decode_args(S=9000)) == 2
    assert f(*decode_args(q=None)) == 1
    assert f(*decode_args(out=A16 + 8)) == 3
    assert f(*decode_args(ws=None)) == 4
    assert f(*decode_args(wsb=16)) == 4
    assert f(*decode_args(S=0)) == 0


def test_decode_workspace_bytes(lib):
    f = lib.pkv_decode_workspace_bytes
    assert f(8, 32, 8, 96, 2049, 0) == 0
    # the size depends on the split plan, which depends on the token bound
    assert f(8, 32, 8, 128, 2049, 10248) > 0
    assert f(8, 32, 8, 128, 2049, 0) > 0
    assert f(272, 32, 8, 128, 32769, 1_830_000) < f(272, 32, 8, 128, 32769, 0)
    # every workspace starts with the 16 KiB of chunk counters, whatever the shape
    assert all(f(S, 4, 1, 64, L, 0) > 16384 for S in (1, 8) for L in (1, 300))


def test_decode_workspace_reset_rejects(lib):
    # the reset validates on the host and launches nothing when it rejects
    f = lib.pkv_decode_workspace_reset
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, 1 << 20, None) == 1
    assert f(A16 + 4, 1 << 20, None) == 3
    assert f(A16, 16383, None) == 4
    assert f(A16, 0, None) == 4


def decode_append_args(**kw):
    a = dict(out=A16, q=A16, kn=A16, vn=A16, kp=A16, vp=A16, table=A16, mbs=9, lens=A16, maxlen=2049, total=0, S=8,
             hq=32, hkv=8, d=128, bs=256, nb=90, scale=0.088, ws=A16, wsb=1 << 30, stream=None)
    a.update(kw)
    return tuple(a[k] for k in ("out", "q", "kn", "vn", "kp", "vp", "table", "mbs", "lens", "maxlen", "total", "S",
                                "hq", "hkv", "d", "bs", "nb", "scale", "ws", "wsb", "stream"))


def test_decode_append_rejects(lib):
    f = lib.pkv_paged_gqa_decode_append
    assert f(*decode_append_args(hq=30)) == 2
    assert f(*decode_append_args(maxlen=9 * 256 + 1)) == 2
    assert f(*decode_append_args(kn=None)) == 1
    assert f(*decode_append_args(vn=None)) == 1
    assert f(*decode_append_args(q=None)) == 1
    assert f(*decode_append_args(kn=A16 + 2)) == 3
    assert f(*decode_append_args(ws=None)) == 4
    assert f(*decode_append_args(S=0)) == 0


def prefill_args(**kw):
    a = dict(out=A16, q=A16, cu=A16, T=1000, maxq=512, kp=A16, vp=A16, table=A16, mbs=8, lens=A16, maxlen=1536,
             S=2, hq=32, hkv=8, d=128, bs=256, nb=20, scale=0.088, stream=None)
    a.update(kw)
    return tuple(a[k] for k in ("out", "q", "cu", "T", "maxq", "kp", "vp", "table", "mbs", "lens", "maxlen", "S", "hq",
                                "hkv", "d", "bs", "nb", "scale", "stream"))


def test_prefill_rejects(lib):
    f = lib.pkv_paged_gqa_prefill
    assert f(*prefill_args(maxq=2000)) == 2        # chunk longer than the sequence bound
    assert f(*prefill_args(T=2000)) == 2           # more rows than num_seqs * max_q_len
    assert f(*prefill_args(mbs=2)) == 2            # table too short for max_seq_len
    assert f(*prefill_args(hkv=3)) == 2
    assert f(*prefill_args(cu=None)) == 1
    assert f(*prefill_args(q=A16 + 4)) == 3
    assert f(*prefill_args(T=0)) == 0


def append_int8_args(**kw):
    a = dict(kc=A16, vc=A16, ks=A16, vs=A16, k_new=A16, v_new=A16, cu=A16, ctx=A16, table=A16, mbs=4, S=2, T=3,
             hkv=8, d=128, bs=256, nb=10, stream=None)
    a.update(kw)
    return tuple(a[k] for k in ("kc", "vc", "ks", "vs", "k_new", "v_new", "cu", "ctx", "table", "mbs", "S", "T",
                                "hkv", "d", "bs", "nb", "stream"))


def test_append_int8_rejects(lib):
    f = lib.pkv_kv_append_int8
    assert f(*append_int8_args(d=96)) == 2
    assert f(*append_int8_args(bs=16)) == 2     # INT8 tiles are 32 keys of one block
    assert f(*append_int8_args(bs=48)) == 2
    assert f(*append_int8_args(S=0)) == 2
    assert f(*append_int8_args(ks=None)) == 1
    assert f(*append_int8_args(v_new=None)) == 1
    assert f(*append_int8_args(vs=A16 + 4)) == 3
    assert f(*append_int8_args(kc=A16 + 8)) == 3
    assert f(*append_int8_args(T=0, kc=None)) == 0


def decode_int8_args(**kw):
    a = dict(out=A16, q=A16, kc=A16, vc=A16, ks=A16, vs=A16, table=A16, mbs=9, lens=A16, maxlen=2049, total=0, S=8,
             hq=32, hkv=8, d=128, bs=256, nb=50, scale=0.088, ws=A16, wsb=1 << 30, stream=None)
    a.update(kw)
    return tuple(a[k] for k in ("out", "q", "kc", "vc", "ks", "vs", "table", "mbs", "lens", "maxlen", "total", "S",
                                "hq", "hkv", "d", "bs", "nb", "scale", "ws", "wsb", "stream"))


def test_decode_int8_rejects(lib):
    f = lib.pkv_paged_gqa_decode_int8
    assert f(*decode_int8_args(hq=30)) == 2
    assert f(*decode_int8_args(bs=16, mbs=200)) == 2
    assert f(*decode_int8_args(d=256)) == 2
    assert f(*decode_int8_args(maxlen=9 * 256 + 1)) == 2
    assert f(*decode_int8_args(kc=None)) == 1
    assert f(*decode_int8_args(vs=None)) == 1
    assert f(*decode_int8_args(ks=A16 + 4)) == 3
    assert f(*decode_int8_args(ws=None)) == 4
    assert f(*decode_int8_args(wsb=16)) == 4
    assert f(*decode_int8_args(S=0)) == 0


def test_decode_int8_workspace_bytes(lib):
    f = lib.pkv_decode_int8_workspace_bytes
    assert f(8, 32, 8, 96, 2049, 0) == 0
    assert f(8, 32, 8, 128, 2049, 0) > 0
    assert f(272, 32, 8, 128, 32769, 1_830_000) < f(272, 32, 8, 128, 32769, 0)
    assert f(1, 4, 1, 64, 1, 0) > 16384  # the chunk counters come first here too


def qkv_args(**kw):
    a = dict(q=A16, kp=A16, vp=A16, x=A16, w=A16, cu=A16, ctx=A16, table=A16, mbs=4, S=2, T=3, dm=4096, hq=32,
             hkv=8, d=128, bs=256, nb=10, stream=None)
    a.update(kw)
    return tuple(a[k] for k in ("q", "kp", "vp", "x", "w", "cu", "ctx", "table", "mbs", "S", "T", "dm", "hq", "hkv",
                                "d", "bs", "nb", "stream"))


def test_qkv_project_append_rejects(lib):
    f = lib.pkv_qkv_project_append
    assert f(*qkv_args(dm=4000)) == 2          # d_model not a multiple of 64
    assert f(*qkv_args(hq=30)) == 2
    assert f(*qkv_args(d=96)) == 2
    assert f(*qkv_args(bs=48)) == 2
    assert f(*qkv_args(T=300000)) == 2         # T * d_model past 2^30
    assert f(*qkv_args(S=0)) == 2
    assert f(*qkv_args(w=None)) == 1
    assert f(*qkv_args(q=None)) == 1
    assert f(*qkv_args(x=A16 + 2)) == 3
    assert f(*qkv_args(T=0, x=None)) == 0


def test_decode_append_int8_rejects(lib):
    f = lib.pkv_paged_gqa_decode_append_int8
    base = dict(out=A16, q=A16, kn=A16, vn=A16, kc=A16, vc=A16, ks=A16, vs=A16, table=A16, mbs=9, lens=A16,
                maxlen=2049, total=0, S=8, hq=32, hkv=8, d=128, bs=256, nb=50, scale=0.088, ws=A16, wsb=1 << 30,
                stream=None)
    keys = ("out", "q", "kn", "vn", "kc", "vc", "ks", "vs", "table", "mbs", "lens", "maxlen", "total", "S", "hq",
            "hkv", "d", "bs", "nb", "scale", "ws", "wsb", "stream")
    args = lambda **kw: tuple({**base, **kw}[k] for k in keys)
    assert f(*args(bs=16, mbs=200)) == 2
    assert f(*args(hq=30)) == 2
    assert f(*args(kn=None)) == 1
    assert f(*args(vs=None)) == 1
    assert f(*args(vn=A16 + 2)) == 3
    assert f(*args(ws=None)) == 4
    assert f(*args(S=0)) == 0


def test_decode_append_static_rejects(lib):
    # the static-scratch step validates on the host and launches nothing when
    # it rejects; a plan beyond the 32 MiB scratch gets its own status
    f = lib.pkv_paged_gqa_decode_append_static
    f.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64] + \
        [ctypes.c_int32] * 6 + [ctypes.c_float, ctypes.c_void_p]
    ok = lambda **kw: dict(dict(out=A16, q=A16, kn=A16, vn=A16, kp=A16, vp=A16, table=A16, mbs=9, lens=A16,
                                maxlen=2049, total=0, S=8, hq=32, hkv=8, d=128, bs=256, nb=90, scale=0.088,
                                stream=None), **kw)
    args = lambda a: tuple(a[k] for k in ("out", "q", "kn", "vn", "kp", "vp", "table", "mbs", "lens", "maxlen",
                                          "total", "S", "hq", "hkv", "d", "bs", "nb", "scale", "stream"))
    assert f(*args(ok(hq=30))) == 2
    assert f(*args(ok(q=None))) == 1
    assert f(*args(ok(kn=None))) == 1
    assert f(*args(ok(vn=A16 + 2))) == 3
    assert f(*args(ok(S=0))) == 0
    big = ok(S=8192, mbs=256, maxlen=65536, nb=100000)
    assert lib.pkv_decode_workspace_bytes(8192, 32, 8, 128, 65536, 0) > 32 << 20
    assert f(*args(big)) == 8
    assert lib.pkv_status_string(8) == b"the call needs more decode scratch than the library's static 32 MiB"



def test_run_cli_arguments():
    # the workload runner's command line (python -m paged_kv_gqa_scatter_amd.run):
    # argument checks and the named cases, without a GPU
    from paged_kv_gqa_scatter_amd import run
    a = run.parse_args(["--config", "3", "--seed", "7", "--repeat", "2"])
    assert (a.config, a.seed, a.repeat, a.int8) == (3, 7, 2, False)
    for bad in (["--config", "9"], ["--config", "2", "--repeat", "0"], ["--config", "3", "--int8"], []):
        with pytest.raises(SystemExit):
            run.parse_args(bad)
    assert run.parse_args(["--config", "5", "--int8"]).int8
    assert run.build_case(4).name == W.config4_mixed().name
    c = run.build_case(3, 7)
    assert c.name == W.config3_prefill(seed=7, draw_values=False).name
    assert np.array_equal(c.steps[0].prefill.cu_q_lens, W.config3_prefill(seed=7, draw_values=False).steps[0].prefill.cu_q_lens)

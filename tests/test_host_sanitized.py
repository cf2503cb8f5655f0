"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (gcc/g++,
in child processes): the oracle's C runs every pin, and the block manager's
C++ (built alone) runs its own test file; an out-of-bounds access, a use
after free or undefined arithmetic aborts the child and fails the test.
GPU code is not built with sanitizers.  Skipped where gcc's sanitizer
runtimes are missing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
import oracle_pins as P
orc = oracle.Oracle({lib!r})
for pin in P.ALL_PINS:
    pin(orc)
print("sanitized pins ok", len(P.ALL_PINS))
"""


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-o", lib, os.path.join(ROOT, "oracle", "pkv_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=580)
    assert r.returncode == 0 and "sanitized pins ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])


@pytest.mark.timeout(600)
def test_sanitized_run_catches_a_planted_overflow(tmp_path):
    # the same run over a copy of the oracle with one byte written past a
    # heap block (kv_append's slot flags) must abort with ASan's report, so
    # that the test above would see such a mistake
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    src = open(os.path.join(ROOT, "oracle", "pkv_oracle.c")).read()
    line = "    if (!written) return ORACLE_ERR_OOM;\n"
    assert line in src
    bad = tmp_path / "bad_oracle.c"
    bad.write_text(src.replace(line, line + "    written[nslots ? nslots : 1] = 1;\n", 1))
    lib = str(tmp_path / "liboracle_bad.so")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-o", lib, str(bad), "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", OMP_NUM_THREADS="4")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=580)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.returncode, r.stderr[-2000:])


BM_CHILD = r"""
import ctypes, os, sys
sys.path[:0] = [{root!r}, {tests!r}]
import paged_kv_gqa_scatter_amd as pkv
real = pkv.lib()
san = ctypes.CDLL({lib!r})
names = [n for n in pkv.BLOCK_EXPORTS if n.startswith("pkv_bm_")]
for n in names:
    f, g = getattr(san, n), getattr(real, n)
    f.argtypes, f.restype = g.argtypes, g.restype


class Shim:
    # the block manager's entry points from the sanitized build, the rest from libpkv.so
    def __getattr__(self, n):
        return getattr(san if n in names else real, n)


pkv._lib = Shim()
import pytest
sys.exit(pytest.main([os.path.join({tests!r}, "test_block_manager.py"), "-q", "-p", "no:cacheprovider",
                      "-m", "not gpu"]))
"""


@pytest.mark.timeout(600)
def test_block_manager_tests_under_asan_and_ubsan(tmp_path):
    # the host block manager (csrc/block_manager.cpp, plain C++) built alone
    # with the sanitizers, under its own test file
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    if not os.path.exists(os.path.join(ROOT, "paged_kv_gqa_scatter_amd", "libpkv.so")):
        pytest.skip("libpkv.so not built")
    lib = str(tmp_path / "libbm_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "paged_kv_gqa_scatter_amd", "csrc", "block_manager.cpp"), "-o", lib], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = BM_CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=580)
    assert r.returncode == 0 and "passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])

"""The oracle's C built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, on the host) runs every pin in a child process: an out-of-bounds access,
a use after free or undefined arithmetic in the oracle aborts the child and
fails this test.  Skipped where gcc's sanitizer runtimes are missing."""
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

"""The oracle's pins once more with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, on the CPU): its allocations, frees, indexing and
OpenMP loops must run clean on every pin's inputs.  A planted out-of-bounds write in a
copy of the source shows that the harness reports what it is meant to."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_format.py", "tests/test_oracle_linear.py", "tests/test_oracle_route_sort.py",
        "tests/test_oracle_moe.py", "tests/test_oracle_a8.py"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    return p


def _run_pins(src_path, tmp_path, pins):
    so = tmp_path / "liboracle_san.so"
    flags = [f for f in oracle.CFLAGS if f != "-O2"] + ["-O1"] + SANITIZE
    subprocess.run(["gcc", *flags, str(src_path), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=_libasan(), MXMOE_ORACLE_LIB=str(so), OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report goes to fd 2 and ends the process; captured output would be lost
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", *pins],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    r = _run_pins(oracle._SRC, tmp_path, PINS)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert r.returncode == 0 and " passed" in r.stdout, out


def test_the_harness_reports_a_planted_out_of_bounds_write(tmp_path):
    src = open(oracle._SRC).read()
    old = "for (int64_t e = na; e < E; ++e) active[e] = -1;"
    assert src.count(old) == 1
    bad = tmp_path / "mx_oracle_oob.c"
    bad.write_text(src.replace(old, "for (int64_t e = na; e <= E; ++e) active[e] = -1;"))
    r = _run_pins(bad, tmp_path, ["tests/test_oracle_route_sort.py"])
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]

"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; gcc): an instrumented copy of attn_oracle.c runs every
oracle pin in a child process, so an out-of-bounds access, a use after free,
a signed overflow or a misaligned load anywhere on the pinned paths stops
the run.  Leak checking is off: the Python interpreter itself does not free
everything at exit."""
import os
import subprocess
import sys
import textwrap
from pathlib import Path

import pytest

import oracle

ROOT = Path(__file__).resolve().parent.parent


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _run_pins(tmp_path, src=None):
    libasan = _runtime("libasan.so")
    if libasan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build(src=src, out=tmp_path / "liboracle_asan.so", extra_flags=SAN_FLAGS)
    runner = tmp_path / "run_pins.py"
    runner.write_text(textwrap.dedent("""
        import sys
        sys.path[:0] = [%r, %r]
        import oracle, oracle_pins
        oracle._lib = oracle.load(%r)
        for check in oracle_pins.ALL_CHECKS:
            check()
            print("ok", check.__name__, flush=True)
        print("all", len(oracle_pins.ALL_CHECKS), flush=True)
    """ % (str(ROOT), str(ROOT / "tests"), str(lib))))
    env = dict(os.environ)
    env["LD_PRELOAD"] = libasan
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:detect_odr_violation=0:alloc_dealloc_mismatch=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return subprocess.run([sys.executable, str(runner)], env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_under_asan_ubsan(tmp_path):
    res = _run_pins(tmp_path)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "all %d" % len(__import__("oracle_pins").ALL_CHECKS) in res.stdout, tail
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail


def test_sanitizer_build_catches_a_planted_overflow(tmp_path):
    """Negative control: a copy of the oracle whose per-head key-limit buffer
    is one element short must stop with an AddressSanitizer report."""
    src = oracle._SRC.read_text()
    anchor = "int64_t* lim = malloc(sizeof(int64_t) * Nq);"
    assert src.count(anchor) == 1
    bad = tmp_path / "attn_oracle_short.c"
    bad.write_text(src.replace(anchor, "int64_t* lim = malloc(sizeof(int64_t) * (Nq - 1));"))
    res = _run_pins(tmp_path, src=bad)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr, (res.stdout + res.stderr)[-3000:]

"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): a copy of libattn_gfx950.so whose host side is instrumented
(device code unchanged) runs the host-side ABI tests (tests/test_abi_cpu.py:
argument validation, launch options, the paged split planner, workspace
sizes, status strings) in a child process, so an out-of-bounds access, a use
after free, a signed overflow or an invalid enum value on those paths stops
the run.  Leak checking is off: the Python interpreter and the HIP runtime do
not free everything at exit.  A negative control plants a stack overflow in
the planner's entry point and must be caught."""
import os
import shutil
import subprocess
import sys
import textwrap
from pathlib import Path

import pytest

from tiled_online_softmax_attention_amd import _build

ROOT = Path(__file__).resolve().parent.parent

# each sanitizer flag applies to host code only
HOST_SAN = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def _asan_runtime():
    """The AddressSanitizer runtime of the compiler that builds the library."""
    res = subprocess.run([_build.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    for cand in sorted(Path("/opt/rocm/lib/llvm/lib/clang").glob("*/lib/linux/libclang_rt.asan-x86_64.so")):
        return str(cand)
    return None


def _build_lib(csrc: Path, out: Path):
    cmd = [_build.HIPCC, *_build.FLAGS, *HOST_SAN, "-I", str(csrc), "-I", str(ROOT / "include"),
           *[str(csrc / s) for s in _build.SOURCES], "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, (res.stdout + res.stderr)[-3000:]
    return out


def _run_abi_tests(tmp_path, lib: Path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime for the library's compiler")
    runner = tmp_path / "run_abi.py"
    runner.write_text(textwrap.dedent("""
        import sys
        from pathlib import Path
        sys.path[:0] = [%r, %r]
        import tiled_online_softmax_attention_amd as attn
        attn.LIB_PATH = Path(%r)
        import pytest
        rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", %r])
        print("pytest exit", int(rc), flush=True)
        sys.exit(int(rc))
    """ % (str(ROOT), str(ROOT / "tests"), str(lib), str(ROOT / "tests" / "test_abi_cpu.py"))))
    logs = tmp_path / "san"
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = ("detect_leaks=0:halt_on_error=1:detect_odr_violation=0:alloc_dealloc_mismatch=0:"
                           "log_path=%s" % logs)
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:log_path=%s" % logs
    res = subprocess.run([sys.executable, str(runner)], env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(p.read_text(errors="replace") for p in tmp_path.glob("san*"))
    return res, reports


def test_host_library_under_asan_ubsan(tmp_path):
    lib = _build_lib(ROOT / "tiled_online_softmax_attention_amd" / "csrc", tmp_path / "libattn_san.so")
    res, reports = _run_abi_tests(tmp_path, lib)
    tail = (res.stdout + res.stderr)[-3000:] + reports[:3000]
    assert res.returncode == 0 and "pytest exit 0" in res.stdout, tail
    assert "ERROR: AddressSanitizer" not in reports and "runtime error" not in reports, tail


def test_host_sanitizer_build_catches_a_planted_overflow(tmp_path):
    """Negative control: a copy of the host code whose workspace query writes
    past a small stack array for num_seqs >= 4 (the ABI tests ask for
    64-request plans) must stop with a sanitizer report naming that file."""
    csrc = tmp_path / "csrc"
    shutil.copytree(ROOT / "tiled_online_softmax_attention_amd" / "csrc", csrc)
    api = csrc / "attn_api.hip"
    src = api.read_text()
    anchor = "    attn_launch_opts_t op;\n    if (read_opts(opts, &op) != ATTN_OK) return 0;\n"
    assert src.count(anchor) == 1
    api.write_text(src.replace(anchor, anchor + "    volatile int planted[4];\n    planted[num_seqs & 7] = 1;\n"))
    lib = _build_lib(csrc, tmp_path / "libattn_planted.so")
    res, reports = _run_abi_tests(tmp_path, lib)
    assert res.returncode != 0, res.stdout[-2000:]
    # UBSan's bounds check sees the constant-size array first; ASan would
    # report the same write as a stack-buffer overflow
    found = reports + res.stderr
    assert ("AddressSanitizer" in found or "runtime error: index 4 out of bounds" in found) and \
        "attn_api.hip" in found, (res.stdout + res.stderr)[-3000:] + found[:3000]

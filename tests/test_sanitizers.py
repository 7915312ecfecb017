"""Host sanitizers on the HIP-free validation unit (csrc/fa_check.c).

fa_check.c and a small driver (tests/sanitize/fa_check_harness.c) are built
with gcc under AddressSanitizer and UndefinedBehaviorSanitizer (every finding
fatal), and every argument table of test_boundary.py is run through it: the
status codes must equal the ones the library returns, and the sanitizers must
report nothing (signed overflow in the size checks, out-of-bounds reads,
misaligned accesses...).  CPU only."""

import os
import shutil
import struct
import subprocess

import pytest

import io_aware_tiled_fa_amd as fa
import test_boundary as tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "io_aware_tiled_fa_amd", "csrc", "fa_check.c")
HARNESS = os.path.join(ROOT, "tests", "sanitize", "fa_check_harness.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _hexf(x: float) -> str:
    """The fp32 value the library receives, as an exact C99 hex float."""
    return float(struct.unpack("<f", struct.pack("<f", x))[0]).hex() if x == x else "nan"


def _fmt(v) -> str:
    if isinstance(v, float):
        return _hexf(v)
    return str(int(v))


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("san") / "fa_check_harness")
    cmd = [cc, "-O1", "-g", "-std=c11", *SAN, f"-I{os.path.join(ROOT, 'include')}", SRC, HARNESS,
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip(f"sanitizer runtime unavailable: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr
    return exe


def _rows():
    rows = []
    for kw, code in tb.FWD_CHECK_CASES:
        args = tb.fwd_args(kw)
        rows.append(("F", args, code, fa.fa_check_args(*args)))
    for kw, code in tb.BWD_CHECK_CASES:
        args = tb.bwd_args(kw)
        rows.append(("B", args, code, fa.fa_bwd_check_args(*args)))
    for kw, code in tb.SPLIT_CHECK_CASES:
        args = tb.split_args(kw)
        rows.append(("S", args, code, fa.fa_splitkv_check_args(*args)))
    return rows


def test_every_boundary_table_under_asan_and_ubsan(harness):
    rows = _rows()
    text = "".join(kind + " " + " ".join(_fmt(a) for a in args) + "\n" for kind, args, _, _ in rows)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)  # the sanitized binary must be the only allocator
    r = subprocess.run([harness], input=text, capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    got = [int(line.split()[0]) for line in r.stdout.splitlines()]
    assert len(got) == len(rows)
    for (kind, args, code, lib_code), st in zip(rows, got):
        assert st == code == lib_code, (kind, args, st, code, lib_code)

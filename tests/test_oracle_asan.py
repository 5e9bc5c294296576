"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/pa_oracle.c is built with -fsanitize=address,undefined (gcc, host code
only) and oracle_pins.py runs every pin against that build in a child process
whose first loaded library is the ASan runtime.  The committed oracle must
exit cleanly.  A control copy with one heap buffer allocated an element short
must abort with an ASan report, which shows that the sanitizer is live in the
child process (a clean run is not just a run without instrumentation).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")
PINS = os.path.join(ROOT, "tests", "oracle_pins.py")


def _run_pins(lib):
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    env = {**os.environ, "LD_PRELOAD": obuild.sanitizer_preload(),
           "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
           "OMP_NUM_THREADS": "4"}
    return subprocess.run([sys.executable, PINS, "--lib", lib], capture_output=True, text=True,
                          timeout=600, env=env)


@pytest.fixture(scope="module")
def asan_ok():
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    if not os.path.exists(obuild.sanitizer_preload()):
        pytest.skip("gcc's libasan runtime is not installed")


def test_oracle_clean_under_asan_ubsan(asan_ok, tmp_path):
    from oracle import build as obuild
    lib = obuild.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    r = _run_pins(lib)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert "pins passed" in r.stdout, report


def test_asan_catches_a_short_buffer(asan_ok, tmp_path):
    """Control: the decode's query buffer one element short is a heap
    overflow the sanitized child must report."""
    from oracle import build as obuild
    text = open(SRC).read()
    old = "double *qbuf = malloc(sizeof(double) * (size_t)head_dim);"
    assert old in text
    src = tmp_path / "short_qbuf.c"
    src.write_text(text.replace(old, "double *qbuf = malloc(sizeof(double) * (size_t)(head_dim - 1));", 1))
    lib = obuild.build_sanitized(str(tmp_path / "liboracle_short.so"), src=str(src))
    r = _run_pins(lib)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stderr[-2000:]

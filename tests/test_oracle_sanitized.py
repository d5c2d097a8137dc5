"""The oracle's CPU tests, run again on a build of the oracle instrumented
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc), in a child
process with the ASan runtime preloaded: any out-of-bounds access, use after
free or undefined behaviour in wi_oracle.c aborts the child and fails this
test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(900)
def test_oracle_suite_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ)
    env.update(WIO_SANITIZE="1", LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = ["tests/test_oracle_pins.py", "tests/test_oracle_stream.py",
             "tests/test_oracle_props.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert os.path.exists(os.path.join(ROOT, "oracle", "libwi_oracle_san.so"))

"""The oracle's C core under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the core is rebuilt with both sanitizers, any finding aborting,
and the oracle's pins run against that build in a child process that
preloads the sanitizer runtime.  Out-of-bounds reads or writes, use of freed
memory and undefined integer or shift behaviour in the core fail the pins."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_ce.py", "tests/test_oracle_linear.py", "tests/test_oracle_shard.py",
        "tests/test_oracle_shift.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "libce_ref_san.so"))
    env = dict(os.environ)
    env.update(VCE_ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               # the interpreter and its libraries leak by design; bounds and
               # use-after-free checks stay on
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail

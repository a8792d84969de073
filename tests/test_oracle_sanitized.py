"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c is built with -fsanitize=address,undefined (recovery off) and the pin
tests run against that build in a child interpreter with the ASan runtime
preloaded.  A second build with one planted out-of-bounds read must be stopped
by ASan, which shows that the sanitizer is live in that process and not silently
absent."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC"]


def _asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(so, tmp_path, *select):
    env = dict(os.environ, ORACLE_LIB=str(so), LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report ends the process at once, and pytest's own capture
    # of stderr would be lost with it
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py"), *select],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def need_asan():
    if _asan_runtime() is None:
        pytest.skip("gcc's ASan runtime is not installed")


def test_pins_pass_under_asan_and_ubsan(tmp_path, need_asan):
    so = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *SAN, SRC, "-o", str(so), "-lm"])
    r = _run_pins(so, tmp_path)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]


def test_planted_overflow_is_caught(tmp_path, need_asan):
    src = open(SRC).read()
    old = "for (int64_t j = 0; j < nb; j++)\n        if (b[j] <= x) k++;"
    assert src.count(old) == 1
    mut = tmp_path / "oracle_oob.c"
    mut.write_text(src.replace(old, "for (int64_t j = 0; j <= nb; j++)\n        if (b[j] <= x) k++;"))
    so = tmp_path / "liboracle_oob.so"
    subprocess.check_call(["gcc", *SAN, str(mut), "-o", str(so), "-lm"])
    r = _run_pins(so, tmp_path, "-k", "bucketize")
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stdout + r.stderr

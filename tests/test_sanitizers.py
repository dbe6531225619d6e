"""The CPU oracle and its C pins under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; gcc).

- ``tests/c/oracle_sanitize.c`` drives every exported oracle function on
  small and edge-case shapes (one leaf, ragged and strided operands,
  28- and 11-leaf groups, every valid shard count, rejected shapes) with the
  oracle compiled into the same executable;
- ``tests/c/pins.c`` runs its four modes on a sampled subset of the fp32 /
  bf16 patterns against a sanitized build of the oracle library.

Any invalid access, leak, signed overflow or other undefined behaviour
aborts the run (``-fno-sanitize-recover=all``).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
NUM = ["-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def _gcc(args):
    os.makedirs(OUT, exist_ok=True)
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-pthread", *SAN, *NUM, *args],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_oracle_driver_under_asan_ubsan():
    exe = os.path.join(OUT, "oracle_sanitize")
    _gcc([os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "tbik_oracle.c"), "-o", exe, "-lm"])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok calls="), r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.parametrize("mode", ["exp", "log", "prod", "rne"])
def test_pins_under_asan_ubsan(mode):
    # one build per process: parallel test workers must not race on the files
    lib = os.path.join(OUT, "liboracle_tbik_san_%d.so" % os.getpid())
    exe = os.path.join(OUT, "pins_san_%d" % os.getpid())
    if not (os.path.exists(lib) and os.path.exists(exe)):
        _gcc(["-fPIC", "-shared", os.path.join(ROOT, "oracle", "tbik_oracle.c"), "-o", lib,
              "-lm"])
        _gcc([os.path.join(ROOT, "tests", "c", "pins.c"), "-o", exe, "-ldl", "-lm"])
    # every 4099th pattern: about a million per mode
    r = subprocess.run([exe, lib, mode, "4", "4099"], capture_output=True, text=True, env=ENV,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    kv = dict(tok.split("=") for tok in r.stdout.split())
    assert int(kv["bad"]) == 0, kv
    if mode in ("exp", "log"):
        assert float(kv["max_ulp"]) < 1.0, kv
    assert "runtime error" not in r.stderr, r.stderr[-4000:]

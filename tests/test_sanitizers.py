"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer: the fp64 oracle
(oracle/kda_oracle.c) and the input generator (datagen/datagen.c) are built with
-fsanitize=address,undefined and the pins that exercise every entry point of both run on those
builds in a child process (the sanitizer runtimes preloaded, since the Python executable itself is
not instrumented): the brute-force product form, decode = prefill, varlen = independent
sequences, finite differences of the backward, and the generator's reference values.  A copy of
the oracle with one planted out-of-bounds read must fail the same run, which shows the sanitizer
is active in that process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")
DATAGEN_SRC = os.path.join(ROOT, "datagen", "datagen.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]

RUNNER = r'''
import sys
sys.path.insert(0, {root!r})
import datagen, oracle
oracle._LIB_PATH, datagen._LIB_PATH = {olib!r}, {dlib!r}
oracle.build = lambda force=False: oracle._LIB_PATH
datagen.build = lambda force=False: datagen._LIB_PATH
from tests import test_datagen, test_oracle_backward_pins, test_oracle_pins
test_oracle_pins.test_p1_brute_force_product_form(7, 8, 5)
test_oracle_pins.test_p12_decode_equals_prefill()
test_oracle_pins.test_p13_varlen_independent_sequences()
test_oracle_pins.test_forward_units_equals_batched_slices()
test_oracle_backward_pins.test_p17_finite_differences_every_element()
test_datagen.test_splitmix64_reference_outputs()
test_datagen.test_deterministic_and_slice_independent()
test_datagen.test_varlen_lengths()
print("SANITIZED_PINS_OK")
'''


def runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def build(src, out):
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-pthread"] + SAN + [src, "-o", out, "-lm"])


def run_pins(olib, dlib):
    preload = [runtime("libasan.so"), runtime("libubsan.so")]
    env = dict(os.environ, LD_PRELOAD=":".join(preload), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = RUNNER.format(root=ROOT, olib=olib, dlib=dlib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                          timeout=600)


@pytest.fixture(scope="module")
def sanitized_datagen(tmp_path_factory):
    if not (runtime("libasan.so") and runtime("libubsan.so")):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    d = tmp_path_factory.mktemp("san")
    lib = str(d / "libdatagen_san.so")
    build(DATAGEN_SRC, lib)
    return lib


def test_oracle_and_datagen_under_asan_ubsan(sanitized_datagen, tmp_path):
    olib = str(tmp_path / "libkda_oracle_san.so")
    build(ORACLE_SRC, olib)
    r = run_pins(olib, sanitized_datagen)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0 and "SANITIZED_PINS_OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_planted_overflow_is_reported(sanitized_datagen, tmp_path):
    """The output row of the last token read one element past its end: the sanitized run fails."""
    old = "for (int j = 0; j < dv; ++j) o[j] += S[(size_t)c * dv + j] * qq[c];"
    text = open(ORACLE_SRC).read()
    assert text.count(old) == 1
    src = tmp_path / "planted.c"
    src.write_text(text.replace(old, "for (int j = 0; j <= dv; ++j) o[j] += S[(size_t)c * dv + j] * qq[c];"))
    olib = str(tmp_path / "libplanted.so")
    build(str(src), olib)
    r = run_pins(olib, sanitized_datagen)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]

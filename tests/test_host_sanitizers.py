"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host-side parts are built with `-fsanitize=address,undefined -fno-sanitize-recover=all`
and exercised:
  - the oracle (oracle/kvq_oracle.cpp): every pin of tests/oracle_pins.py runs against the
    instrumented build in a child process with the ASan runtime preloaded;
  - the library's argument checks and size computations (csrc/kvq_validate.cpp, which
    needs no HIP): tests/native/validate_driver.cpp replays the documented statuses and
    sweeps extreme sizes.
A sanitizer finding aborts the child, so a clean exit with the expected last line means
no finding. Two copies of the oracle with a planted mistake (one heap read past a row,
one signed overflow) must abort, which shows the instrumentation is live.
Built with gcc/g++ only; nothing here uses a GPU.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "kvq_oracle.cpp")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins as pins
with oracle.using({lib!r}):
    for chk in pins.ALL_CHECKS + [lambda: pins.check_f16_conversion_f16c(full=False)]:
        chk()
print("PINS PASSED", len(pins.ALL_CHECKS))
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None,
                                reason="gcc with the ASan runtime is needed")


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run_pins(lib):
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=900, env=_env())


def _build_oracle(src_text, tmp, name):
    src = os.path.join(tmp, f"{name}.cpp")
    with open(src, "w") as f:
        f.write(src_text)
    return oracle.build(src, os.path.join(tmp, f"lib{name}.so"), extra=SAN + [f"-I{os.path.dirname(ORACLE_SRC)}"])


def test_oracle_pins_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_oracle(open(ORACLE_SRC).read(), tmp, "kvq_oracle_san")
        r = _run_pins(lib)
    assert r.returncode == 0 and "PINS PASSED" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


PLANTED = [
    # the group min/max scan reads one element past the group: past the row for the last
    ("heap_read_past_row", "for (int i = 1; i < group; ++i) {\n      if (xg[i] < mn)",
     "for (int i = 1; i <= group; ++i) {\n      if (xg[i] < mn)", "AddressSanitizer"),
    # a signed counter pushed past INT_MAX
    ("signed_overflow", "  int c = 0;\n  while (v) {", "  int c = 2147483647;\n  while (v) {", "runtime error"),
]


@pytest.mark.parametrize("name,old,new,marker", PLANTED, ids=[p[0] for p in PLANTED])
def test_sanitizers_catch_planted_mistakes(name, old, new, marker):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_oracle(src.replace(old, new), tmp, f"planted_{name}")
        r = _run_pins(lib)
    assert r.returncode != 0 and marker in r.stderr, (name, r.returncode, r.stderr[-2000:])


def test_validation_under_asan_and_ubsan():
    if shutil.which("g++") is None:
        pytest.skip("g++ is needed")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "validate_driver")
        cmd = ["g++", "-std=c++17", "-O1", *SAN, f"-I{os.path.join(ROOT, 'include')}",
               os.path.join(ROOT, "tests", "native", "validate_driver.cpp"),
               os.path.join(ROOT, "bit_kv_cache_quantize_amd", "csrc", "kvq_validate.cpp"), "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout[-1000:] + r.stderr[-4000:]

"""The CPU pins under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle's and the input generator's C are rebuilt with both sanitizers (host
code only) and the pins and golden checks run against those builds in a
separate process, which aborts on the first report."""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    with tempfile.TemporaryDirectory() as tmp:
        orc = os.path.join(tmp, "liboracle.so")
        syn = os.path.join(tmp, "libsynth.so")
        flags = [f for f in oracle.CFLAGS if f != "-O2"]
        subprocess.check_call(["gcc", *flags, *SAN, os.path.join(ROOT, "oracle", "csa2_oracle.c"), "-o", orc, "-lm"])
        subprocess.check_call(["gcc", "-std=c11", "-pthread", "-shared", "-fPIC", *SAN,
                               os.path.join(ROOT, "synth", "csa2_synth.c"), "-o", syn, "-lm"])
        env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", CSA2_ORACLE_SO=orc, CSA2_SYNTH_SO=syn)
        r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "tests/test_golden.py", "-q",
                            "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]

"""The oracle's pins again, against a build of the oracle with AddressSanitizer
and UndefinedBehaviorSanitizer: an out-of-bounds access, a use after free or
undefined behaviour anywhere the pins reach aborts the child process.

The sanitizer runtime must be the first library loaded, so the pins run in a
child interpreter that preloads it and loads oracle/liboracle_asan.so through
MXFP8_ORACLE_LIB (host code only; nothing here touches a GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_codec.py", "test_oracle_quant.py", "test_oracle_gemm_dense.py", "test_oracle_routing.py",
        "test_oracle_moe.py"]


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_address_and_ub_sanitizers():
    from oracle import build as ob
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("g++ sanitizer runtimes not installed")
    src = os.path.join(ROOT, "oracle", "mxfp8_oracle.cpp")
    if not os.path.exists(ob.ASAN_LIB) or os.path.getmtime(ob.ASAN_LIB) < os.path.getmtime(src):
        ob.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", MXFP8_ORACLE_LIB=ob.ASAN_LIB)
    probe = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.lib()._name)"], cwd=ROOT, env=env,
                           capture_output=True, text=True)
    assert probe.returncode == 0 and probe.stdout.strip() == ob.ASAN_LIB, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(ROOT, "tests", f) for f in PINS]], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "failed" not in r.stdout

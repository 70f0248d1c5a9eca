"""The host side under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

libkda's host code (argument validation, the planner, workspace sizing, launch set-up) is built
with g++ -fsanitize=address,undefined and linked with the regular device objects; the oracle is
built the same way.  The ABI validation tests and the oracle's pins then run in a child process
with gcc's sanitizer runtimes preloaded, and must pass with no sanitizer report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_code_is_clean_under_sanitizers(tmp_path):
    from chunked_gated_delta_13_amd import build as kbuild
    import oracle
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    built = os.path.isdir(kbuild.BUILD_DIR) and any(f.endswith(".hip.o") for f in os.listdir(kbuild.BUILD_DIR))
    if not built:
        pytest.skip("no device objects: the regular build has not run here")
    lib = kbuild.build_sanitized(str(tmp_path))
    ora = oracle.build(sanitized_out=str(tmp_path / "libkda_oracle_san.so"))
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    files = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_spec_pins.py",
             "tests/test_oracle_ckpt_pins.py", "tests/test_oracle_gate_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        f"--kda-library={lib}", f"--oracle-library={ora}", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    print(tail)
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail

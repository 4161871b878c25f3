"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer:
  - the oracle's pins (tests/test_oracle_*.py and the checked-permute
    reference) against a sanitized build of oracle/moe_oracle.c (gcc);
  - the host layer's validation, workspace and saved-tensor arithmetic and
    its error paths (tests/test_abi.py) against a build of libmoe whose host
    code is sanitized (clang; device code as always).
Each run is a child process that preloads the sanitizer runtime; a report
aborts it (halt_on_error), which fails the test.  Leak checking is off: the
interpreter itself keeps memory until exit."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _runtime(compiler, name):
    r = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not found for {compiler}")
    return path


def _pytest(env_extra, files):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + files, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(force=True, out=str(tmp_path / "libmoe_oracle_san.so"), sanitize=True)
    asan = _runtime("gcc", "libasan.so")
    out = _pytest(dict(LD_PRELOAD=asan, MOE_ORACLE_LIBRARY=lib),
                  ["tests/test_oracle_routing.py", "tests/test_oracle_expert.py",
                   "tests/test_oracle_mx.py", "tests/test_checked_permute_reference.py"])
    print(out.strip().splitlines()[-1])


def test_host_layer_under_asan_ubsan(tmp_path):
    from grouped_gemm_expert_amd import build
    lib = build.build(out=str(tmp_path / "libmoe_san.so"), sanitize_host=True)
    asan = _runtime("/opt/rocm/llvm/bin/clang", "libclang_rt.asan-x86_64.so")
    out = _pytest(dict(LD_PRELOAD=asan, MOE_LIBRARY=lib), ["tests/test_abi.py"])
    print(out.strip().splitlines()[-1])

"""Host-side sanitizer runs (CPU only): AddressSanitizer and
UndefinedBehaviorSanitizer over

- the CPU oracle (oracle/mobmoe_oracle.cpp, built with g++ and the
  sanitizers), exercised by the oracle pin tests, and
- the C ABI's host-side argument checks (sparse_moe_ffn_amd/csrc/api.hip
  compiled with the sanitizers on its host pass only; every kernel object is
  the regular build), exercised by the host-check tests.

Each runs the named tests in a child process with the sanitizer runtimes
preloaded; any report fails the child (halt_on_error, no recovery) and so
this test.  No GPU is touched: the host checks fail before any launch.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name: str) -> str:
    return subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _child_env(extra: dict) -> dict:
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}"
    # Python's own allocations are not under test; stop at the first report
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def _run_tests(env: dict, *args) -> subprocess.CompletedProcess:
    # -s: the sanitizer report goes to the child's stderr, which pytest would
    # otherwise capture and lose when the report ends the child
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                           "-p", "no:xdist", *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


def test_oracle_under_sanitizers(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", *SAN, os.path.join(ROOT, "oracle", "mobmoe_oracle.cpp"), "-o",
                    str(lib)], check=True)
    r = _run_tests(_child_env({"MOBMOE_ORACLE_LIB": str(lib), "OMP_NUM_THREADS": "1"}),
                   "tests/test_oracle_pins.py", "-m", "not gpu")
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_host_checks_under_sanitizers(tmp_path):
    objs = sorted(glob.glob(os.path.join(ROOT, "sparse_moe_ffn_amd", "_build", "*.hip.o")))
    if not objs:
        pytest.skip("library objects not built (python -m sparse_moe_ffn_amd.build)")
    api = tmp_path / "api_san.o"
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    subprocess.run(["hipcc", *flags, *host_san, "-c",
                    os.path.join(ROOT, "sparse_moe_ffn_amd", "csrc", "api.hip"), "-o", str(api)],
                   check=True)
    lib = tmp_path / "libmobmoe_san.so"
    others = [o for o in objs if not o.endswith("api.hip.o")]
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address,undefined", str(api), *others, "-o", str(lib)], check=True)
    r = _run_tests(_child_env({"MOBMOE_LIB": str(lib)}), "tests/test_abi_host.py", "-m", "not gpu")
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr

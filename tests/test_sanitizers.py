"""CPU-side sanitizer runs (no GPU): the library's C ABI host code and the fp64 oracle, each built with
AddressSanitizer and UndefinedBehaviorSanitizer, run their own tests in a child process with the matching
runtime preloaded -- tests/test_abi.py against the library (argument checks, size queries, error paths) and
tests/test_oracle_pins.py against the oracle.  Any out-of-bounds access, use after free or undefined behaviour
aborts the child and fails here."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_child(env_extra, test_file, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", test_file)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"{test_file} under sanitizers failed (rc {r.returncode}):\n{tail}"
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    return r.stdout


def test_abi_host_code_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from mla_latent_kv_fwd_amd import build as B
    rt = B.asan_runtime()
    if not rt:
        pytest.skip("no clang ASan runtime next to hipcc")
    lib = B.build_host_sanitized(str(tmp_path / "san"))
    out = _run_child({"MLA_DECODE_LIB": lib, "LD_PRELOAD": rt}, "test_abi.py")
    assert "passed" in out


def test_oracle_under_asan_ubsan():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(asan) and os.path.isabs(ubsan)):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    env = {"ORACLE_SANITIZE": "1", "LD_PRELOAD": f"{asan}:{ubsan}", "OMP_NUM_THREADS": "2"}
    # build in this process (no preload needed to compile), then run the pins in the child
    subprocess.run([sys.executable, "-c", "from oracle import oracle; oracle.build(force=True)"], cwd=ROOT,
                   env={**os.environ, "ORACLE_SANITIZE": "1"}, check=True, timeout=300)
    out = _run_child(env, "test_oracle_pins.py")
    assert "passed" in out

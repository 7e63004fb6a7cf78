"""The library driven from plain C (tests/c_client/mla_client.c): device buffers from the HIP runtime, the
split plan, the attention kernel (forced to split the long request over 7 workgroups) and the merge, every output
row checked against the fp64 oracle inside the program.  Built by the repository's build step."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "mla_client")


def test_c_client_matches_oracle():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is missing: run the build step first")
    print("[gpu-test] c client", flush=True)
    sys.stdout.flush()
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, f"mla_client exited with {r.returncode}: {r.stdout} {r.stderr}"
    assert "out max-abs" in r.stdout

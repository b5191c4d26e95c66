"""A prune step driven from C through the C ABI alone, checked against the
oracle's C functions (tests/c_abi/prune_from_c.c): scores within 2e-3 * M,
the top-B of the GPU's own scores with ties to the lower slot, the oracle's
clearly kept and clearly evicted keys, and bit-exact compaction.  The
program is built by __graft_entry__.build() and runs as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BINARY = os.path.join(HERE, "c_abi", "prune_from_c")


def test_prune_step_from_c():
    if not os.path.exists(BINARY):
        pytest.fail("tests/c_abi/prune_from_c is not built (run __graft_entry__.build())")
    r = subprocess.run([BINARY], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed checks" in r.stdout

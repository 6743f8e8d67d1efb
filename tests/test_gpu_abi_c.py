"""The C ABI from a plain C program (tests/abi_example.c, built by
__graft_entry__.build()): hipMalloc'd buffers, one stream, no Python binding.
It checks layout invariants, rows bit-equal to their tokens and an exact
identity-expert combine, and exits 0 on success."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "_build", "abi_example")


def test_c_program_runs_the_path():
    if not os.path.exists(EXE):
        pytest.skip("tests/_build/abi_example not built (built by __graft_entry__.build())")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi example: ok" in r.stdout

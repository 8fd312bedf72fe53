"""The hot path driven from C through the ABI alone (no Python between the
caller and the library): tests/c_abi/ep_c_test.c runs layout, dispatch,
combine and the one-call layout and dispatch on two problems and checks them
against the C oracle it links.  __graft_entry__.build() compiles it."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "ep_c_test")


def test_c_caller_matches_the_oracle():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built; run __graft_entry__.build()")
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count(": ok") == 2

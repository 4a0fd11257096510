"""The C ABI driven from C++ (tests/host/abi_example.cpp, built by
__graft_entry__.build()): warm-up with the variance norm, freeze, deferred
steps with the implicit momentum, checked against the oracle inside the
program."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "abi_example")


def test_abi_example_program_matches_oracle():
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build() first"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "abi_example: ok" in r.stdout

"""The C ABI from a plain C program: tests/c_abi_e2e (built by
__graft_entry__.build(), source tests/c_abi_e2e.c) allocates device memory
with the HIP runtime, calls libtide's reduce-scatter and placement without
Python or torch, and compares every output bit with the CPU oracle.
"""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_program_through_the_abi():
    exe = os.path.join(HERE, "c_abi_e2e")
    if not os.path.exists(exe):
        pytest.fail("tests/c_abi_e2e is not built: run __graft_entry__.build()")
    say("c-abi: running %s" % exe)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi: ok" in r.stdout, r.stdout

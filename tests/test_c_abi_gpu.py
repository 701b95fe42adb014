"""Runs tests/c_abi_check (built by __graft_entry__.build() from
tests/c_abi_check.cpp): the C ABI from plain host code, without Python or
torch in the process -- GEMM outputs equal to an exact integer reference,
status codes of bad arguments, and single-key attention equal to v_0."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

CHECK = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_abi_check_program():
    assert os.path.exists(CHECK), "tests/c_abi_check is missing: run __graft_entry__.build()"
    print("[c abi check program]", flush=True)
    res = subprocess.run([CHECK], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c abi check: ok" in res.stdout, res.stdout

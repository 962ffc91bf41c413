"""The C ABI called from a C program (tests/c_abi_roundtrip.c, built by
__graft_entry__.build() into bulk_async_tensor_amd/_build/): plain hipMalloc
pointers and the null stream, checked through layout invariants, bitwise
dispatch and the exact identity round trip.  The program runs as a child
process."""

import os
import subprocess

import pytest

from bulk_async_tensor_amd.build import C_TEST_BIN

pytestmark = pytest.mark.gpu


def test_c_program_round_trip():
    if not os.path.exists(C_TEST_BIN):
        pytest.fail(f"{C_TEST_BIN} is not built (run __graft_entry__.build())")
    res = subprocess.run([C_TEST_BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c_abi_roundtrip: ok" in res.stdout

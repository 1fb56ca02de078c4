"""The C ABI driven from plain C on the GPU: tests/c/abi_check (built by the
build step from tests/c/abi_check.c, no Python or torch inside) checks that
dual = two singles, multi-part = one call per part, packed = u8 codes, fused
q|k|v = product then split and the split itself, bit for bit, on GEMV rows
and on matrix-core rows, and that a bad argument returns QG_EINVAL."""
import os
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

BIN = os.path.join(ROOT, "tests", "c", "abi_check")


def test_c_program_checks_the_stated_equalities():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() (or python tests/c/build.py)"
    print(f"running {BIN}", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_check: ok (argument checks; dual" in res.stdout, res.stdout

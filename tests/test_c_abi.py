"""The C ABI driven from a plain C program (tests/c_abi/abi_check.c): no
Python, no torch in that process, device buffers from hipMalloc.  The host
run checks validation paths only; the GPU run checks every call family
against the fp64 oracle linked into the same program."""
import os
import subprocess

import pytest

from tests.c_abi import build as cbuild


def _exe():
    if not os.path.exists(cbuild.EXE):
        cbuild.build()
    return cbuild.EXE


def test_c_program_host_validation():
    r = subprocess.run([_exe(), "--host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout


@pytest.mark.gpu
def test_c_program_on_gpu():
    r = subprocess.run([_exe()], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout

"""The C ABI driven from a plain C program (tests/c_abi/abi_check.c): no
Python, no torch in that process, device buffers from hipMalloc.  The host
run checks validation paths only; the GPU run checks every call family
against the fp64 oracle linked into the same program.  The host-only runs
(validation, and the oracle's functions alone) are also built with
AddressSanitizer and UBSan (gcc; the HIP library itself is not
instrumented) and must finish without a report."""
import os
import subprocess

import pytest

from tests.c_abi import build as cbuild


def _exe():
    srcs = [os.path.join(cbuild.HERE, "abi_check.c"), os.path.join(cbuild.ROOT, "oracle", "oracle.c")]
    if not os.path.exists(cbuild.EXE) or os.path.getmtime(cbuild.EXE) < max(map(os.path.getmtime, srcs)):
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


def test_c_program_oracle_checks():
    r = subprocess.run([_exe(), "--oracle"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout


@pytest.mark.parametrize("mode", ["--oracle", "--host"])
def test_sanitized_host_runs(mode):
    """oracle.c and the host side of abi_check.c under -fsanitize=address,undefined
    with every report fatal (leak checking off: the HIP runtime keeps its
    allocations to process end)."""
    exe = cbuild.build(sanitize=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, mode], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr

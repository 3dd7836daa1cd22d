"""The C ABI from plain C: tests/c_abi_example (built from
tests/c_abi_example.c by the package's build step, linked against
libkda.so with gcc) runs a prefill call and decode steps through
include/kda.h with device buffers from the HIP runtime's C API, and checks
closed forms (alpha = 1, beta = 0 keeps the state and reads rows of S0; a
zero-valued write with beta = 1 erases a row).  It runs as a child process."""
import os
import subprocess

import pytest

from tests.gpu_harness import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_example")


def test_plain_c_caller():
    assert os.path.exists(EXE), "build the package first: it links tests/c_abi_example"
    log("[c abi] tests/c_abi_example")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip() + (" | " + r.stderr.strip() if r.stderr.strip() else ""))
    assert r.returncode == 0, r.stderr
    assert "c-abi example: ok" in r.stdout

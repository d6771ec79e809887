"""The C ABI from C: tests/c_abi_check (built from tests/c_abi_check.c by
tests/c_abi_build.py, which __graft_entry__.build() runs) drives the linear,
the fused SwiGLU linear and the prepared-code contraction through
include/convrot.h on a HIP stream of its own, with hipMalloc'd memory, and
checks them against the oracle's C functions (bit for bit, the fused SwiGLU
within one bf16 ulp of the exact value) and the status of every argument
error."""
import os
import subprocess

import pytest

from tests import c_abi_build

pytestmark = pytest.mark.gpu


def test_c_abi_from_c():
    exe = c_abi_build.EXE
    if not os.path.exists(exe):
        c_abi_build.build()
    print("running %s" % exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, "C ABI check failed (rc %d):\n%s\n%s" % (r.returncode, r.stdout, r.stderr)
    assert "c abi check: ok" in r.stdout

"""The C ABI from C++ without Python: tests/c_abi/abi_roundtrip (built with the
library) allocates with hipMalloc, drives the standard step and ReplaySSM
append-decode on one HIP stream, and checks that the outputs agree and that the
pointer word follows the flush-when-full schedule.  Run as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_roundtrip")


def test_c_program_drives_the_abi():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with `python -m ssm_recurrent_decode_amd.build`")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout

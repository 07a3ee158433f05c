"""The C ABI driven from a plain C program (tests/c_abi/uf_c_check.c, built with the library):
no Python in that process, device memory from the HIP runtime, a rolling cache that wraps,
attention steps and an error path, checked on what holds exactly (see the program's header)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "uf_c_check")


def test_c_program_drives_the_abi():
    assert os.path.exists(BIN), "tests/c_abi/uf_c_check is built with the library (windowed_attention_amd.build)"
    print("running tests/c_abi/uf_c_check", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().splitlines()[-1] == "uf_c_check: ok"

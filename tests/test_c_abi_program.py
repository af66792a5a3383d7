"""The decode driven from a plain C program (tests/c_abi_decode.c) through the
library's C ABI alone: no Python or torch between the caller and the
kernels. The program checks its own result against the C oracle and reports
through its exit status (0 pass, 1 mismatch, 2 setup error)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "tests", "c_abi_decode.c")
BINARY = os.path.join(ROOT, "tests", "c_abi_decode")


def _binary():
    """The built program; built here only if nothing is built (a fresh
    checkout), and refused when older than its source."""
    if not os.path.exists(BINARY):
        import __graft_entry__
        __graft_entry__.build()
    assert os.path.getmtime(BINARY) >= os.path.getmtime(SOURCE), \
        "tests/c_abi_decode is older than its source: run __graft_entry__.build()"
    return BINARY


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0


def test_program_loads_without_a_device():
    """It links against both libraries and starts; with no GPU it stops at
    the device check with status 2 (nothing is launched)."""
    if _gpu_present():
        pytest.skip("a GPU is present: the GPU test runs the program")
    res = subprocess.run([_binary()], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2, (res.returncode, res.stdout, res.stderr)
    assert "no HIP device" in res.stderr


@pytest.mark.gpu
def test_program_decodes_through_the_c_abi():
    print("\n[gpu case] plain-C program: 5 rows x 40 heads, D 256, width 300", flush=True)
    res = subprocess.run([_binary()], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert "sets equal" in res.stdout

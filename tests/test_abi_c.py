"""The boundary from plain C: include/ttl.h compiles as strict C99 with gcc, a C program links
against libttl.so, and its validation-only calls (tests/c/abi_check.c) return the documented
statuses.  No call reaches the device."""

import os
import shutil
import subprocess

import pytest

from tensor_transformer_linear_amd import ttl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0  # counts devices without initialising one


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.skipif(_gpu_present(), reason="passes fake device pointers; CPU-only check")
def test_c_program_links_and_validates(tmp_path):
    libdir = os.path.dirname(ttl.LIB_PATH)
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-o", str(exe), "-L", libdir, "-lttl", f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ALL OK" in out.stdout

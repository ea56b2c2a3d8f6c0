"""The C ABI from plain C (CPU only): include/drafter_attn.h compiles as C99 with all
warnings as errors, links against the library, and the host-only queries answer."""
import os
import shutil
import subprocess

import pytest

from speculative_decoding_drafter_amd import _lib
from speculative_decoding_drafter_amd.build import INCLUDE

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_as_c99_and_links(tmp_path):
    lib = _lib.library_path()
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    exe = tmp_path / "abi_host_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE,
           os.path.join(HERE, "c", "abi_host_check.c"), "-o", str(exe), lib, f"-Wl,-rpath,{os.path.dirname(lib)}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok ")

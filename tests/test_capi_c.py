"""The C ABI from C: tests/capi/check_capi.c compiled as strict C11 with gcc against
include/fa.h, linked with libfa.so and run on the CPU. Every library call in it is refused by
host validation or is a pure size query, so no GPU work is enqueued."""
import os
import shutil
import subprocess

import pytest

from tests import _lib

import exact_attention_27_amd as fa


def test_c11_consumer(tmp_path):
    _lib.ensure_built()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    root = _lib.ROOT
    exe = os.path.join(str(tmp_path), "check_capi")
    libdir = os.path.dirname(fa.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(root, "include"),
           os.path.join(root, "tests", "capi", "check_capi.c"), "-o", exe, "-L", libdir, "-l:libfa.so",
           f"-Wl,-rpath,{libdir}", "-Wl,-rpath-link,/opt/rocm/lib"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr

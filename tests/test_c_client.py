"""The C ABI from C: tests/abi_client.c, a C99 program that includes only
include/qsa.h and the HIP runtime API, is compiled with strict warnings
(-std=c99 -pedantic -Werror; the ROCm headers as system headers) and linked
against the built libqsa.so.

* CPU: the version, and the NULL, shape, alignment and scratch-size errors
  that the header promises before any device work.
* GPU: one qsa_quantize call on hipMalloc'd memory and a stream, checked
  against the closed form of constant blocks (scale |x|/127, codes +-127,
  pooled sums +-127 x rows, a zero block, a ragged last block).
"""
import os
import shutil
import subprocess

import pytest

from quantized_sparse_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libqsa.so is not built")
    exe = str(tmp_path_factory.mktemp("c_client") / "abi_client")
    libdir = os.path.dirname(os.path.abspath(B.LIB_PATH))
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "abi_client.c"),
           "-o", exe, os.path.abspath(B.LIB_PATH), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_client_compiles_links_and_gets_argument_errors(client):
    r = subprocess.run([client], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr


@pytest.mark.gpu
def test_c_client_quantizes_on_the_device(client):
    r = subprocess.run([client, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr

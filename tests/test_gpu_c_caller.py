"""The library from a torch-free C program on the GPU (tests/abi_c/device_check.c):
device memory and copies through the HIP runtime's C API, the small parity
configuration run as one block and token by token, both compared with the
oracle (linked as a test library) and with each other."""
import os
import shutil
import subprocess

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_c_program_block_and_decode_match_the_oracle(tmp_path):
    import oracle
    from kv_cache_token_amd import _lib
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib, orc = _lib.LIB_PATH, oracle.build(force=False)
    exe = str(tmp_path / "device_check")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    dirs = [os.path.dirname(lib), os.path.dirname(orc), os.path.join(rocm, "lib")]
    subprocess.check_call([gcc, "-std=gnu11", "-w", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_c", "device_check.c"),
                           "-o", exe, "-L", dirs[0], "-l:" + os.path.basename(lib), "-L", dirs[1],
                           "-l:" + os.path.basename(orc), "-L", dirs[2], "-lamdhip64", "-lm",
                           "-Wl,-rpath," + ":".join(dirs)])
    say("running the C caller")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert got == {"scores_within_tolerance": "1", "block_equals_oracle": "1", "decode_equals_oracle": "1",
                   "block_equals_decode": "1"}, r.stdout

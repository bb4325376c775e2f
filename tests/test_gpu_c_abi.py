"""The C ABI driven from a C program on the GPU (tests/c_gpu_step.c): device
memory from hipMalloc, or the streamed buffers carved from one contiguous
block as the header's placement note advises, the library's calls in the
order a rank's step makes them, the oracle linked beside it.  Built here with gcc -std=c11 against
include/zshard.h, libzshard.so, liboracle.so and the HIP runtime."""
import os
import shutil
import subprocess

import pytest

import oracle
from fsdp_sharded_optimizer_amd import _binding as B

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.parametrize("placement", ["hipMalloc", "contiguous"])
def test_c_program_runs_a_tiled_step_like_the_oracle(tmp_path, placement):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(B.LIB_PATH):
        raise RuntimeError(f"{B.LIB_PATH} is missing: build the library first")
    oracle.lib()   # builds liboracle.so if needed
    orc_so = os.path.join(ROOT, "oracle", "liboracle.so")
    exe = str(tmp_path / "c_gpu_step")
    print("c gpu step: build", flush=True)
    subprocess.run([gcc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    "-o", exe, os.path.join(ROOT, "tests", "c_gpu_step.c"), B.LIB_PATH, orc_so,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
                    f"-Wl,-rpath,{os.path.dirname(B.LIB_PATH)}:{os.path.dirname(orc_so)}:{os.path.join(ROCM, 'lib')}"],
                   check=True)
    print(f"c gpu step: run ({placement})", flush=True)
    out = subprocess.run([exe] + (["contiguous"] if placement == "contiguous" else []), capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == "c gpu step: ok"

"""The C ABI from a plain C program: tests/cabi/hot_path_client.c, built with
gcc against include/bq8.h, libbq8.so and the HIP runtime, runs the hot path on
its own stream with device memory from hipMalloc and checks every step against
the CPU oracle's C library (see the program's header for the bars).  No
Python, torch or binding is involved in the calls."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_quantized_gemv_q8_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gpu_present():
    try:
        import torch
    except ImportError:
        return False
    return torch.cuda.device_count() > 0


if not _gpu_present():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_c_client_runs_the_hot_path(tmp_path):
    lib = os.path.join(PKG, "libbq8.so")
    olib = os.path.join(ORACLE, "libbq8_oracle.so")
    assert os.path.exists(lib), "libbq8.so is not built"
    assert os.path.exists(olib), "the oracle library is not built"
    exe = str(tmp_path / "hot_path_client")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "cabi", "hot_path_client.c"), "-o", exe,
           f"-L{PKG}", "-lbq8", f"-L{ORACLE}", "-lbq8_oracle", f"-L{ROCM}/lib", "-lamdhip64",
           "-lm", f"-Wl,-rpath,{PKG}:{ORACLE}:{ROCM}/lib"]
    subprocess.run(cmd, check=True)
    print("running the C client", file=sys.stderr, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    print(r.stdout, file=sys.stderr)
    print(r.stderr, file=sys.stderr, flush=True)
    assert r.returncode == 0, f"C client exited {r.returncode}: {r.stderr}"
    assert "all checks passed" in r.stdout

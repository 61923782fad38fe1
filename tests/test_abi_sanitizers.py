"""The C ABI's host-side validation under the address and undefined-behaviour
sanitizers: the library's host code is rebuilt with them (the device code
with the usual flags) and tests/sanitize/abi_drive.c calls every family of
entry points with arguments that fail validation, plus the host-only size
queries.  Nothing reaches a GPU."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def _asan_runtime_dir():
    hits = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(hits[0]) if hits else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _asan_runtime_dir()),
                    reason="needs hipcc, clang and the clang sanitizer runtime")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    from block_quantized_gemv_q8_amd import build as bqbuild

    lib = tmp_path / "libbq8_san.so"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"]
    flags = [f for f in bqbuild.HIPCC_FLAGS if f != "-O3"] + ["-O1"]
    subprocess.run([HIPCC, *flags, *host_san, f"-I{bqbuild.INCLUDE}", f"-I{bqbuild.CSRC}",
                    *bqbuild.sources(), "-o", str(lib)], check=True, capture_output=True,
                   text=True, timeout=600)
    exe = tmp_path / "abi_drive"
    rt = _asan_runtime_dir()
    subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-shared-libasan",
                    "-fno-sanitize-recover=all", f"-I{bqbuild.INCLUDE}",
                    os.path.join(ROOT, "tests", "sanitize", "abi_drive.c"), str(lib),
                    f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{rt}", "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LD_LIBRARY_PATH=f"{rt}:{os.environ.get('LD_LIBRARY_PATH', '')}")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip() == "ok"

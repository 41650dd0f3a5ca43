"""The C ABI's host-side argument validation under the address and undefined-behaviour
sanitizers.  `tests/native/abi_validation.c` calls every entry point with arguments the
library must refuse (NULL, misaligned or overflowing shapes, bad scalars, short workspaces,
out-of-range enum values) and the size helpers with extreme shapes; nothing reaches the GPU.
`api.hip` is rebuilt here with the sanitizers on its host code only and linked with the
library's other objects, so a signed overflow, an invalid enum load or an out-of-bounds
host access in the validation aborts the program."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_quantized_finetuning_quant_amd")
OBJS = ["codec", "qgemm", "lora", "gemv", "linear", "optim", "dropout"]


def test_validation_is_clean_under_host_sanitizers(tmp_path):
    from bit_quantized_finetuning_quant_amd import build

    objdir = os.path.join(PKG, "_build")
    objs = [os.path.join(objdir, f"{o}.o") for o in OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library objects are not built (run the build first)")
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang) or not shutil.which(build.hipcc()):
        pytest.skip("the ROCm compilers are not installed")
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    api_o, drv_o, exe = str(tmp_path / "api_san.o"), str(tmp_path / "drv.o"), str(tmp_path / "abi_validation")
    # the sanitizers instrument the host code only (each option after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    subprocess.run([build.hipcc(), *flags, *san, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "native", "abi_validation.c"),
                    "-o", drv_o], check=True, capture_output=True)
    subprocess.run([clang + "++", "-fsanitize=address,undefined", drv_o, api_o, *objs, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:protect_shadow_gap=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all refusals as documented" in r.stdout

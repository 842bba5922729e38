"""The C interface used from C: include/tp.h compiles as strict C, and a C program
that calls the library (tests/c/mlp_example.c) builds against libtp_amd.so and,
on a GPU, reproduces an exact integer MLP both as one tp_mlp call and as the
three separate calls.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "tensor_sharded_linear_amd")
LIB = os.path.join(PKG, "libtp_amd.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXAMPLE = os.path.join(ROOT, "tests", "c", "mlp_example.c")
STRICT = ["-Wall", "-Wextra", "-Werror", "-pedantic"]


def _gcc():
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc is not installed")
    return cc


def build_example(out_path: str) -> str:
    if not os.path.exists(LIB):
        pytest.skip("libtp_amd.so is not built")
    cmd = [_gcc(), "-std=c99", *STRICT, "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-isystem",
           os.path.join(ROCM, "include"), EXAMPLE, "-o", out_path, "-L", PKG, "-ltp_amd", "-L",
           os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"building the C example failed:\n{r.stdout}\n{r.stderr}"
    return out_path


@pytest.mark.parametrize("std", ["c89", "c99", "c11"])
def test_header_is_strict_c(tmp_path, std):
    src = tmp_path / "use_header.c"
    src.write_text('#include "tp.h"\nint main(void) { tp_matrix m; m.dtype = TP_BF16; return (int)TP_OK + m.dtype - 1; }\n')
    r = subprocess.run([_gcc(), f"-std={std}", *STRICT, "-I", INCLUDE, "-c", str(src), "-o", str(tmp_path / "u.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_example_builds(tmp_path):
    build_example(str(tmp_path / "mlp_example"))


@pytest.mark.gpu
def test_c_example_runs_exact(tmp_path):
    exe = build_example(str(tmp_path / "mlp_example"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stdout}\n{r.stderr}"
    assert "exact" in r.stdout

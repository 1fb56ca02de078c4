"""Build tests/c/abi_check: a plain C program that drives libqgemv_q4 through
its C ABI alone (host code only, gcc; device memory from the HIP runtime's C
API).  Run as a script, or build(out) from the tests and the build entry."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str) -> list:
    lib = os.path.join(ROOT, "gemm_qgemv_q4_amd", "lib")
    rel = os.path.relpath(lib, os.path.dirname(os.path.abspath(out)))
    cc = shutil.which("gcc") or "cc"
    return [cc, "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
            os.path.join(HERE, "abi_check.c"), "-o", out,
            "-L", lib, "-lqgemv_q4", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/" + rel, "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(out: str = os.path.join(HERE, "abi_check")) -> str:
    res = subprocess.run(command(out), capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"building {out} failed ({res.returncode})")
    return out


if __name__ == "__main__":
    print("built", build())

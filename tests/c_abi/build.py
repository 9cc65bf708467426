"""Build tests/c_abi/abi_check: the C ABI test program, linked against the
in-tree liblse.so, the HIP runtime and the oracle's C source (test code)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "abi_check")


def build() -> str:
    pkg = os.path.join(ROOT, "log_softmax_reductions_amd")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "abi_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-L", pkg, "-llse", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{pkg}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", EXE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_check build failed:\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())

"""Build tests/c_abi/abi_check: the C ABI test program, linked against the
in-tree liblse.so, the HIP runtime and the oracle's C source (test code)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "abi_check")
EXE_SAN = os.path.join(HERE, "abi_check_san")
# Host-only C build (gcc, no GPU code on the line): AddressSanitizer and
# UBSan, every UB report fatal.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-g"]


def build(sanitize: bool = False) -> str:
    pkg = os.path.join(ROOT, "log_softmax_reductions_amd")
    exe = EXE_SAN if sanitize else EXE
    cmd = ["gcc", "-std=c11", "-O1" if sanitize else "-O2", *(SANITIZE if sanitize else []),
           "-fopenmp", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "abi_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
           "-L", pkg, "-llse", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{pkg}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_check build failed:\n{r.stderr}")
    os.replace(exe + ".tmp", exe)
    return exe


if __name__ == "__main__":
    print(build())

"""Builds the plain C caller of libmoe_dispatch.so (tests/c/moe_c_caller.c) with gcc, in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBDIR = os.path.join(ROOT, "unpermute_combine_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def binary_path() -> str:
    return os.path.join(HERE, "moe_c_caller")


def build(out: str = None) -> str:
    """C11, the public header only, linked against the built library and the HIP runtime."""
    out = out or binary_path()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", os.path.join(HERE, "moe_c_caller.c"),
           f"-L{LIBDIR}", "-lmoe_dispatch", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib", "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())

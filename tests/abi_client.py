"""Build of tests/abi_client.c, a plain C99 program that uses the library
through include/msda.h only (gcc, the HIP runtime and libmsda.so; no PyTorch).
Test infrastructure: __graft_entry__.build() builds it next to its source."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "abi_client.c")
BINARY = os.path.join(HERE, "abi_client")
LIBDIR = os.path.join(ROOT, "scale_deformable_attention_amd")


def build(verbose=False):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), SOURCE,
           "-L", LIBDIR, "-lmsda", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           # the library is found next to the package wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../scale_deformable_attention_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", BINARY + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stdout + r.stderr)
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY

"""Build the HIP library (gfx950) in-tree: scale_deformable_attention_amd/libmsda.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "msda.hip"), os.path.join(HERE, "csrc", "linear.hip"),
           os.path.join(HERE, "csrc", "layer.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libmsda.so")
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc would otherwise pair fp32 adds/muls/fmas into
# packed instructions by itself.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(output=LIBRARY, extra_flags=(), verbose=False):
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, *SOURCES, "-o", output + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so: harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)

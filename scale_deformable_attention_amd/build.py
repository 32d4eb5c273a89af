"""Build the HIP library (gfx950) in-tree: scale_deformable_attention_amd/libmsda.so.

Each source is compiled to an object on its own (in parallel), then linked."""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "msda.hip"), os.path.join(HERE, "csrc", "linear.hip"),
           os.path.join(HERE, "csrc", "layer.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libmsda.so")
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc would otherwise pair fp32 adds/muls/fmas into
# packed instructions by itself.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
               "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the host pass does not know the packed-fp32 feature and says so: harmless
_NOISE = "is not a recognized feature for this target"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _messages(r):
    return [l for l in (r.stdout + r.stderr).splitlines() if _NOISE not in l]


def build(output=LIBRARY, extra_flags=(), verbose=False):
    with tempfile.TemporaryDirectory(prefix="msda_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                          text=True))
            objs.append(obj)
        failed = []
        for src, pr in zip(SOURCES, procs):
            out, err = pr.communicate()
            r = subprocess.CompletedProcess(pr.args, pr.returncode, out, err)
            msgs = _messages(r)
            if pr.returncode != 0:
                failed.append(f"{os.path.basename(src)}:\n" + "\n".join(msgs))
            elif verbose and msgs:
                print("\n".join(msgs))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", output + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(_messages(r)))
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    args = sys.argv[1:]
    out = LIBRARY
    if len(args) >= 2 and args[0] == "--output":
        out, args = args[1], args[2:]
    build(output=out, extra_flags=args, verbose=True)

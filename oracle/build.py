"""Build the CPU oracle (plain C, gcc) into oracle/libmsda_oracle.so.

Test infrastructure: the library is loaded only by the test suite, the smoke
check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "msda_oracle.c")
LIBRARY = os.path.join(HERE, "libmsda_oracle.so")

# -O2 and no -ffast-math: the oracle must keep IEEE semantics (NaN tests,
# correctly rounded fmaf). -ffp-contract=off keeps every double operation
# rounded where it is written.
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
          "-Werror"]


def build(extra_flags=(), output=LIBRARY, verbose=False):
    """Compile the oracle; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *extra_flags, SOURCE, "-o", output + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)

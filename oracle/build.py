"""Build the CPU oracle (plain C, gcc) into oracle/libmsda_oracle.so.

Test infrastructure: the library is loaded only by the test suite, the smoke
check and the benchmark's CPU-baseline leg.
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "msda_oracle.c")
LIBRARY = os.path.join(HERE, "libmsda_oracle.so")
# digest of the source and flags the library was built from, written next to it
STAMP = LIBRARY + ".stamp"

# -O2 and no -ffast-math: the oracle must keep IEEE semantics (NaN tests,
# correctly rounded fmaf). -ffp-contract=off keeps every double operation
# rounded where it is written.
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
          "-Werror"]


def source_digest(extra_flags=()):
    """sha256 of the oracle source and the compiler flags."""
    h = hashlib.sha256()
    with open(SOURCE, "rb") as f:
        h.update(f.read())
    h.update(" ".join([*CFLAGS, *extra_flags]).encode())
    return h.hexdigest()


def is_current():
    """True when the in-tree library exists and was built from the current
    source (an edited msda_oracle.c makes it stale)."""
    if not (os.path.exists(LIBRARY) and os.path.exists(STAMP)):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_digest()


def build(extra_flags=(), output=LIBRARY, verbose=False):
    """Compile the oracle; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *extra_flags, SOURCE, "-o", output + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    if output == LIBRARY:
        with open(STAMP + ".tmp", "w") as f:
            f.write(source_digest(extra_flags) + "\n")
        os.replace(STAMP + ".tmp", STAMP)
    return output


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)

"""Compile the fp64 CPU oracle (test infrastructure only) into oracle/libssd_oracle.so.

Plain gcc, no fast-math, so the oracle keeps IEEE double semantics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ssd_oracle.c")
LIBRARY = os.path.join(HERE, "libssd_oracle.so")


def compile_oracle(source=SOURCE, output=LIBRARY, extra_flags=()):
    """Build `source` into the shared library `output`; raises on a compiler error."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-I", HERE, *extra_flags,
           source, "-o", output + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(compile_oracle(), file=sys.stderr)

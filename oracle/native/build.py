"""Compile the C++ oracle (oracle.cpp) into liboracle.so next to it.

Plain g++, no GPU code: -O2 without fast-math and with -ffp-contract=off, so
every double and fp32 operation rounds on its own as written.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = [os.environ.get("CXX", "g++"), *FLAGS, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

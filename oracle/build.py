"""Compile the reference oracle into ``oracle/liboracle.so`` with g++.

Test infrastructure: plain host C++, no GPU code.  ``-ffp-contract=off``
keeps every multiply and add separately rounded, as written.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.cpp")
LIBRARY = os.path.join(HERE, "liboracle.so")
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build(source: str = SOURCE, output: str = LIBRARY, include_dir: str = HERE) -> str:
    cmd = ["g++", *FLAGS, "-I", include_dir, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(build(*sys.argv[1:]))

"""Builds the CPU oracle library (test infrastructure only).

`g++ -O2 -std=c++17 -shared -fPIC -pthread oracle.cpp -o liboracle.so`, in
this folder. Plain host C++: no HIP, no GPU, nothing shared with the product
library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(source=SRC, output=LIB, extra_flags=()):
    """Compiles `source` into the shared library `output` and returns its path."""
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread",
           *extra_flags, source, "-o", output + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(build_oracle())

"""Build the CPU oracle shared library (test infrastructure only).

Plain gcc, no fast-math: the oracle relies on IEEE round-to-nearest-even and x87 long double.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hq_oracle.c")
LIB = os.path.join(HERE, "libhq_oracle.so")


def build(verbose=False, out=None, sanitize=False):
    """Build the library (to `out`, default oracle/libhq_oracle.so). sanitize: an AddressSanitizer
    and UndefinedBehaviorSanitizer build, for the host-side sanitizer test (the process that
    loads it must preload gcc's libasan)."""
    lib = out or LIB
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc"] + flags + ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                             "-fno-fast-math", SRC, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the CPU oracle (test infrastructure only) with the host C++ compiler.

    python oracle/build.py            # -> oracle/libhikv_ref.so
    python oracle/build.py --selftest # also build + run the sanitized self-test
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libhikv_ref.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           os.path.join(HERE, "hikv_ref.cpp"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_selftest(out_dir: str) -> str:
    """Sanitized (address + undefined) native self-test binary of the oracle."""
    exe = os.path.join(out_dir, "hikv_ref_selftest")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(HERE, "hikv_ref.cpp"), os.path.join(HERE, "selftest.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


if __name__ == "__main__":
    print(build(verbose=True))
    if "--selftest" in sys.argv:
        import tempfile
        d = tempfile.mkdtemp()
        exe = build_selftest(d)
        subprocess.run([exe], check=True)

"""Build the fp64 CPU oracle (test infrastructure) with the host C compiler.

Only tests, the smoke check and the benchmark's CPU-baseline leg load the result.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile oracle/gdn_oracle.c into oracle/liboracle.so (always recompiles). `src` and
    `out` let the mutation tests build altered copies elsewhere."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))

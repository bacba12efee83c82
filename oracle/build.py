"""Build the CPU oracle libraries (test infrastructure only).

Two shared objects come from the one C source: ``liboracle_f64.so`` computes in
double, ``liboracle_f32.so`` in float.  Both are compiled without fast math and
with floating-point contraction off, so every sum is evaluated in the written
order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")


def lib_path(precision: str) -> str:
    # GDN_ORACLE_LIB_DIR lets a mutation check load deliberately broken builds.
    return os.path.join(os.environ.get("GDN_ORACLE_LIB_DIR", HERE), f"liboracle_{precision}.so")


def build(verbose: bool = False) -> None:
    for precision, real in (("f64", "double"), ("f32", "float")):
        out = lib_path(precision)
        tmp = out + ".tmp"
        cmd = [
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            "-Wno-unused-parameter", f"-DORACLE_REAL={real}", "-o", tmp, SRC, "-lm",
        ]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)

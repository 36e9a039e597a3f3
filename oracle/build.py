"""Build the CPU oracle (test infrastructure) with gcc: plain -O2, no fast-math,
no floating-point contraction, so each operation rounds as written.  OpenMP
spreads independent outputs over threads (oracle.set_threads); no output's
arithmetic depends on the thread count."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    out = os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

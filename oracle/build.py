"""Build the CPU oracle (test infrastructure) with gcc: plain -O2, no fast-math,
no floating-point contraction, so each operation rounds as written.  OpenMP
spreads independent outputs over threads (oracle.set_threads); no output's
arithmetic depends on the thread count."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


FLAGS = ["-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]
# checks of the oracle itself: any undefined behaviour (or, in the driver
# executable, any invalid memory access) stops the program
UBSAN = ["-fsanitize=undefined", "-fno-sanitize-recover=all", "-g"]
ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
              "-g"]


def build(verbose: bool = False, ubsan: bool = False) -> str:
    """liboracle.so, or with ubsan=True liboracle_ubsan.so (the same code
    under UndefinedBehaviorSanitizer; load it with TD_ORACLE_LIB)."""
    src = os.path.join(HERE, "oracle.c")
    out = os.path.join(HERE, "liboracle_ubsan.so" if ubsan else "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", *FLAGS, "-O1" if ubsan else "-O2", *(UBSAN if ubsan else []),
           "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_sanitize_driver(out_dir: str, verbose: bool = False) -> str:
    """The sanitizer driver (sanitize_driver.c) linked with the oracle under
    AddressSanitizer and UndefinedBehaviorSanitizer, as an executable in
    out_dir."""
    out = os.path.join(out_dir, "oracle_sanitize_driver")
    cmd = ["gcc", *FLAGS, "-O1", *ASAN_UBSAN, "-o", out, os.path.join(HERE, "sanitize_driver.c"),
           os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

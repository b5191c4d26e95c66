"""Builds tests/c_abi/prune_from_c: a C99 program that drives one prune step
through the C ABI (libtri.so) and checks it against the oracle's C library.
Test infrastructure; run by __graft_entry__.build() after both libraries are
built.  The binary finds both libraries next to their sources through an
rpath relative to itself."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "prune_from_c.c")
BINARY = os.path.join(HERE, "prune_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "rope_aware_eviction_amd")
    orc = os.path.join(ROOT, "oracle")
    tmp = BINARY + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           "-o", tmp, SOURCE,
           "-L" + pkg, "-l:libtri.so", "-L" + orc, "-l:libtri_oracle.so",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../rope_aware_eviction_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("gcc failed building the C ABI test program")
    os.replace(tmp, BINARY)
    return BINARY


if __name__ == "__main__":
    print(build(verbose=True))

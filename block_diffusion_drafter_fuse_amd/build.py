"""Build the gfx950 shared library `libdflash_fuse.so` in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "dflash.hip")
LIB = os.path.join(HERE, "libdflash_fuse.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build_library(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to `out` (default: in-tree); `defines` are extra
    -D options (tuning sweeps build variants outside the tree)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[f"-D{x}" for x in defines], "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msg)
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))

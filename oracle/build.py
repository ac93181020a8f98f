"""Build liboracle.so from sgqa_oracle.c with the host C compiler (test infrastructure only)."""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "sgqa_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    # -ffp-contract=off: every product and sum is rounded as written (no fused multiply-add).
    # -fno-semantic-interposition: calls to the exported bf16 helpers inside the library may be
    # inlined (with -fPIC they would otherwise go through the PLT); the arithmetic is unchanged.
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-semantic-interposition",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build ``lib/libspecfold_correction.so`` from ``correction.hip`` with the library's flags."""

from __future__ import annotations

import os
import sys

from sparse_layer_rho_amd.build import ARCH, FLAGS, _hipcc, _run

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libspecfold_correction.so")


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), *FLAGS, "-I", HERE, "-shared", "-o", tmp, os.path.join(HERE, "correction.hip")]
    assert f"--offload-arch={ARCH}" in cmd
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

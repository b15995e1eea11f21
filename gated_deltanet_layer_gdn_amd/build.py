"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_deltanet_layer_gdn_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "conv.hip", "decode.hip", "prep.hip", "prefill.hip"]
HEADERS = ["gdn_device.h", "gdn_internal.h"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libgdn.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = SO + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))

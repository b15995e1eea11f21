"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_deltanet_layer_gdn_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "conv.hip", "decode.hip", "prep.hip", "prefill.hip", "epilogue.hip", "proj.hip", "attn.hip"]
HEADERS = ["gdn_device.h", "gdn_internal.h"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
    "-fvisibility=hidden",
]
OBJ_DIR = os.path.join(HERE, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and err:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc per source, in parallel) and link
    libgdn.so (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [["hipcc", *FLAGS, "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0") or 0) or os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = SO + ".tmp"
    _run(["hipcc", *FLAGS, "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))

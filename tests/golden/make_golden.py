"""Write tests/golden/tiny_layer_oracle.txt from the fp64 oracle alone.

The pages print no worked example for the GDN layer, so this fixture is not a
value from them: it freezes the oracle's answer on the tiny fp32 workload
(B=1, T=64, 2 key / 2 value heads, d=16, seed 0) so that any later change to
the oracle's arithmetic shows up as a failing test and has to be argued for.
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from gdn_inputs import workload_inputs  # noqa: E402

EPS = 1e-6
ROWS = (0, 1, 2, 31, 63)


def compute():
    wl, I = workload_inputs(0)
    g = wl.geom
    y, S, _ = oracle.layer(I["x"], I["z"], I["g"], I["beta"], I["w"], I["hist"], I["S"],
                           H_k=g.H_k, H_v=g.H_v, d_k=g.d_k, d_v=g.d_v, eps=EPS)
    vals = {}
    for t in ROWS:
        for h in range(g.H_v):
            vals[f"y[0,{t},{h},:]"] = y[0, t, h]
    for h in range(g.H_v):
        vals[f"S[0,{h},0,:]"] = S[0, h, 0]
        vals[f"|S[0,{h}]|_F"] = np.array([np.linalg.norm(S[0, h])])
    return vals


def main():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer_oracle.txt")
    with open(path, "w") as f:
        f.write("# fp64 oracle, tiny fp32 GDN layer (seed 0, eps 1e-6, q_scale 1); "
                "written by tests/golden/make_golden.py\n")
        for k, v in compute().items():
            f.write(k + " " + " ".join(repr(float(a)) for a in v) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

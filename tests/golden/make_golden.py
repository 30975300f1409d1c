"""Write tests/golden/tiny_oracle.json: the oracle's outputs for the tiny workload
(N=2, C=3, H=W=8, K=4, R=S=3, pad 1, stride 1; x, W, dy uniform[-1,1] with seeds
101, 102, 103).  Calls only oracle/ and the seeded input generators; it guards the
oracle and the generators against unnoticed changes.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import WORKLOADS, inputs  # noqa: E402


def main():
    wl = WORKLOADS["tiny"]
    s = wl.shape
    t = inputs(wl, "f32")
    x, w, dy = (t[k].numpy() for k in ("x", "w", "dy"))
    y = oracle.conv2d_fwd(x, w, s.pad, s.stride)
    dx = oracle.conv2d_bwd_data(dy, w, (s.H, s.W), s.pad, s.stride)
    dw = oracle.conv2d_bwd_filter(x, dy, (s.R, s.S), s.pad, s.stride)
    out = {
        "_about": "oracle outputs for the tiny workload; written by tests/golden/make_golden.py",
        "shape": list(s.args13()),
        "y": [float(v) for v in y.ravel()],
        "dx": [float(v) for v in dx.ravel()],
        "dw": [float(v) for v in dw.ravel()],
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()

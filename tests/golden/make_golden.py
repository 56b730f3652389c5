"""Writes tiny_oracle.json: sampled outputs of the fp64 oracle on the seeded
tiny workload (B=1, H=2, N=256, d=R=16, M=16, W=4, fp32 storage, seed 0).

The pages print no worked example of the mixer, so this fixture is a
regression guard on the oracle itself: it is written by this script, which
calls only the oracle and the seeded input generator, and a test checks that
the oracle still reproduces it.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as WL  # noqa: E402

POSITIONS = [0, 1, 2, 3, 63, 64, 127, 200, 255]


def main():
    c = WL.make_case("tiny")
    o, st, tl = oracle.forward(c.q, c.k, c.v, c.params)
    out = {
        "workload": "tiny: B=1 H=2 N=256 d=R=16 M=16 W=4 f32 seed=0",
        "eps_feat": 1e-6,
        "eps_norm": 1e-6,
        "positions": POSITIONS,
        "o": {str(i): o[0, i].tolist() for i in POSITIONS},
        "state_out_mode0_head0_re": st[0, 0, 0].real.tolist(),
        "state_out_mode5_head1_im": st[0, 1, 5].imag.tolist(),
        "o_rms": float(np.sqrt((o ** 2).mean())),
    }
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()

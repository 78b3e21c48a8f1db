"""Write tests/golden/bob_n6_d4.json: a small oracle case kept as a regression fixture.

The pages print no worked numeric example, so this fixture is not a pin of the
oracle against the pages: it freezes the oracle's fp64 output on one tiny input
so that any later change to the oracle's arithmetic shows up as a diff of this
file, which then has to be justified by a passage of the pages.  Calls only oracle/.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import bob, forward  # noqa: E402


def main():
    rng = np.random.default_rng(20260921)
    N, d, tau = 6, 4, 0.5
    t = {k: np.round(rng.standard_normal((N, d)), 3)
         for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV")}
    O, L, D = forward(t["Q"], t["K"], t["V"], t["dO"], tau)
    out = bob(t["Q"], t["K"], t["V"], t["dO"], t["UQ"], t["UK"], t["UV"], tau)
    doc = {
        "about": "oracle regression fixture (not from the pages); N=6 d=4 tau=0.5, non-causal",
        "tau": tau,
        "inputs": {k: v.tolist() for k, v in t.items()},
        "forward": {"O": O.tolist(), "L": L.tolist(), "D": D.tolist()},
        "bob": {k: v.tolist() for k, v in out.items()},
    }
    with open(os.path.join(HERE, "bob_n6_d4.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()

"""Write robertson_target.json: the state at t = 1e5 of the Robertson system at
the nominal rates k = (0.04, 3e7, 1e4), y0 = (1, 0, 0), solved by the oracle
(Rosenbrock23, rtol 1e-6, atol 1e-10).  It is the target of the Robertson
ensemble's squared-error loss; only the oracle is called.

Run from the repository root:  python tests/golden/make_robertson_target.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), "..", ".."))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

k = np.array([[0.04], [3e7], [1e4]])
y0 = np.array([[1.0], [0.0], [0.0]])
r = oracle.solve("robertson", "rosenbrock23", k, y0, 0.0, 1e5, 1e-6, 1e-10, s_cap=20000)
assert r["status"][0] == 0
out = {"y": [float(v) for v in r["y1"][:, 0]], "accepted_steps": int(r["count"][0]),
       "source": "oracle Rosenbrock23 solve at nominal rates, t = 1e5, rtol 1e-6, atol 1e-10"}
with open(os.path.join(ROOT, "tests", "golden", "robertson_target.json"), "w") as f:
    json.dump(out, f, indent=1)
print(out)

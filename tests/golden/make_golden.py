"""Write oracle_tiny.json: a tiny fwd+bwd case computed by the fp64 oracle.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def case():
    rng = np.random.default_rng(1234)
    B, T, H, dk, dv = 1, 9, 2, 3, 2
    q = np.round(rng.standard_normal((B, T, H, dk)), 3)
    k = np.round(rng.standard_normal((B, T, H, dk)), 3)
    v = np.round(rng.standard_normal((B, T, H, dv)), 3)
    g = np.round(-rng.uniform(0, 0.5, (B, T, H)), 3)
    beta = np.round(rng.uniform(0, 1, (B, T, H)), 3)
    h0 = np.round(rng.standard_normal((B, H, dk, dv)), 3)
    do = np.round(rng.standard_normal((B, T, H, dv)), 3)
    dht = np.round(rng.standard_normal((B, H, dk, dv)), 3)
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, do=do, dht=dht, scale=0.5)


def main():
    c = case()
    o, ht = oracle.fwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["h0"], scale=c["scale"])
    grads = oracle.bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], c["h0"], c["dht"],
                       scale=c["scale"])
    out = {key: (val.tolist() if isinstance(val, np.ndarray) else val) for key, val in c.items()}
    out["expected"] = {"o": o.tolist(), "ht": ht.tolist()}
    for name, val in zip("dq dk dv dg dbeta dh0".split(), grads):
        out["expected"][name] = val.tolist()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()

"""Write ``oracle_regression.json``: small seeded inputs and the oracle's outputs.

This script calls only ``oracle/``.  The fixture is a regression pin: it
detects any later change in the oracle's arithmetic.  It is not an
independent pin (the explainer pages print no worked numeric example; the
independent pins are the closed forms and forward-view sums in the tests).

Run from the repository root:  python tests/golden/make_regression.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402


def main():
    g = np.random.Generator(np.random.PCG64(2024))
    N, T = 3, 8
    inp = {
        "r": g.standard_normal((N, T)).round(3),
        "v": g.standard_normal((N, T + 1)).round(3),
        "q": g.standard_normal((N, T)).round(3),
        "eq": g.standard_normal((N, T)).round(3),
        "lr": (g.standard_normal((N, T)) * 0.5).round(3),
        "tv": g.standard_normal((N, T)).round(3),
        "B": g.standard_normal(N).round(3),
        "term": (g.random((N, T)) < 0.2).astype(np.uint8),
        "trunc": (g.random((N, T)) < 0.2).astype(np.uint8),
    }
    p = {"gamma": 0.9, "lam": 0.8, "rho_bar": 1.0, "c_bar": 0.95, "pg_rho_bar": 1.2}
    out = {}
    out["returns"] = oracle.returns(inp["r"], inp["term"], inp["trunc"], inp["tv"], inp["B"],
                                    gamma=p["gamma"])
    out["adv"], out["tgt"] = oracle.gae(inp["r"], inp["v"], inp["term"], inp["trunc"], inp["tv"],
                                        gamma=p["gamma"], lam=p["lam"])
    out["td_lambda"] = oracle.td_lambda(inp["r"], inp["v"], inp["term"], inp["trunc"], inp["tv"],
                                        gamma=p["gamma"], lam=p["lam"])
    out["vs"], out["pg"] = oracle.vtrace(inp["r"], inp["v"], inp["lr"], inp["term"], inp["trunc"],
                                         inp["tv"], gamma=p["gamma"], lam=p["lam"],
                                         rho_bar=p["rho_bar"], c_bar=p["c_bar"],
                                         pg_rho_bar=p["pg_rho_bar"])
    out["qret"] = oracle.retrace(inp["r"], inp["q"], inp["eq"], inp["lr"], inp["term"],
                                 inp["trunc"], gamma=p["gamma"], lam=p["lam"], c_bar=p["c_bar"])
    out["eligibility"] = oracle.eligibility_trace(inp["r"], inp["term"], inp["trunc"], inp["B"],
                                                  gamma=p["gamma"], lam=p["lam"])
    out["cumsum"] = oracle.episodic_cumsum(inp["r"], inp["term"], inp["trunc"], inp["B"])
    doc = {
        "about": "Oracle regression fixture written by tests/golden/make_regression.py "
                 "(calls only oracle/). Not an independent pin.",
        "params": p,
        "inputs": {k: v.tolist() for k, v in inp.items()},
        "outputs": {k: [[float.hex(float(x)) for x in row] for row in v] for k, v in out.items()},
    }
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()

"""Write tests/golden/oracle_small_case.json from the float64 oracle (and nothing else).

The pages print no worked numerical example, so this fixture is a regression
record of the oracle itself on one small seeded case: B=1, T=5, H=1, d_k=3,
d_v=2, nonzero S0 and dS_final. Run from the repository root:

    python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def case():
    rng = np.random.default_rng(2026)
    B, T, H, Dk, Dv = 1, 5, 1, 3, 2
    inp = {
        "q": rng.standard_normal((B, T, H, Dk)),
        "k": rng.standard_normal((B, T, H, Dk)) * 0.7,
        "v": rng.standard_normal((B, T, H, Dv)),
        "log_alpha": -np.log1p(np.exp(rng.standard_normal((B, T, H, Dk)) - 1.0)),
        "b": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, Dk)))),
        "w": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, Dv)))),
        "S0": rng.standard_normal((B, H, Dk, Dv)) * 0.5,
        "dO": rng.standard_normal((B, T, H, Dv)),
        "dS_final": rng.standard_normal((B, H, Dk, Dv)),
    }
    return inp


def main():
    inp = case()
    o, ST = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    g = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"], inp["dO"],
                        inp["dS_final"], checkpoint_every=2)
    out = {"source": "tests/golden/make_golden.py (float64 oracle only)",
           "inputs": {k: v.tolist() for k, v in inp.items()},
           "outputs": {"o": o.tolist(), "S_T": ST.tolist(), **{k: v.tolist() for k, v in g.items()}}}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_case.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()

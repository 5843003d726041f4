"""Writes tests/golden/tiny_gma.json -- a regression lock of the fp64 oracle.

The pages (arXiv 2606.18283 summaries) print no worked numerical example of the
forward mixer, so no stored value here is the pages'.  Every expected value in
the fixture is written by this script, which calls only ``oracle/``; the
inputs are drawn from a fixed numpy seed.  The fixture pins the oracle against
accidental change and gives the GPU tests a tiny hand-checkable case.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(20260609)
    B, H, N, dr, dv, K = 1, 2, 6, 2, 3, 3
    # values rounded to bf16-exact binary fractions so the same inputs are exact in f32 and bf16
    def q(x):
        return np.round(np.asarray(x) * 16.0) / 16.0
    case = {
        "qr": q(rng.normal(size=(B, H, N, dr))), "kr": q(rng.normal(size=(B, H, N, dr))),
        "v": q(rng.normal(size=(B, H, N, dv))), "mu": q(rng.normal(size=(H, K, dr))),
        "var_raw": q(0.5 * rng.normal(size=(H, K, dr))), "prior_logits": q(rng.normal(size=(H, K))),
    }
    eps, floor = 1e-6, 1e-3
    fixture = {
        "source": "oracle/ (fp64), written by tests/golden/make_golden.py; the pages print no "
                  "worked example. Method: Gaussian Mixture Attention, arXiv 2606.18283, "
                  "Core mechanism items 1-3 (GMM posterior responsibilities, write/read, "
                  "causal prefix sums).",
        "eps": eps, "var_floor": floor,
        "inputs": {k: v.tolist() for k, v in case.items()},
    }
    for causal in (False, True):
        out, gq, gk = oracle.forward(case["qr"], case["kr"], case["v"], case["mu"],
                                     case["var_raw"], case["prior_logits"], causal, eps, floor,
                                     return_gamma=True)
        key = "causal" if causal else "bidirectional"
        fixture[key] = {"out": out.tolist(), "gamma_q": gq.tolist(), "gamma_k": gk.tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_gma.json")
    with open(path, "w") as f:
        json.dump(fixture, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

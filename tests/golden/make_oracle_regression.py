"""Writes oracle_regression_tiny.txt: sampled outputs of the fp64 oracle on a
small seeded case.  Calls nothing but ``oracle`` and the seeded input
generators.  The file guards the oracle against unnoticed drift; it is not a pin
(a pin compares the oracle with something independent of it).

    python tests/golden/make_oracle_regression.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "oracle_regression_tiny.txt")
# (b, t, h, j) sample points of o and (b, h, c, j) of the final state
O_POINTS = [(0, t, h, j) for t in (0, 1, 63, 64, 65, 129, 199) for h in (0, 1) for j in (0, 17, 63)]
S_POINTS = [(0, h, c, j) for h in (0, 1) for c in (0, 31, 63) for j in (0, 40, 63)]


def compute():
    inp = W.make_inputs(W.TINY_FP32, T=200)
    # a nonzero initial state exercises the carried-in term too
    g = np.random.default_rng(11)
    s0 = g.standard_normal((1, 2, 64, 64)) * 0.05
    o, s = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], s0)
    return s0, o, s


def main():
    _, o, s = compute()
    with open(OUT, "w") as f:
        f.write("# fp64 oracle, workload tiny_fp32 (seed 0) cut to T=200, initial state "
                "0.05 * N(0,1) from numpy default_rng(11); written by make_oracle_regression.py\n")
        for p in O_POINTS:
            f.write("o %d %d %d %d %.17e\n" % (p + (o[p],)))
        for p in S_POINTS:
            f.write("S %d %d %d %d %.17e\n" % (p + (s[p],)))
    print("wrote", OUT)


if __name__ == "__main__":
    main()

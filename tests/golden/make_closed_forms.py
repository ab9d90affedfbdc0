"""Writes the closed-form attention fixtures in this folder.

Uses only Python's ``math``: every expected value below is a hand-derived
formula (stated in each fixture's ``derivation``), not the output of the
oracle or of the GPU library. The pages print no worked numeric example, so
these closed forms stand in for one. Softmax-weighted averaging of values and
log-sum-exp are the definition being pinned (XY-Serve review, "What carries
the argument": the matmul-softmax-matmul pattern; "Assumptions & free
parameters": online softmax equals standard softmax).
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def write(name, fx):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(fx, f, indent=1)
        f.write("\n")


def main():
    e = math.e
    write("two_keys_logistic.json", dict(
        derivation="scores s0 = q.k0 = 0 and s1 = q.k1 = 1 (scale 1); weights 1/(1+e) and "
                   "e/(1+e); values are unit vectors so the output is the weight vector; "
                   "lse = ln(e^0 + e^1) = ln(1+e).",
        head_dim=2, scale=1.0, query=[1.0, 0.0], keys=[[0.0, 0.0], [1.0, 0.0]],
        values=[[1.0, 0.0], [0.0, 1.0]],
        expected_output=[1.0 / (1.0 + e), e / (1.0 + e)], expected_lse=math.log(1.0 + e),
        tolerance=1e-15))
    write("equal_scores_mean.json", dict(
        derivation="q = 0 gives equal scores 0, weights 1/3 each: output = mean of the three "
                   "value rows = (4, 5, 19/3); lse = ln 3.",
        head_dim=3, scale=0.5, query=[0.0, 0.0, 0.0],
        keys=[[1.5, -2.0, 0.25], [3.0, 1.0, -1.0], [-0.5, 0.75, 2.0]],
        values=[[1.0, 2.0, 3.0], [4.0, 5.0, 6.0], [7.0, 8.0, 10.0]],
        expected_output=[4.0, 5.0, 19.0 / 3.0], expected_lse=math.log(3.0), tolerance=1e-15))
    # 18 keys: keys 0..16 score 0, key 17 (block 1, slot 1) scores 2; only key 17 carries value 1.
    keys = [[0.0]] * 17 + [[2.0]]
    vals = [[0.0]] * 17 + [[1.0]]
    write("block_edge_one_hot.json", dict(
        derivation="d = 1, q = 1, scale 1. Keys 0..16 score 0 and key 17 (second block, slot 1) "
                   "scores 2, so its weight is e^2 / (17 + e^2); it is the only non-zero value, "
                   "so the output equals that weight. lse = ln(17 + e^2).",
        head_dim=1, scale=1.0, query=[1.0], keys=keys, values=vals,
        expected_output=[e ** 2 / (17.0 + e ** 2)], expected_lse=math.log(17.0 + e ** 2),
        tolerance=1e-15))


if __name__ == "__main__":
    main()

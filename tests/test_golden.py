"""The oracle against the hand-derived worked example in tests/golden/.

The values in worked_example.txt were derived on paper from the method's
definition (see the comments in that file); this test only parses them.
"""
import os

import numpy as np
import pytest

import oracle
from tests.helpers import problem

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cases(path):
    cases, cur = {}, None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = cases.setdefault(line[1:-1], {})
                continue
            key, val = line.split(":", 1)
            cur[key.strip()] = [[float(x) for x in row.split()] for row in val.split(";")]
    return cases


CASES = _cases(os.path.join(HERE, "worked_example.txt"))


@pytest.mark.parametrize("name", sorted(CASES))
def test_oracle_matches_worked_example(name):
    c = CASES[name]
    T = int(c["q_len"][0][0])
    L = int(c["seq_len"][0][0])
    K = int(c["top_k"][0][0])
    q_idx = np.array(c["q_idx"], np.float32).reshape(1, T, -1, 2)
    head_w = np.array(c["head_w"], np.float32).reshape(1, T, -1)
    k_idx = np.array(c["k_idx"], np.float32).reshape(1, L, -1)
    q = np.array(c["q"], np.float32).reshape(1, T, 1, -1)
    kv = np.array(c["kv"], np.float32).reshape(1, L, -1)
    w = problem(q_idx, head_w, k_idx, q=q, kv=kv, seq_lens=[L], top_k=K, v_dim=1, softmax_scale=1.0)
    r = oracle.forward(w)
    want_scores = np.array(c["scores"], np.float64).reshape(1, T, L)
    vis = ~np.isnan(want_scores)
    assert np.array_equal(np.isnan(r["scores"]), ~vis)
    assert np.array_equal(r["scores"][vis], want_scores[vis])
    assert np.array_equal(r["idx"], np.array(c["topk"], np.int64).reshape(1, T, K))
    assert np.array_equal(r["count"], np.array(c["count"], np.int64).reshape(1, T))
    np.testing.assert_allclose(r["out"].reshape(-1), np.array(c["out"]).reshape(-1), rtol=1e-7, atol=0)
    np.testing.assert_allclose(r["lse"].reshape(-1), np.array(c["lse"]).reshape(-1), rtol=1e-7, atol=0)

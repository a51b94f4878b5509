"""The oracle still reproduces its stored regression fixtures (tests/golden)."""
import os

import numpy as np

import oracle
import workloads

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    rows = []
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            if line.startswith("#"):
                continue
            rows.append([float(x) for x in line.split()])
    return np.array(rows)


def test_golden_W_reproduced():
    W = oracle.draw_w(1002, 16, 16).astype(np.float32)
    np.testing.assert_array_equal(W, _load("tiny_f32_W.txt").astype(np.float32))


def test_golden_outputs_reproduced():
    w = workloads.workload("tiny_f32")
    W = _load("tiny_f32_W.txt").astype(np.float32).astype(np.float64)
    Q, K, V = (t.double().numpy()[0, 0] for t in workloads.host_qkv(w))
    for name, fn in (("bidir", oracle.bidir), ("causal", oracle.causal)):
        g = _load(f"tiny_f32_{name}_rows.txt")
        out = fn(Q, K, V, W)
        rows = g[:, 0].astype(int)
        np.testing.assert_allclose(out[rows], g[:, 1:], rtol=1e-13, atol=1e-15)

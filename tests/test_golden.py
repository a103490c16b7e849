"""The oracle still reproduces the stored tiny-workload fixture (drift check)."""
import json
import os

import numpy as np

import datagen
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_fixture():
    with open(os.path.join(HERE, "golden", "tiny_fp32_oracle.json")) as f:
        g = json.load(f)
    inp = datagen.make(0)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    assert r.n_valid == g["n_valid"] == 461
    assert abs(r.loss - g["loss"]) <= 1e-13 * abs(g["loss"])
    assert np.allclose(r.lse[:8], g["lse_first8"], rtol=1e-13, atol=0)
    assert np.allclose(r.dX[0, :8], g["dX_row0_first8"], rtol=1e-11, atol=1e-18)
    assert np.allclose(r.dW[0, :8], g["dW_row0_first8"], rtol=1e-11, atol=1e-18)
    assert abs(abs(r.dX).sum() - g["dX_abs_sum"]) <= 1e-12 * g["dX_abs_sum"]
    assert abs(abs(r.dW).sum() - g["dW_abs_sum"]) <= 1e-12 * g["dW_abs_sum"]

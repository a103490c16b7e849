"""Write tests/golden/tiny_fp32_oracle.json from the fp64 oracle only.

The pages print no numeric worked example for the loss, so this fixture does
not pin the oracle to the pages; it records the oracle's output on the tiny
fp32 workload (512 tokens, H = 128, V = 256, seed 20260) so that any later
change to the oracle's arithmetic shows up as a diff.  Run from the
repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import oracle   # noqa: E402


def main():
    inp = datagen.make(0)
    r = oracle.flce(inp.X_f64(), inp.W_f64(), inp.labels)
    out = {
        "workload": "tiny-fp32 N=512 H=128 V=256 seed=20260",
        "source": "oracle.flce (fp64), written by tests/golden/make_golden.py",
        "loss": r.loss,
        "n_valid": r.n_valid,
        "lse_first8": r.lse[:8].tolist(),
        "dX_row0_first8": r.dX[0, :8].tolist(),
        "dW_row0_first8": r.dW[0, :8].tolist(),
        "dX_abs_sum": float(abs(r.dX).sum()),
        "dW_abs_sum": float(abs(r.dW).sum()),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()

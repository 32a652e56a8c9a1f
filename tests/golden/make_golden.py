"""Write the oracle regression fixture for the tiny workload.

Calls only the oracle (and the shared seeded input generator).  The pages print
no worked numerical example for the mLSTM cell, so the stored values are the
oracle's own, kept to catch unintended changes to its arithmetic; they are not
an independent pin (the pins in ``tests/oracle_pins.py`` are).
Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from mlstm_matrix_memory_amd import inputs  # noqa: E402

SAMPLES = [(0, 0, t, r) for t, r in [(0, 0), (1, 3), (5, 7), (15, 15), (16, 0), (31, 9), (47, 2), (63, 15)]]


def main():
    w = inputs.WORKLOADS["tiny"]
    x = inputs.fwd_inputs(w)
    h, C, n, m = oracle.fwd(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    out = {
        "workload": "tiny (B=1, NH=1, S=64, d_qk=d_v=16, fp32, seed 1)",
        "source": "oracle/mlstm_oracle.c via tests/golden/make_golden.py",
        "h_samples": [[list(ix), float(h[ix])] for ix in SAMPLES],
        "h_sum": float(h.sum()),
        "h_abs_sum": float(np.abs(h).sum()),
        "C_sum": float(C.sum()),
        "C_00": float(C[0, 0, 0, 0]),
        "n_sum": float(n.sum()),
        "m": float(m[0, 0]),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

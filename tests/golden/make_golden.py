"""Write the stored oracle outputs used as regression fixtures.

Calls only the fp64 oracle and the seeded input generator; no value here comes
from the HIP library. Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from non_linear_matrix_amd.inputs import CONFIGS, generate  # noqa: E402
from oracle import m2rnn_fwd_ref  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def write(name, cfg, seed):
    x = generate(cfg, seed)
    y, HT = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype)
    path = os.path.join(HERE, name)
    with open(path, "w") as fh:
        fh.write(f"# fp64 oracle output, workload {cfg.name} seed {seed}: "
                 f"B={cfg.B} H={cfg.H} K={cfg.K} V={cfg.V} T={cfg.T} dtype={cfg.dtype}\n")
        fh.write("# update: gist.science M2RNN technical summary (zh) 2.1 state-update equations;"
                 " readout y_t = H_t^T q_t (documented reading)\n")
        fh.write(f"y {' '.join(str(d) for d in y.shape)}\n")
        for val in y.reshape(-1):
            fh.write(f"{val:.17e}\n")
        fh.write(f"H_T {' '.join(str(d) for d in HT.shape)}\n")
        for val in HT.reshape(-1):
            fh.write(f"{val:.17e}\n")


if __name__ == "__main__":
    write("c1_seed0.txt", CONFIGS["C1"], 0)

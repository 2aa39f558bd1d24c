"""Write the oracle's golden fixtures (calls only oracle/ and the seeded input
generator).  Re-run only when the oracle's arithmetic changes for a reason the
pages justify; the commit that changes a fixture must name that reason.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from gated_delta_rule_87_amd.inputs import WORKLOADS, decoded, make_inputs  # noqa: E402
from oracle.recurrence import recurrence_c  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    w = WORKLOADS[0]
    x = decoded(make_inputs(w))
    o, hT = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], nthreads=4)
    rng = np.random.default_rng(0)
    idx = [tuple(int(i) for i in (rng.integers(w.B), rng.integers(w.T), rng.integers(w.H_v),
                                   rng.integers(w.d_v))) for _ in range(32)]
    fixture = {
        "what": "fp64 token-recurrence oracle on the scalar-gate fp32 workload "
                "(B1 T256 H2 d64), seeded inputs; sampled o entries and norms",
        "source": "Systolic Linear Attention, section 2.1, Eq. (2); written by tests/golden/make_golden.py",
        "workload": w.name,
        "seed": w.seed,
        "o_samples": [[list(i), float(o[i])] for i in idx],
        "o_rms": float(np.sqrt(np.mean(o ** 2))),
        "o_absmax": float(np.max(np.abs(o))),
        "hT_fro": [[float(np.linalg.norm(hT[b, h])) for h in range(w.H_v)] for b in range(w.B)],
    }
    with open(os.path.join(HERE, "oracle_gdn_f32_tiny.json"), "w") as f:
        json.dump(fixture, f, indent=1)


if __name__ == "__main__":
    main()

"""The oracle against its stored golden fixture (regression pin, no GPU).

The fixture was written by tests/golden/make_golden.py from the oracle alone;
agreement also pins the seeded input generator's draw order."""
import json
import os

import numpy as np

from gated_delta_rule_87_amd.inputs import WORKLOADS, decoded, make_inputs
from oracle.recurrence import recurrence_c, recurrence_np

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_golden():
    with open(os.path.join(HERE, "golden", "oracle_gdn_f32_tiny.json")) as f:
        fx = json.load(f)
    w = WORKLOADS[0]
    assert fx["seed"] == w.seed
    x = decoded(make_inputs(w))
    for impl in (lambda *a: recurrence_c(*a, nthreads=2), recurrence_np):
        o, hT = impl(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"])
        for idx, val in fx["o_samples"]:
            assert abs(o[tuple(idx)] - val) <= 1e-12
        assert abs(np.sqrt(np.mean(o ** 2)) - fx["o_rms"]) <= 1e-12
        assert abs(np.max(np.abs(o)) - fx["o_absmax"]) <= 1e-12
        for b, row in enumerate(fx["hT_fro"]):
            for h, val in enumerate(row):
                assert abs(np.linalg.norm(hT[b, h]) - val) <= 1e-11

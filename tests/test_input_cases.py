"""Properties of the GPU test inputs themselves (CPU only).

The prep stage takes one of two routes per chunk: a chunk-wide pivot when no
log alpha of the chunk is positive and the chunk's total decay
-Lambda_{C-1} = -sum(log alpha) is at most 64 in every decay group, 16-token
block pivots otherwise.  The mixed-range cases must hold chunks of both kinds
in one launch, or they would not test the hand-off between the two kernels.
"""
import numpy as np
import pytest

from gated_delta_rule_87_amd.inputs import decode, make_inputs
from test_gpu_fullsize import MIXED_LONG
from test_gpu_parity import MIXED, SMALL

PIVOT_RANGE = 64.0


def wide_fraction(w):
    """Fraction of (batch, key head, chunk) items that need block pivots: a
    positive log alpha, or a total decay beyond the limit in some decay group
    (rows past T are zero log-decay)."""
    la = decode(make_inputs(w)["log_alpha"]).astype(np.float64)   # [B, T, H_k, G]
    B, T, H, G = la.shape
    C = w.chunk
    nc = -(-T // C)
    pad = np.zeros((B, nc * C, H, G))
    pad[:, :T] = la
    chunks = pad.reshape(B, nc, C, H, G)
    wide = ((-chunks.sum(axis=2) > PIVOT_RANGE) | (chunks > 0).any(axis=2)).any(axis=-1)
    return float(wide.mean())


@pytest.mark.parametrize("name", MIXED)
def test_mixed_cases_hold_both_chunk_kinds(name):
    f = wide_fraction(SMALL[name])
    assert 0.0 < f < 1.0, f


def test_long_mixed_case_holds_both_chunk_kinds():
    f = wide_fraction(MIXED_LONG)
    assert 0.2 < f < 0.8, f


def test_mild_decay_workloads_take_the_chunk_pivot():
    # the scalar and per-channel workloads at C = 64 never need block pivots
    for name in ("gdn_bf16", "kda_bf16", "gva_g4_bf16", "dk256_kda_bf16"):
        assert wide_fraction(SMALL[name]) == 0.0, name

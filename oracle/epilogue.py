"""Output epilogue of the SLA layer in fp64 -- TEST INFRASTRUCTURE ONLY.

"Systolic Linear Attention: Co-Designing Tile-Grouped Gated Delta Attention
for TPUs", section 2.3 (the token-level recurrence box): each value head's
readout is normalised on its own and gated by the sigmoid of the output-gate
slice of that head,

    y_{t,m} = sigmoid(z_{t,m}) (.) RMSNorm(o_{t,m}),
    RMSNorm(x) = x / sqrt(mean_i x_i^2 + eps) (.) w,

the mean running over the d_v entries of one value head.  The pages give no
epsilon and no scale vector; this build takes a caller-given eps and an
optional per-channel scale w of length d_v shared by all heads (w = 1 when
absent).
"""
import numpy as np


def gated_rmsnorm(o, z, weight=None, eps=1e-6):
    """o, z: [..., d_v] (any leading shape); weight: [d_v] or None.
    Returns y in float64."""
    o = np.asarray(o, np.float64)
    z = np.asarray(z, np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    w = 1.0 if weight is None else np.asarray(weight, np.float64)
    return (1.0 / (1.0 + np.exp(-z))) * (o / rms) * w

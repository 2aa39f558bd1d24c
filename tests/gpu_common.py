"""Shared helpers for the GPU tests (helper module, not collected)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd.inputs import decoded, make_inputs

# Tolerance on max |o_gpu - o_ref| / rms(o_ref) (and the same for hT):
# 1e-2 for bf16 inputs, 1e-4 for fp32 inputs.
TOL = {"bf16": 1e-2, "f32": 1e-4}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def to_torch(arr, device="cuda"):
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr.astype(np.float32, copy=False)).to(device)


def device_inputs(raw, device="cuda"):
    return {n: to_torch(a, device) for n, a in raw.items()}


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / rms) if ref.size else 0.0


def draw(w, **kw):
    raw = make_inputs(w, **kw)
    return raw, decoded(raw)


def run_chunk(dev, w, h0=None, solve="exact", **kw):
    return_state = kw.pop("return_final_state", True)
    o, hT = __import__("gated_delta_rule_87_amd.binding", fromlist=["x"]).gdr_chunk_fwd(
        dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], h0, chunk=w.chunk, solve=solve,
        neumann_order=w.neumann_order, neumann_residual_steps=w.neumann_residual,
        return_final_state=return_state, **kw)
    return o, hT

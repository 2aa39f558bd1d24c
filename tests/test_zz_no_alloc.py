"""gdr_chunk_fwd_noalloc (the entry point for callers that cannot allocate)
against gdr_chunk_fwd through the C ABI: the same kernels over the library's
static per-device scratch instead of a workspace.  Two calls in a row, the
second on a smaller problem (the scratch keeps the first call's bytes), each
equal to gdr_chunk_fwd bit for bit and within the parity bar of the fp64
oracle; a problem beyond the scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import Workload
from gpu_common import TOL, device_inputs, draw, need_gpu, rel_err, run_chunk
from oracle.recurrence import recurrence_c

pytestmark = pytest.mark.gpu

FIRST = Workload("noalloc_kda", 2, 1000, 4, 4, 128, 128, 64, 128, "bf16", beta_scale=2.0, seed=201)
SECOND = Workload("noalloc_small", 1, 300, 2, 4, 128, 64, 128, 128, "bf16", alpha_mu=1.0, alpha_sigma=2.0,
                  beta_per_key_head=True, seed=202)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def call_noalloc(dev, w, h0, o, hT):
    lib = gb.load()
    p = gb.make_problem(dev["q"], dev["v"], dev["log_alpha"], dev["beta"], chunk=w.chunk, out_dtype=o.dtype)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gdr_chunk_fwd_noalloc(ctypes.byref(p), _ptr(dev["q"]), _ptr(dev["k"]), _ptr(dev["v"]),
                                     _ptr(dev["beta"]), _ptr(dev["log_alpha"]), _ptr(h0), _ptr(o), _ptr(hT),
                                     stream), p


def test_noalloc_matches_chunk_fwd_twice():
    need_gpu()
    for w in (FIRST, SECOND):
        raw, x = draw(w)
        dev = device_inputs(raw)
        h0 = torch.randn(w.B, w.H_v, w.d_k, w.d_v, device="cuda") if w is SECOND else None
        print(f"[case] noalloc {w.name}", flush=True)
        o_ref, h_ref = run_chunk(dev, w, h0=h0)
        o = torch.full_like(o_ref, float("nan"))
        hT = torch.full_like(h_ref, float("nan"))
        status, p = call_noalloc(dev, w, h0, o, hT)
        assert status == gb.GDR_OK, gb.last_error()
        assert gb.gdr_chunk_fwd_workspace_size(p) <= gb.NOALLOC_SCRATCH_BYTES
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
        o64, h64 = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"],
                                None if h0 is None else h0.cpu().numpy().astype(np.float64), w.beta_per_key_head)
        eo, eh = rel_err(o.cpu().numpy(), o64), rel_err(hT.cpu().numpy(), h64)
        print(f"  identical to gdr_chunk_fwd; vs oracle o={eo:.3e} hT={eh:.3e}", flush=True)
        assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


def test_noalloc_refuses_problems_beyond_its_scratch():
    """Host-side check: the per-channel workload at B2 T8192 H32 needs a
    541 MB workspace, beyond the 128 MiB scratch."""
    p = gb.GdrProblem()
    for name, val in dict(B=2, T=8192, H_k=32, H_v=32, d_k=128, d_v=128, chunk=64, gate_groups=128,
                          beta_per_key_head=0, in_dtype=gb.GDR_BF16, out_dtype=gb.GDR_F32, solve=0,
                          neumann_order=4, neumann_residual_steps=1).items():
        setattr(p, name, val)
    assert gb.gdr_chunk_fwd_workspace_size(p) > gb.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    status = gb.load().gdr_chunk_fwd_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, None, fake, None, None)
    assert status == gb.GDR_ERR_UNSUPPORTED
    assert "scratch" in gb.last_error()

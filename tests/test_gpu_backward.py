"""Training forward and backward pass on the GPU against the fp64 oracle
(Systolic Linear Attention, section 2.5: custom VJP that keeps S_{c-1} and
recomputes the chunk quantities).

* gdr_chunk_fwd_train: o and hT bit-identical to gdr_chunk_fwd; the saved
  chunk-entry states (fp16 for bf16 inputs, fp32 for fp32 inputs) equal the
  oracle's state after c chunks (fp64 chunk form on the first c C tokens)
  within the forward's bars, and the first is h0 rounded to that type.
* gdr_chunk_bwd: every gradient (dq, dk, dv, dbeta, dlog_alpha, dh0) against
  the fp64 reverse-mode gradient of the token recurrence itself
  (oracle.backward.vjp_autograd).  Statistic: max |g_gpu - g_ref| / rms(g_ref)
  per gradient.  Bars: the forward's, 1e-4 for fp32 inputs (every product in
  fp32) and 1e-2 for bf16 inputs (the prep's and reverse scan's operand tiles
  are fp16, 11 significant bits, as in the forward; the gradient kernel
  multiplies fp16 operands for bf16 inputs and fp32 ones for fp32 inputs).
  Measured: at most 4e-5 (fp32) and 4.7e-3 (bf16, dlog_alpha).

Cases: scalar, per-channel and four-tile gates; beta per value and per key
head; grouped value heads (H_v = 2 H_k); ragged final chunks; a nonzero h0
and dhT; fp32 and bf16 outputs (d_o in the output's dtype); chunks whose
decay range exceeds the pivot bound (the gradient kernel's entry-by-entry
route) and T = 0.  At the full sizes of the scalar-gate and per-channel
benchmark workloads (the shapes bench.py --train times), sampled (batch,
key head) units are checked against the fp64 chunkwise backward
(oracle.backward.vjp_chunk, pinned to vjp_autograd on the CPU).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import Workload
from gpu_common import TOL, device_inputs, draw, need_gpu, rel_err
from oracle import chunk as och
from oracle.backward import vjp_autograd, vjp_chunk

pytestmark = pytest.mark.gpu

BWD_TOL = TOL

CASES = {
    "gdn_f32": Workload("gdn_f32", 2, 200, 2, 2, 64, 64, 64, 1, "f32", seed=401),
    "kda_f32_gva": Workload("kda_f32_gva", 1, 150, 2, 4, 128, 64, 64, 128, "f32", beta_scale=2.0, seed=402),
    "kda_bf16": Workload("kda_bf16", 2, 300, 2, 2, 128, 128, 64, 128, "bf16", seed=403),
    "sla_bf16_keybeta": Workload("sla_bf16_keybeta", 1, 260, 2, 4, 64, 64, 64, 4, "bf16", beta_per_key_head=True,
                                 beta_scale=2.0, seed=404),
    "kda_f32_strong": Workload("kda_f32_strong", 1, 200, 1, 2, 64, 64, 64, 64, "f32", alpha_mu=-1.0,
                               alpha_sigma=2.0, seed=405),
    "gdn_bf16_strong": Workload("gdn_bf16_strong", 1, 190, 2, 2, 128, 64, 64, 1, "bf16", alpha_mu=-2.0,
                                alpha_sigma=1.0, seed=406),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _normal(shape, seed, scale=1.0):
    return (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)


def _rounded(x, dtype):
    """x (fp32 numpy) on the GPU in `dtype`, and the exact fp64 value it holds."""
    t = torch.from_numpy(x).cuda().to(dtype).contiguous()
    return t, t.float().cpu().numpy().astype(np.float64)


def _run(w, out_dtype=torch.float32, with_h0=True, with_dhT=True):
    raw, dec = draw(w)
    dev = device_inputs(raw)
    B, T = w.B, w.T
    sshape = (B, w.H_v, w.d_k, w.d_v)
    h0 = _normal(sshape, w.seed + 1, 0.5) if with_h0 else None
    dhT = _normal(sshape, w.seed + 2, 0.5) if with_dhT else None
    d_o_t, d_o = _rounded(_normal((B, T, w.H_v, w.d_v), w.seed + 3), out_dtype)
    h0_t = torch.from_numpy(h0).cuda() if with_h0 else None
    dhT_t = torch.from_numpy(dhT).cuda() if with_dhT else None
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"])
    o, hT, states = gb.gdr_chunk_fwd_train(*args, h0_t, chunk=w.chunk, out_dtype=out_dtype)
    g = gb.gdr_chunk_bwd(*args, states, d_o_t, dhT_t, chunk=w.chunk)
    torch.cuda.synchronize()
    return raw, dec, dev, h0, dhT, d_o, (o, hT, states), g


def _ref(w, dec, h0, dhT, d_o):
    return vjp_autograd(dec["q"], dec["k"], dec["v"], dec["beta"], dec["log_alpha"], h0, d_o, dhT,
                        beta_per_key_head=w.beta_per_key_head)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    w = CASES[name]
    print(f"case {name}", flush=True)
    raw, dec, dev, h0, dhT, d_o, fwd, g = _run(w)
    ref = _ref(w, dec, h0, dhT, d_o)
    tol = BWD_TOL[w.dtype]
    errs = {n: rel_err(g[n].cpu().numpy(), ref[n]) for n in ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dh0")}
    print(name, {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= tol, f"{name} {n}: {e:.3e} > {tol}"


@pytest.mark.parametrize("name", ["kda_bf16", "gdn_f32"])
def test_backward_bf16_output_and_zero_state(name):
    """d_o in bf16 (an fp32 or bf16 forward output's gradient), no h0 and no dhT."""
    w = CASES[name]
    print(f"case {name} bf16 out", flush=True)
    raw, dec, dev, h0, dhT, d_o, fwd, g = _run(w, out_dtype=torch.bfloat16, with_h0=False, with_dhT=False)
    ref = _ref(w, dec, None, None, d_o)
    tol = BWD_TOL[w.dtype]
    for n in ("dq", "dk", "dv", "dbeta", "dlog_alpha"):
        e = rel_err(g[n].cpu().numpy(), ref[n])
        assert e <= tol, f"{name} {n}: {e:.3e} > {tol}"
    # without h0 the gradient of the initial state is still defined (S_0 = 0)
    ref_h = _ref(w, dec, np.zeros((w.B, w.H_v, w.d_k, w.d_v)), None, d_o)
    assert rel_err(g["dh0"].cpu().numpy(), ref_h["dh0"]) <= tol


@pytest.mark.parametrize("name", ["kda_f32_gva", "sla_bf16_keybeta", "kda_f32_strong"])
def test_training_forward_states(name):
    w = CASES[name]
    print(f"case {name} states", flush=True)
    raw, dec, dev, h0, dhT, d_o, (o, hT, states), g = _run(w)
    o2, hT2 = gb.gdr_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"],
                               torch.from_numpy(h0).cuda(), chunk=w.chunk)
    assert torch.equal(o, o2) and torch.equal(hT, hT2)
    st = states.float().cpu().numpy()
    nc = -(-w.T // w.chunk)
    assert st.shape == (w.B, w.H_v, nc, w.d_k, w.d_v)
    # fp16 for bf16 inputs (the precision the gradient kernel multiplies in)
    assert states.dtype == (torch.float16 if w.dtype == "bf16" else torch.float32)
    assert np.array_equal(st[:, :, 0], torch.from_numpy(h0).to(states.dtype).float().numpy())
    for c in sorted({1, nc // 2, nc - 1}):
        if c < 1:
            continue
        n = c * w.chunk
        cut = {k_: dec[k_][:, :n] for k_ in ("q", "k", "v", "beta", "log_alpha")}
        _, ref = och.chunk_forward(cut["q"], cut["k"], cut["v"], cut["beta"], cut["log_alpha"], h0, chunk=w.chunk,
                                   beta_per_key_head=w.beta_per_key_head)
        assert rel_err(st[:, :, c], ref) <= TOL[w.dtype], f"state entering chunk {c}"


def test_backward_no_tokens():
    """T = 0: dh0 = dhT and nothing else is touched."""
    w = CASES["gdn_f32"].with_(T=0)
    q = torch.zeros((1, 0, 2, 64), device="cuda")
    v = torch.zeros((1, 0, 2, 64), device="cuda")
    beta = torch.zeros((1, 0, 2), device="cuda")
    la = torch.zeros((1, 0, 2, 1), device="cuda")
    states = torch.zeros((1, 2, 0, 64, 64), device="cuda")
    dhT = torch.from_numpy(_normal((1, 2, 64, 64), 9)).cuda()
    g = gb.gdr_chunk_bwd(q, q, v, beta, la, states, v, dhT, chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dhT)


def test_backward_rejects_unsupported():
    w = CASES["gdn_f32"]
    raw, dec = draw(w.with_(T=64))
    dev = device_inputs(raw)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"])
    with pytest.raises(gb.GdrError, match="UNSUPPORTED"):
        gb.gdr_chunk_fwd_train(*args, chunk=128)
    p = gb.make_problem(dev["q"], dev["v"], dev["log_alpha"], dev["beta"], solve="neumann")
    assert gb.gdr_chunk_bwd_workspace_size(p) == 0
    assert gb.gdr_chunk_states_size(p) == 0


FULL_UNITS = {1: [(0, 0), (3, 15)], 2: [(0, 0), (1, 17), (1, 31)]}


@pytest.mark.parametrize("cfg", sorted(FULL_UNITS))
def test_backward_full_size_sampled(cfg):
    from gated_delta_rule_87_amd.inputs import WORKLOADS
    w = WORKLOADS[cfg]
    print(f"case full-size backward {w.name}", flush=True)
    raw, dec = draw(w)
    dev = device_inputs(raw)
    d_o = _normal((w.B, w.T, w.H_v, w.d_v), w.seed + 3)
    args = (dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"])
    o, hT, states = gb.gdr_chunk_fwd_train(*args, chunk=w.chunk)
    g = gb.gdr_chunk_bwd(*args, states, torch.from_numpy(d_o).cuda(), None, chunk=w.chunk)
    torch.cuda.synchronize()
    R = w.H_v // w.H_k
    for b, hk in FULL_UNITS[cfg]:
        hv = slice(hk * R, hk * R + R)
        sk = lambda a: a[b:b + 1, :, hk:hk + 1]
        sv = lambda a: a[b:b + 1, :, hv]
        ref = vjp_chunk(sk(dec["q"]), sk(dec["k"]), sv(dec["v"]), sv(dec["beta"]), sk(dec["log_alpha"]), None,
                        sv(d_o), None, chunk=w.chunk)
        got = {"dq": g["dq"][b:b + 1, :, hk:hk + 1], "dk": g["dk"][b:b + 1, :, hk:hk + 1],
               "dv": g["dv"][b:b + 1, :, hv], "dbeta": g["dbeta"][b:b + 1, :, hv],
               "dlog_alpha": g["dlog_alpha"][b:b + 1, :, hk:hk + 1]}
        errs = {n: rel_err(t.cpu().numpy(), ref[n]) for n, t in got.items()}
        print(f"  unit b={b} hk={hk}", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
        for n, e in errs.items():
            assert e <= BWD_TOL[w.dtype], f"{w.name} b={b} hk={hk} {n}: {e:.3e}"

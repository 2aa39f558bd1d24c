"""The segment-parallel scan (used when the (batch, value head, 32-column)
units cannot fill the GPU: the sequence is cut into segments whose affine
maps S -> J S + B are composed, Systolic Linear Attention section 3.3)
against the fp64 oracle.  Every case here has fewer than 256 units and at
least 18 chunks, so the library splits it (into 3 to 10 segments); together
they cover both transfer-pass tile widths (64 columns at C = 64 and 128 with
d_k <= 128 or C = 64 with d_k = 256; 32 columns otherwise and for fp32),
ragged final chunks, a nonzero h0, per-key-head beta up to 2, document
resets and the Neumann mode.  Bars as everywhere: max |x_gpu - x_ref| /
rms(x_ref) <= 1e-2 (bf16 inputs) / 1e-4 (fp32 inputs), for o and hT.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import Workload, make_resets
from gpu_common import TOL, device_inputs, draw, need_gpu, rel_err, run_chunk, to_torch
from oracle import chunk as och
from oracle.recurrence import layer_c, recurrence_c

pytestmark = pytest.mark.gpu

SEG = {
    "kda_c64": Workload("kda_c64", 1, 3000, 2, 2, 128, 64, 64, 128, "bf16", seed=401),
    "sla_c64_dk256": Workload("sla_c64_dk256", 1, 2100, 1, 4, 256, 128, 64, 4, "bf16", beta_scale=2.0, seed=402),
    "sla_c128_bkh": Workload("sla_c128_bkh", 1, 4100, 2, 8, 256, 64, 128, 4, "bf16", beta_per_key_head=True,
                             beta_scale=2.0, seed=403),
    "kda_c128_strong": Workload("kda_c128_strong", 1, 3000, 2, 2, 128, 128, 128, 128, "bf16", alpha_mu=1.0,
                                alpha_sigma=2.0, seed=404),
    "kda_c64_mixed": Workload("kda_c64_mixed", 2, 2500, 2, 2, 128, 64, 64, 128, "bf16", alpha_mu=0.75,
                              alpha_sigma=2.0, seed=405),
    "gdn_f32": Workload("gdn_f32", 2, 2500, 2, 2, 64, 64, 64, 1, "f32", seed=406),
    "kda_c32": Workload("kda_c32", 1, 2000, 2, 2, 128, 64, 32, 128, "bf16", seed=412),
    # chunk 16: the padded sequence (3008 tokens at chunk 32) is split too
    "kda_c16": Workload("kda_c16", 1, 1500, 2, 2, 128, 64, 16, 128, "bf16", seed=413),
    "kda_f32_c128": Workload("kda_f32_c128", 1, 2200, 2, 2, 128, 64, 128, 128, "f32", seed=407),
    # long memory (log alpha = logsigmoid(N(7, 1)), about -1e-3 per token):
    # each segment's transition J stays of order 1, so the composed entry
    # states carry real weight (with the decays above J underflows to 0)
    "kda_c64_longmem": Workload("kda_c64_longmem", 1, 3000, 2, 2, 128, 64, 64, 128, "bf16", alpha_mu=7.0,
                                seed=408),
    "sla_c128_longmem": Workload("sla_c128_longmem", 1, 4100, 2, 8, 256, 64, 128, 4, "bf16",
                                 beta_per_key_head=True, beta_scale=2.0, alpha_mu=7.0, seed=409),
    "gdn_f32_longmem": Workload("gdn_f32_longmem", 2, 2500, 2, 2, 64, 64, 64, 1, "f32", alpha_mu=7.0, seed=410),
    "kda_c128_longmem": Workload("kda_c128_longmem", 1, 2200, 2, 2, 128, 128, 128, 128, "bf16", alpha_mu=7.0,
                                 seed=411),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def h0_for(w):
    """An initial state of the magnitude the inputs' own states reach (entries
    of about 0.2): the state's per-chunk operand copy is fp16, so the output
    error of the first tokens scales with |h0|, and an h0 far larger than the
    states the inputs produce would be measured against an output rms that
    the inputs set."""
    return 0.2 * np.random.default_rng(w.seed).standard_normal((w.B, w.H_v, w.d_k, w.d_v)).astype(np.float32)


@pytest.mark.parametrize("name", sorted(SEG))
def test_segmented_exact(name):
    w = SEG[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    h0 = h0_for(w)
    units = w.B * w.H_v * (w.d_v // 32)
    print(f"[case] segmented {name}: {units} units of 32 columns, {-(-w.T // w.chunk)} chunks", flush=True)
    assert units < 256 and w.T >= 16 * w.chunk
    o, hT = run_chunk(dev, w, h0=to_torch(h0))
    torch.cuda.synchronize()
    o_ref, h_ref = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], h0.astype(np.float64),
                                w.beta_per_key_head)
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(hT.cpu().numpy(), h_ref)
    print(f"  err o={eo:.3e} hT={eh:.3e}", flush=True)
    assert np.all(np.isfinite(o.cpu().numpy()))
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["kda_c128_strong", "sla_c128_bkh", "gdn_f32", "kda_c128_longmem"])
def test_segmented_neumann(name):
    w = SEG[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] segmented neumann {name}", flush=True)
    o, hT = run_chunk(dev, w, solve="neumann")
    o_n, h_n = och.chunk_forward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], chunk=w.chunk,
                                 solve="neumann", order=w.neumann_order, residual_steps=w.neumann_residual,
                                 beta_per_key_head=w.beta_per_key_head)
    eo, eh = rel_err(o.cpu().numpy(), o_n), rel_err(hT.cpu().numpy(), h_n)
    print(f"  err vs neumann chunk form o={eo:.3e} hT={eh:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["kda_c64", "sla_c128_bkh", "gdn_f32", "kda_c64_longmem", "sla_c128_longmem"])
def test_segmented_with_resets(name):
    """Document resets inside segments and on segment edges: a reset makes a
    segment's transition J zero from there on."""
    w = SEG[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    rs = make_resets(w.B, w.T, 700, seed=w.seed + 7, extra=[(0, 0), (0, 10 * w.chunk), (w.B - 1, 8 * w.chunk + 3)])
    h0 = h0_for(w)
    print(f"[case] segmented with resets {name}: documents={int(rs.sum())}", flush=True)
    o, hT = gb.gdr_chunk_fwd_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], to_torch(h0),
                                reset=torch.from_numpy(rs).cuda(), chunk=w.chunk)
    o_ref, h_ref, _ = layer_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], h0.astype(np.float64),
                              w.beta_per_key_head, reset=rs)
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(hT.cpu().numpy(), h_ref)
    print(f"  err o={eo:.3e} hT={eh:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["kda_c64_longmem", "gdn_f32_longmem"])
def test_segment_transitions_carry_weight(name):
    """The long-memory cases really exercise the composition: the entry
    state handed to the last segment differs from the one a run of the last
    segment alone from zero would use by a large fraction of its size, so a
    wrong J would fail the parity test above."""
    w = SEG[name]
    raw, x = draw(w)
    T = w.T
    cut = (T // w.chunk // 2) * w.chunk
    sl = lambda a: np.ascontiguousarray(a[:, cut:])
    o_full, _ = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"])
    o_tail, _ = recurrence_c(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["log_alpha"]))
    d = rel_err(o_tail, o_full[:, cut:])
    print(f"[case] {name}: output of the second half with and without the first half's state differs by {d:.2f}",
          flush=True)
    assert d > 0.1


def test_segmented_is_deterministic_and_hT_may_alias_h0():
    w = SEG["kda_c64"]
    raw, _ = draw(w)
    dev = device_inputs(raw)
    h0 = to_torch(h0_for(w))
    o1, h1 = run_chunk(dev, w, h0=h0.clone())
    buf = h0.clone()
    o2, h2 = run_chunk(dev, w, h0=buf, hT=buf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, buf)

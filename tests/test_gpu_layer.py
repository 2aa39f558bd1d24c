"""The SLA layer semantics on the GPU against the fp64 oracle: document
resets, chunk-boundary momentum (Systolic Linear Attention, Table 2: Z_c,
mu = 0.25, kappa_c; section 2.3) and the gated RMSNorm epilogue (section 2.3,
token-level recurrence box), through gdr_chunk_fwd_ex and gdr_gated_rmsnorm.

Statistic: max |x_gpu - x_ref| / rms(x_ref) for o, hT and the momentum
buffer zT; bars 1e-2 (bf16 inputs) and 1e-4 (fp32 inputs).  The exact mode
is held to the token recurrence with resets and momentum (oracle.recurrence
.layer_c); the Neumann mode to the fp64 chunk form with the same series and
the same resets.  Resets fall on token 0, on chunk edges, inside chunks and
twice in one 16-token block, in chunks of both prep routes.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import WORKLOADS, Workload, make_resets
from gpu_common import TOL, decode_workspace, device_inputs, draw, need_gpu, rel_err, to_torch
from oracle import chunk as och
from oracle.epilogue import gated_rmsnorm
from oracle.recurrence import layer_c

pytestmark = pytest.mark.gpu

LAYER = {
    "kda_c64": Workload("kda_c64", 2, 700, 2, 2, 128, 64, 64, 128, "bf16", beta_scale=2.0, seed=301),
    "kda_c64_mixed": Workload("kda_c64_mixed", 1, 650, 2, 2, 128, 64, 64, 128, "bf16", alpha_mu=0.75,
                              alpha_sigma=2.0, seed=302),
    "sla_c64": Workload("sla_c64", 1, 600, 2, 8, 256, 64, 64, 4, "bf16", beta_per_key_head=True, beta_scale=2.0,
                        seed=303),
    "sla_c128": Workload("sla_c128", 1, 600, 2, 8, 256, 64, 128, 4, "bf16", beta_per_key_head=True,
                         beta_scale=2.0, seed=304),
    "kda_c128_strong": Workload("kda_c128_strong", 1, 700, 2, 2, 128, 128, 128, 128, "bf16", alpha_mu=1.0,
                                alpha_sigma=2.0, seed=305),
    "gdn_f32": Workload("gdn_f32", 2, 300, 2, 2, 64, 64, 64, 1, "f32", seed=306),
    "kda_c32": Workload("kda_c32", 2, 700, 2, 2, 128, 64, 32, 128, "bf16", beta_scale=2.0, seed=308),
    "kda_c16": Workload("kda_c16", 2, 500, 2, 2, 128, 64, 16, 128, "bf16", beta_scale=2.0, seed=309),
    "kda_f32_c128": Workload("kda_f32_c128", 1, 333, 2, 4, 128, 32, 128, 128, "f32", beta_scale=2.0, seed=307),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def resets_for(w):
    C = w.chunk
    extra = [(0, 0), (0, C), (0, 2 * C + 5), (0, 2 * C + 9), (w.B - 1, 3 * C - 1), (w.B - 1, 4 * C + 17)]
    return make_resets(w.B, w.T, 150, seed=w.seed + 1000, extra=extra)


def dev_bytes(rs):
    return torch.from_numpy(np.ascontiguousarray(rs, dtype=np.uint8)).cuda()


def state(w, seed):
    return np.random.default_rng(seed).standard_normal((w.B, w.H_v, w.d_k, w.d_v)).astype(np.float32)


def run_ex(dev, w, rs, mu, h0=None, z0=None, solve="exact"):
    return gb.gdr_chunk_fwd_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"],
                               None if h0 is None else to_torch(h0), reset=dev_bytes(rs),
                               momentum=mu, z0=None if z0 is None else to_torch(z0), return_momentum_state=True,
                               chunk=w.chunk, solve=solve, neumann_order=w.neumann_order,
                               neumann_residual_steps=w.neumann_residual)


@pytest.mark.parametrize("mu", [0.0, 0.25], ids=["resets", "resets_momentum"])
@pytest.mark.parametrize("name", sorted(LAYER))
def test_layer_exact(name, mu):
    w = LAYER[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    rs = resets_for(w)
    h0, z0 = state(w, 1), state(w, 2)
    print(f"[case] layer exact {name} mu={mu} documents started={int(rs.sum())}", flush=True)
    o, hT, zT = run_ex(dev, w, rs, mu, h0, z0)
    torch.cuda.synchronize()
    o_ref, h_ref, z_ref = layer_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], h0.astype(np.float64),
                                  w.beta_per_key_head, reset=rs, momentum=mu, chunk=w.chunk,
                                  z0=z0.astype(np.float64))
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(hT.cpu().numpy(), h_ref)
    ez = rel_err(zT.cpu().numpy(), z_ref) if mu else 0.0
    print(f"  err o={eo:.3e} hT={eh:.3e} zT={ez:.3e}", flush=True)
    assert np.all(np.isfinite(o.cpu().numpy()))
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype] and ez <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["kda_c64_mixed", "sla_c128", "kda_c128_strong", "kda_f32_c128", "kda_c16"])
def test_layer_neumann(name):
    w = LAYER[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    rs = resets_for(w)
    print(f"[case] layer neumann {name}", flush=True)
    o, hT, zT = run_ex(dev, w, rs, 0.25, solve="neumann")
    o_n, h_n, z_n = och.chunk_forward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], chunk=w.chunk,
                                      solve="neumann", order=w.neumann_order, residual_steps=w.neumann_residual,
                                      beta_per_key_head=w.beta_per_key_head, reset=rs, momentum=0.25,
                                      return_z=True)
    eo, eh, ez = rel_err(o.cpu().numpy(), o_n), rel_err(hT.cpu().numpy(), h_n), rel_err(zT.cpu().numpy(), z_n)
    print(f"  err vs neumann chunk form o={eo:.3e} hT={eh:.3e} zT={ez:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype] and ez <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["kda_c64", "sla_c128", "gdn_f32"])
def test_prepared_workspace_with_resets(name):
    """The prepared chunks of chunks holding resets against the fp64 chunk
    pieces with segment masks; their decay row is -0 in every channel."""
    w = LAYER[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    rs = resets_for(w)
    print(f"[case] prepared with resets {name}", flush=True)
    p = gb.make_problem(dev["q"], dev["v"], dev["log_alpha"], dev["beta"], chunk=w.chunk)
    ws = torch.empty(gb.gdr_chunk_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    gb.gdr_chunk_fwd_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], reset=dev_bytes(rs),
                        chunk=w.chunk, workspace=ws)
    got = decode_workspace(ws, p)
    B, T, Hk, dk = x["q"].shape
    C, nc = w.chunk, -(-w.T // w.chunk)
    Hb = x["beta"].shape[2]
    R = Hb // Hk
    ref = {n: np.zeros_like(got[n]) for n in got}
    has_reset = np.zeros((B, nc), bool)
    for b in range(B):
        for hk in range(Hk):
            qh = np.asarray(x["q"][b, :, hk], np.float64)
            kh = np.asarray(x["k"][b, :, hk], np.float64)
            la = np.repeat(np.asarray(x["log_alpha"][b, :, hk], np.float64), dk // w.G, axis=1)
            for c in range(nc):
                s, e = c * C, min(c * C + C, T)
                n = e - s
                has_reset[b, c] = rs[b, s:e].any()
                pc = och.chunk_pieces(qh[s:e], kh[s:e], np.ones(n), la[s:e], rs[b, s:e])
                ref["L"][b, hk, c, :n, :n] = pc["L"]
                ref["KB"][b, hk, c, :n] = pc["Kbar"]
                ref["QB"][b, hk, c, :n] = pc["Qbar"]
                ref["KH"][b, hk, c, :, :n] = pc["Khat"].T
                ref["GM"][b, hk, c] = pc["gamma"]
                for hb in range(hk * R, (hk + 1) * R):
                    bh = np.asarray(x["beta"][b, s:e, hb], np.float64)
                    A = np.linalg.inv(np.eye(n) + pc["G"] * bh[None, :])
                    ref["A"][b, hb, c, :n, :n] = bh[:, None] * A
    f32 = w.dtype == "f32"
    for key in ("A", "L", "KB", "QB", "KH", "GM"):
        # decay rows are at most 1, and all zero when every chunk holds a reset
        scale = max(np.max(np.abs(ref[key])), 1.0) if key == "GM" else np.max(np.abs(ref[key]))
        err = np.max(np.abs(got[key] - ref[key])) / scale
        bar = 1e-5 if (f32 or key == "GM") else 1e-3
        print(f"  {key}: max err / max ref = {err:.3e} (bar {bar:g})", flush=True)
        assert err <= bar, key
    gm_raw = got["GM"]
    for b in range(B):
        for c in range(nc):
            assert np.all(np.signbit(gm_raw[b, :, c])) == has_reset[b, c], (b, c)
    assert has_reset.any()


def test_momentum_resume_at_chunk_boundary_is_exact():
    """Splitting the sequence at a multiple of the chunk and resuming from
    (hT, zT) reproduces the single run bit for bit."""
    w = LAYER["kda_c64"]
    raw, _ = draw(w)
    dev = device_inputs(raw)
    rs = dev_bytes(resets_for(w))
    o, hT, zT = gb.gdr_chunk_fwd_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], reset=rs,
                                    momentum=0.25, return_momentum_state=True, chunk=w.chunk)
    cut = 4 * w.chunk
    a = {n: t[:, :cut].contiguous() for n, t in dev.items()}
    b = {n: t[:, cut:].contiguous() for n, t in dev.items()}
    oa, ha, za = gb.gdr_chunk_fwd_ex(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"],
                                     reset=rs[:, :cut].contiguous(), momentum=0.25, return_momentum_state=True,
                                     chunk=w.chunk)
    ob, hb, zb = gb.gdr_chunk_fwd_ex(b["q"], b["k"], b["v"], b["beta"], b["log_alpha"], ha,
                                     reset=rs[:, cut:].contiguous(), momentum=0.25, z0=za,
                                     return_momentum_state=True, chunk=w.chunk)
    assert torch.equal(torch.cat([oa, ob], 1), o) and torch.equal(hb, hT) and torch.equal(zb, zT)


def test_no_resets_and_zero_momentum_match_plain_forward():
    w = LAYER["sla_c64"]
    raw, _ = draw(w)
    dev = device_inputs(raw)
    o1, h1 = gb.gdr_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], chunk=w.chunk)
    o2, h2 = gb.gdr_chunk_fwd_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], chunk=w.chunk)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


# ------------------------------------------------------------------ epilogue
@pytest.mark.parametrize("o_dtype,z_dtype", [(torch.float32, torch.bfloat16), (torch.float32, torch.float32),
                                             (torch.bfloat16, torch.bfloat16)])
@pytest.mark.parametrize("d_v", [128, 48])
def test_gated_rmsnorm(o_dtype, z_dtype, d_v):
    g = torch.Generator(device="cpu").manual_seed(d_v)
    o = (torch.randn(2, 37, 3, d_v, generator=g) * 3.0).to(o_dtype).cuda()
    z = torch.randn(2, 37, 3, d_v, generator=g).to(z_dtype).cuda()
    wt = torch.rand(d_v, generator=g).cuda() + 0.5
    print(f"[case] gated rmsnorm o {o_dtype} z {z_dtype} d_v {d_v}", flush=True)
    y = gb.gdr_gated_rmsnorm(o, z, weight=wt, eps=1e-5)
    ref = gated_rmsnorm(o.float().cpu().numpy(), z.float().cpu().numpy(), wt.cpu().numpy(), eps=1e-5)
    bar = 1e-5 if o_dtype == torch.float32 else 2.0 ** -8 * float(np.max(np.abs(ref)) / np.sqrt(np.mean(ref ** 2)))
    err = rel_err(y.float().cpu().numpy(), ref)
    print(f"  err y={err:.3e} (bar {bar:.2e})", flush=True)
    assert err <= bar
    y2 = gb.gdr_gated_rmsnorm(o.clone(), z, eps=1e-5)
    o_in = o.clone()
    gb.gdr_gated_rmsnorm(o_in, z, eps=1e-5, y=o_in)              # in place
    torch.cuda.synchronize()
    assert torch.equal(o_in, y2)


def test_sla_layer_full_size():
    """The widened-key grouped-value workload (B2 T16384, 8 key heads d_k 256,
    32 value heads d_v 128, G = 4, C = 64) as an SLA layer: beta = 2 sigmoid
    per key head, packed documents of mean length 3000, mu = 0.25, then the
    gated RMSNorm epilogue; eight (batch, value head) units over the whole
    sequence against the oracle."""
    w = WORKLOADS[3].with_(beta_scale=2.0, beta_per_key_head=True)
    raw, x = draw(w)
    dev = device_inputs(raw)
    rs = make_resets(w.B, w.T, 3000, seed=777, extra=[(0, 0), (1, 8 * w.chunk)])
    zg = np.random.default_rng(5).standard_normal((w.B, w.T, w.H_v, w.d_v)).astype(np.float32)
    print(f"\n[case] full-size SLA layer {w.name} documents={int(rs.sum())}", flush=True)
    o, hT, zT = gb.gdr_chunk_fwd_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"],
                                    reset=dev_bytes(rs), momentum=0.25, return_momentum_state=True, chunk=w.chunk)
    y = gb.gdr_gated_rmsnorm(o, to_torch(zg).to(torch.bfloat16), eps=1e-6)
    o, hT, zT, y = o.cpu().numpy(), hT.cpu().numpy(), zT.cpu().numpy(), y.cpu().numpy()
    total = w.B * w.H_v
    units = sorted({0, 3, 13, total // 2 - 1, total // 2 + 6, total - 9, total - 2, total - 1})
    o_ref, h_ref, z_ref = layer_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], None, True, reset=rs,
                                  momentum=0.25, chunk=w.chunk, units=units)
    zb = to_torch(zg).to(torch.bfloat16).float().cpu().numpy()      # the gate values the kernel read
    sel = lambda a: np.concatenate([a[u // w.H_v, :, u % w.H_v] for u in units])
    st = lambda a: np.stack([a[u // w.H_v, u % w.H_v] for u in units])
    y_ref = gated_rmsnorm(sel(o_ref), sel(zb), eps=1e-6)
    eo, eh, ez, ey = rel_err(sel(o), sel(o_ref)), rel_err(st(hT), st(h_ref)), rel_err(st(zT), st(z_ref)), \
        rel_err(sel(y), y_ref)
    print(f"  units {units}: err o={eo:.3e} hT={eh:.3e} zT={ez:.3e} y={ey:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert max(eo, eh, ez, ey) <= TOL[w.dtype]

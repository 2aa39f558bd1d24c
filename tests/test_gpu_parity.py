"""GPU path (libgdr.so through the C ABI) against the fp64 CPU oracle.

Statistic: max |x_gpu - x_ref| / rms(x_ref) over all elements, for o and for
hT separately.  Bar: 1e-2 for bf16 inputs, 1e-4 for fp32 inputs.  The oracle
for the exact mode is the token recurrence; for the Neumann mode it is the
fp64 chunk form with the same truncated series (its distance to the exact
recurrence is reported, not bounded).

Sizes here finish in seconds on the CPU side, span several chunks and
16-token tiles, and end in a ragged final chunk.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import Workload
from gpu_common import decode_workspace, TOL, device_inputs, draw, need_gpu, rel_err, run_chunk, to_torch
from oracle import chunk as och
from oracle.recurrence import recurrence_c

pytestmark = pytest.mark.gpu

SMALL = {
    "gdn_f32": Workload("gdn_f32", 2, 300, 2, 2, 64, 64, 64, 1, "f32", seed=1),
    "kda_f32_c128": Workload("kda_f32_c128", 1, 333, 2, 2, 128, 32, 128, 128, "f32", seed=2),
    "gdn_bf16": Workload("gdn_bf16", 2, 300, 2, 2, 128, 128, 64, 1, "bf16", seed=3),
    "kda_bf16": Workload("kda_bf16", 1, 517, 2, 2, 128, 64, 64, 128, "bf16", seed=4),
    "gva_g4_bf16": Workload("gva_g4_bf16", 1, 300, 2, 8, 256, 128, 64, 4, "bf16", seed=5),
    "kda_c128_strong": Workload("kda_c128_strong", 1, 700, 2, 2, 128, 128, 128, 128, "bf16",
                                alpha_mu=1.0, alpha_sigma=2.0, seed=6),
    "dk64_bkh_gva": Workload("dk64_bkh_gva", 2, 190, 2, 4, 64, 48, 64, 8, "bf16", beta_per_key_head=True, seed=7),
    "dk256_kda_bf16": Workload("dk256_kda_bf16", 1, 200, 1, 1, 256, 64, 64, 256, "bf16", seed=8),
    # C = 64 with some chunks whose decay range exceeds the chunk-pivot limit
    # and some within it (both kinds present: test_input_cases.py)
    "kda_c64_mixed": Workload("kda_c64_mixed", 1, 700, 2, 2, 128, 64, 64, 128, "bf16",
                              alpha_mu=0.75, alpha_sigma=2.0, seed=9),
    "gdn_f32_c64_mixed": Workload("gdn_f32_c64_mixed", 2, 450, 2, 2, 64, 64, 64, 1, "f32",
                                  alpha_mu=0.0, alpha_sigma=2.0, seed=10),
    # grouped gates whose 8-channel lanes span 1 group (G = 16) or 2 (G = 32)
    # of a d_k = 128 head, per-key-head beta with grouped value heads, both
    # routes
    "gva_bkh_mixed": Workload("gva_bkh_mixed", 1, 450, 2, 8, 128, 32, 64, 16, "bf16", alpha_mu=0.5,
                              alpha_sigma=2.0, beta_per_key_head=True, seed=13),
    "g32_mixed": Workload("g32_mixed", 2, 333, 2, 2, 128, 48, 64, 32, "bf16", alpha_mu=0.5, alpha_sigma=2.0,
                          seed=14),
    # one token; one ragged chunk with 8 groups of 8 channels
    "t1_bf16": Workload("t1_bf16", 2, 1, 2, 2, 128, 64, 64, 128, "bf16", seed=11),
    "t63_f32_g8": Workload("t63_f32_g8", 1, 63, 2, 2, 64, 32, 64, 8, "f32", seed=12),
    # enough (batch, value head, 32-column) tiles for 32-column scan
    # workgroups (B H_v d_v / 32 >= 256): C = 128 with bf16 inputs, and fp32
    # inputs at C = 64
    "c128_bv32_bf16": Workload("c128_bv32_bf16", 1, 260, 64, 64, 128, 128, 128, 128, "bf16", alpha_mu=2.0,
                               seed=15),
    "f32_bv32": Workload("f32_bv32", 2, 150, 64, 64, 64, 64, 64, 1, "f32", seed=16),
    # chunk 32 (block-pivot route for every chunk, two row blocks per chunk)
    "gdn_f32_c32": Workload("gdn_f32_c32", 2, 300, 2, 2, 64, 64, 32, 1, "f32", seed=31),
    "kda_bf16_c32": Workload("kda_bf16_c32", 1, 517, 2, 2, 128, 64, 32, 128, "bf16", seed=32),
    "sla_c32_bkh": Workload("sla_c32_bkh", 1, 300, 2, 8, 256, 64, 32, 4, "bf16", beta_per_key_head=True,
                            beta_scale=2.0, seed=33),
    "kda_c32_mixed": Workload("kda_c32_mixed", 1, 400, 2, 2, 128, 64, 32, 128, "bf16", alpha_mu=0.0,
                              alpha_sigma=2.0, seed=34),
    # chunk 16: the C = 32 path on the sequence padded with 16 identity tokens
    # after every 16 (ragged tails, fp32 and bf16, d_k = 256 with per-key-head beta)
    "gdn_f32_c16": Workload("gdn_f32_c16", 2, 300, 2, 2, 64, 64, 16, 1, "f32", seed=35),
    "kda_bf16_c16": Workload("kda_bf16_c16", 1, 517, 2, 2, 128, 64, 16, 128, "bf16", seed=36),
    "sla_c16_bkh": Workload("sla_c16_bkh", 1, 250, 2, 8, 256, 64, 16, 4, "bf16", beta_per_key_head=True,
                            beta_scale=2.0, seed=37),
    # chunk 128, d_k <= 128 (eight-wave block-pivot kernel): every log-alpha
    # layout of a lane's eight channels -- at most four groups read as
    # scalars (G = 1, 4), one group per 8-channel vector (G = 16) and two
    # channels per group (G = 32 at d_k = 64) -- and d_k = 64
    "gdn_bf16_c128": Workload("gdn_bf16_c128", 2, 300, 2, 2, 128, 64, 128, 1, "bf16", seed=41),
    "g4_c128_bf16": Workload("g4_c128_bf16", 1, 450, 2, 2, 128, 64, 128, 4, "bf16", alpha_mu=1.0,
                             alpha_sigma=2.0, seed=42),
    "g16_c128_bkh": Workload("g16_c128_bkh", 1, 450, 2, 8, 128, 32, 128, 16, "bf16", alpha_mu=0.5,
                             alpha_sigma=2.0, beta_per_key_head=True, beta_scale=2.0, seed=43),
    "g32_dk64_c128": Workload("g32_dk64_c128", 2, 333, 2, 2, 64, 48, 128, 32, "bf16", seed=44),
    "gdn_f32_c128_dk64": Workload("gdn_f32_c128_dk64", 2, 300, 2, 2, 64, 64, 128, 1, "f32", seed=45),
}

# the cases above with chunks on both sides of the chunk-pivot range limit
MIXED = ("kda_c64_mixed", "gdn_f32_c64_mixed", "gva_bkh_mixed", "g32_mixed")


def oracle(x, w, h0=None, units=None):
    return recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], h0, w.beta_per_key_head,
                        units=units)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    print(f"\n[gpu] {torch.cuda.get_device_name(0)}", flush=True)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_chunk_fwd_small(name):
    w = SMALL[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] chunk_fwd {name}", flush=True)
    o, hT = run_chunk(dev, w)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle(x, w)
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(hT.cpu().numpy(), h_ref)
    print(f"  err o={eo:.3e} hT={eh:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["gdn_f32", "kda_bf16", "dk64_bkh_gva", "kda_bf16_c32", "gdn_f32_c16"])
def test_chunk_fwd_nonzero_h0(name):
    w = SMALL[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    rng = np.random.default_rng(11)
    h0 = rng.standard_normal((w.B, w.H_v, w.d_k, w.d_v)).astype(np.float32)
    print(f"[case] chunk_fwd h0 {name}", flush=True)
    o, hT = run_chunk(dev, w, h0=to_torch(h0))
    o_ref, h_ref = oracle(x, w, h0.astype(np.float64))
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(hT.cpu().numpy(), h_ref)
    print(f"  err o={eo:.3e} hT={eh:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


@pytest.mark.parametrize("name,order,res", [("kda_c128_strong", 4, 1), ("kda_bf16", 2, 1), ("kda_f32_c128", 3, 2),
                                            ("kda_c64_mixed", 3, 1), ("gdn_f32_c64_mixed", 4, 1),
                                            ("gva_g4_bf16", 1, 0), ("kda_bf16_c32", 2, 1), ("gdn_f32_c32", 1, 0),
                                            ("g16_c128_bkh", 2, 1), ("kda_bf16", 2, 2), ("kda_c128_strong", 1, 3),
                                            ("kda_bf16_c32", 0, 2), ("kda_bf16_c16", 2, 1), ("gdn_f32_c16", 3, 1)])
def test_neumann_small(name, order, res):
    w = SMALL[name].with_(neumann_order=order, neumann_residual=res)
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] neumann {name} m={order} r={res}", flush=True)
    o, hT = run_chunk(dev, w, solve="neumann")
    o_n, h_n = och.chunk_forward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], chunk=w.chunk,
                                 solve="neumann", order=order, residual_steps=res,
                                 beta_per_key_head=w.beta_per_key_head)
    o_ref, _ = oracle(x, w)
    eo, eh = rel_err(o.cpu().numpy(), o_n), rel_err(hT.cpu().numpy(), h_n)
    print(f"  err vs neumann oracle o={eo:.3e} hT={eh:.3e}; neumann oracle vs exact recurrence "
          f"{rel_err(o_n, o_ref):.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]


@pytest.mark.parametrize("name,order", [("kda_c128_strong", 1), ("kda_bf16", 1), ("kda_f32_c128", 1),
                                        ("gdn_f32_c64_mixed", 2), ("gva_g4_bf16", 1), ("dk64_bkh_gva", 1),
                                        ("kda_f32_c128", 7), ("gdn_f32", 3), ("kda_bf16_c32", 1), ("sla_c16_bkh", 1),
                                        ("gdn_bf16_c128", 1), ("gdn_f32_c128_dk64", 1)])
def test_block_neumann_small(name, order):
    """SLA section 2.4.3's block-Jacobi Neumann solve (order 1 = 1-Step
    Neumann) against the fp64 chunk form with the same series; at order
    C/16 - 1 the series is complete and matches the exact recurrence too."""
    w = SMALL[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] block_neumann {name} m={order}", flush=True)
    o, hT = gb.gdr_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], chunk=w.chunk,
                             solve="block_neumann", neumann_order=order, neumann_residual_steps=0)
    o_n, h_n = och.chunk_forward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], chunk=w.chunk,
                                 solve="block_neumann", order=order, beta_per_key_head=w.beta_per_key_head)
    o_ref, h_ref = oracle(x, w)
    eo, eh = rel_err(o.cpu().numpy(), o_n), rel_err(hT.cpu().numpy(), h_n)
    print(f"  err vs block-Neumann oracle o={eo:.3e} hT={eh:.3e}; that oracle vs exact recurrence "
          f"{rel_err(o_n, o_ref):.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]
    if order >= w.chunk // 16 - 1:
        assert rel_err(o.cpu().numpy(), o_ref) <= TOL[w.dtype] and rel_err(hT.cpu().numpy(), h_ref) <= TOL[w.dtype]


@pytest.mark.parametrize("name", ["kda_bf16", "gdn_bf16", "f32_bv32", "c128_bv32_bf16", "kda_bf16_c32",
                                  "seg_kda_c64", "kda_bf16_c16"])
def test_chunk_fwd_bf16_output(name):
    """out_dtype bf16 (its own o staging and row pieces, 16- and 32-column scan
    tiles, the segment-parallel scan): o is the fp32-output result rounded once
    to bf16, bit for bit, and hT is unchanged."""
    w = SMALL[name] if name in SMALL else SEG_CASE
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] chunk_fwd bf16 output {name}", flush=True)
    o32, h32 = run_chunk(dev, w)
    o16, h16 = run_chunk(dev, w, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(h16, h32)


# enough chunks and few enough (batch, head) units for the segment-parallel scan
SEG_CASE = Workload("seg_kda_c64", 1, 3000, 2, 2, 128, 64, 64, 128, "bf16", seed=17)


@pytest.mark.parametrize("name", ["kda_bf16", "f32_bv32", "seg_kda_c64", "kda_bf16_c16"])
def test_hT_may_alias_h0(name):
    """gdr.h: hT may alias h0 (each workgroup reads its h0 tile before writing
    its hT tile; the segment-parallel path reads h0 in the combine, before the
    scan writes hT)."""
    w = SMALL[name] if name in SMALL else SEG_CASE
    raw, x = draw(w)
    dev = device_inputs(raw)
    h0 = torch.from_numpy((0.2 * np.random.default_rng(3).standard_normal((w.B, w.H_v, w.d_k, w.d_v)))
                          .astype(np.float32)).cuda()
    print(f"[case] hT aliases h0 {name}", flush=True)
    o1, h1 = run_chunk(dev, w, h0=h0.clone())
    buf = h0.clone()
    o2, h2 = run_chunk(dev, w, h0=buf, hT=buf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, buf) and h2.data_ptr() == buf.data_ptr()


def expected_operands(x, w):
    """The scan operands of every chunk from the fp64 chunk pieces: Kbar,
    Qbar, Khat^T and exp(Lambda_C) per key head, token rows past T zero."""
    B, T, Hk, dk = x["q"].shape
    C = w.chunk
    nc = -(-T // C)
    KB = np.zeros((B, Hk, nc, C, dk)); QB = np.zeros_like(KB)
    KH = np.zeros((B, Hk, nc, dk, C)); GM = np.zeros((B, Hk, nc, dk))
    for b in range(B):
        for hk in range(Hk):
            q = np.asarray(x["q"][b, :, hk], np.float64)
            k = np.asarray(x["k"][b, :, hk], np.float64)
            la = np.repeat(np.asarray(x["log_alpha"][b, :, hk], np.float64), dk // w.G, axis=1)
            for c in range(nc):
                s, e = c * C, min(c * C + C, T)
                pc = och.chunk_pieces(q[s:e], k[s:e], np.ones(e - s), la[s:e])
                KB[b, hk, c, :e - s] = pc["Kbar"]
                QB[b, hk, c, :e - s] = pc["Qbar"]
                KH[b, hk, c, :, :e - s] = pc["Khat"].T
                GM[b, hk, c] = pc["gamma"]
    return {"KB": KB, "QB": QB, "KH": KH, "GM": GM}


@pytest.mark.parametrize("name", ["gdn_f32", "kda_f32_c128", "kda_bf16", "gva_g4_bf16", "kda_c128_strong",
                                  "dk64_bkh_gva", "dk256_kda_bf16", "kda_c64_mixed", "gdn_f32_c64_mixed",
                                  "gva_bkh_mixed", "g32_mixed", "t63_f32_g8", "g16_c128_bkh", "gdn_f32_c128_dk64"])
@pytest.mark.parametrize("solve", ["exact", "neumann"])
def test_prepared_workspace(name, solve):
    """Every prepared chunk quantity against the fp64 chunk pieces: diag(beta)
    A_c, L_c, Kbar, Qbar, Khat^T, exp(Lambda_C).  Bars on max|err| / max|ref|:
    fp16 tiles (bf16 inputs) 1e-3 (one fp16 rounding is 2^-11 relative),
    fp32 tiles and the fp32 gate vector 1e-5."""
    w = SMALL[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] prepare {name} {solve}", flush=True)
    ws, p = gb.gdr_chunk_prepare(dev["q"], dev["k"], dev["beta"], dev["log_alpha"], chunk=w.chunk, solve=solve,
                                 neumann_order=w.neumann_order, neumann_residual_steps=w.neumann_residual,
                                 H_v=w.H_v)
    got = decode_workspace(ws, p)
    A_ref, L_ref = och.chunk_stage_matrices(x["q"], x["k"], x["beta"], x["log_alpha"], w.chunk, solve=solve,
                                            order=w.neumann_order, residual_steps=w.neumann_residual,
                                            beta_per_key_head=w.beta_per_key_head)
    B, T = x["q"].shape[:2]
    C = w.chunk
    nc = A_ref.shape[2]
    beta = np.zeros((B, nc * C, x["beta"].shape[2]))
    beta[:, :T] = x["beta"]
    beta = beta.reshape(B, nc, C, -1).transpose(0, 3, 1, 2)      # [B, H_beta, N_c, C]
    ref = dict(expected_operands(x, w), A=beta[..., None] * A_ref, L=L_ref)
    f32 = w.dtype == "f32"
    for key in ("A", "L", "KB", "QB", "KH", "GM"):
        err = np.max(np.abs(got[key] - ref[key])) / np.max(np.abs(ref[key]))
        bar = 1e-5 if (f32 or key == "GM") else 1e-3
        print(f"  {key}: max err / max ref = {err:.3e} (bar {bar:g})", flush=True)
        assert err <= bar, key


RECUR = {
    "f32_g1": Workload("f32_g1", 2, 37, 2, 2, 64, 32, 64, 1, "f32", seed=21),
    "bf16_kda": Workload("bf16_kda", 1, 50, 2, 4, 128, 64, 64, 128, "bf16", seed=22),
    "bf16_g4_dk256": Workload("bf16_g4_dk256", 1, 20, 1, 2, 256, 128, 64, 4, "bf16", seed=23),
    "bf16_bkh": Workload("bf16_bkh", 2, 9, 2, 4, 64, 16, 64, 64, "bf16", beta_per_key_head=True, seed=24),
}


@pytest.mark.parametrize("name", sorted(RECUR))
def test_recurrent_step(name):
    w = RECUR[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    rng = np.random.default_rng(5)
    s0 = rng.standard_normal((w.B, w.H_v, w.d_k, w.d_v)).astype(np.float32)
    state = to_torch(s0)
    print(f"[case] recurrent {name}", flush=True)
    o = gb.gdr_recurrent_step(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], state)
    o_ref, h_ref = oracle(x, w, s0.astype(np.float64))
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(state.cpu().numpy(), h_ref)
    print(f"  err o={eo:.3e} state={eh:.3e}", flush=True)
    assert eo <= 1e-5 and eh <= 1e-5


@pytest.mark.parametrize("name", ["kda_bf16_c16", "gdn_f32_c16"])
def test_chunk16_prepare_then_scan(name):
    """Chunk 16 through the split entry points: gdr_chunk_prepare pads the
    key side into the workspace, gdr_chunk_scan pads v and gathers o; the
    result equals gdr_chunk_fwd bit for bit."""
    w = SMALL[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    print(f"[case] chunk 16 prepare + scan {name}", flush=True)
    o1, h1 = run_chunk(dev, w)
    ws, _ = gb.gdr_chunk_prepare(dev["q"], dev["k"], dev["beta"], dev["log_alpha"], chunk=16, H_v=w.H_v,
                                 d_v=w.d_v)
    o2, h2 = gb.gdr_chunk_scan(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], None, workspace=ws,
                               chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("T", [0, 5, 16, 17])
def test_chunk16_short_sequences(T):
    """Chunk 16 on sequences shorter than one padded chunk, exactly one chunk
    and one token more: o and hT against the fp64 recurrence; T = 0 copies
    h0 to hT."""
    w = SMALL["gdn_f32_c16"].with_(T=max(T, 1))
    raw, x = draw(w)
    dev = device_inputs(raw)
    h0 = (0.2 * np.random.default_rng(5).standard_normal((w.B, w.H_v, w.d_k, w.d_v))).astype(np.float32)
    print(f"[case] chunk 16 T={T}", flush=True)
    if T == 0:
        dev = {n: t[:, :0].contiguous() for n, t in dev.items()}
        o, hT = run_chunk(dev, w, h0=to_torch(h0))
        torch.cuda.synchronize()
        assert o.numel() == 0 and np.array_equal(hT.cpu().numpy(), h0)
        return
    o, hT = run_chunk(dev, w, h0=to_torch(h0))
    torch.cuda.synchronize()
    o_ref, h_ref = oracle(x, w, h0.astype(np.float64))
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(hT.cpu().numpy(), h_ref)
    print(f"  err o={eo:.3e} hT={eh:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype]

"""The serving path on the GPU against the fp64 oracle: speculative
verification of up to 16 drafted tokens from a state (Systolic Linear
Attention, section 3.2), committing each sequence's accepted prefix with the
recurrent step, document resets in the step, and the row-scaled E4M3 state
(bit-exact conversions; the step over an FP8 state).

Bars: verification and the fp32 step compute in fp32 from exact inputs, so
max |x_gpu - x_ref| / rms(x_ref) <= 1e-5 (as the recurrent step's tests).
E4M3 codes and scales: bit-exact against oracle.fp8 on the same fp32 input.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import Workload, make_resets
from gpu_common import device_inputs, draw, need_gpu, rel_err, to_torch
from oracle.fp8 import dequantize_rows, e4m3_value, quantize_rows
from oracle.recurrence import layer_c, recurrence_c

pytestmark = pytest.mark.gpu

DRAFT = {
    "kda_t16": Workload("kda_t16", 4, 16, 2, 4, 128, 64, 64, 128, "bf16", seed=501),
    "kda_t8_f32": Workload("kda_t8_f32", 3, 8, 2, 2, 128, 128, 64, 128, "f32", seed=502),
    "sla_t16": Workload("sla_t16", 2, 16, 2, 8, 256, 64, 64, 4, "bf16", beta_per_key_head=True, beta_scale=2.0,
                        seed=503),
    "gdn_t5_dk64": Workload("gdn_t5_dk64", 2, 5, 2, 2, 64, 48, 64, 1, "bf16", seed=504),
    "t1": Workload("t1", 2, 1, 2, 2, 128, 32, 64, 128, "bf16", seed=505),
    # strong decay: Lambda spans ~30 over the drafted tokens (first-token
    # pivot with factors up to e^30) ...
    "kda_t16_decay": Workload("kda_t16_decay", 2, 16, 2, 4, 128, 64, 64, 128, "f32", alpha_mu=-1.5,
                              alpha_sigma=1.0, seed=508),
    # ... and ~80, beyond the pivot bound (each pair's exponential on its own)
    "kda_t16_wide": Workload("kda_t16_wide", 2, 16, 2, 4, 64, 64, 64, 64, "bf16", alpha_mu=-5.0,
                             alpha_sigma=1.0, seed=509),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def natural_state(w, seed):
    return (0.2 * np.random.default_rng(seed).standard_normal((w.B, w.H_v, w.d_k, w.d_v))).astype(np.float32)


@pytest.mark.parametrize("name", sorted(DRAFT))
def test_verify(name):
    w = DRAFT[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    s0 = natural_state(w, 1)
    state = to_torch(s0)
    keep = state.clone()
    print(f"[case] verify {name} T={w.T}", flush=True)
    o = gb.gdr_verify(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], state)
    torch.cuda.synchronize()
    assert torch.equal(state, keep)                              # the state is not advanced
    o_ref, _ = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], s0.astype(np.float64),
                            w.beta_per_key_head)
    err = rel_err(o.cpu().numpy(), o_ref)
    print(f"  err o={err:.3e}", flush=True)
    assert err <= 1e-5


def test_verify_bf16_output_and_refusal():
    w = DRAFT["kda_t16"]
    raw, x = draw(w)
    dev = device_inputs(raw)
    s0 = natural_state(w, 2)
    o = gb.gdr_verify(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], to_torch(s0),
                      out_dtype=torch.bfloat16)
    o_ref, _ = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], s0.astype(np.float64))
    bar = 1e-5 + 2.0 ** -8 * float(np.max(np.abs(o_ref)) / np.sqrt(np.mean(o_ref ** 2)))
    assert rel_err(o.float().cpu().numpy(), o_ref) <= bar
    w17 = w.with_(T=17)
    raw17, _ = draw(w17)
    d17 = device_inputs(raw17)
    with pytest.raises(gb.GdrError, match="UNSUPPORTED"):
        gb.gdr_verify(d17["q"], d17["k"], d17["v"], d17["beta"], d17["log_alpha"], to_torch(natural_state(w17, 3)))


@pytest.mark.parametrize("name", ["kda_t16", "sla_t16", "kda_t8_f32"])
def test_speculative_round_trip(name):
    """Verify T drafted tokens, accept a random prefix n_b per sequence, commit
    it with the per-sequence step: the committed state equals the oracle state
    after exactly n_b tokens, and the step's outputs for the accepted tokens
    equal the verified ones; outputs past n_b are not written."""
    w = DRAFT[name]
    raw, x = draw(w)
    dev = device_inputs(raw)
    s0 = natural_state(w, 4)
    state = to_torch(s0)
    o_ver = gb.gdr_verify(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], state)
    n = np.random.default_rng(5).integers(0, w.T + 1, w.B).astype(np.int32)
    n[0] = w.T
    n[-1] = 0
    o_com = torch.full((w.B, w.T, w.H_v, w.d_v), float("nan"), device="cuda")
    gb.gdr_recurrent_step_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], state,
                             n_tokens=torch.from_numpy(n).cuda(), o=o_com)
    torch.cuda.synchronize()
    print(f"[case] speculative round trip {name}: accepted {n.tolist()}", flush=True)
    got_state, o_ver, o_com = state.cpu().numpy(), o_ver.cpu().numpy(), o_com.cpu().numpy()
    for b in range(w.B):
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, :n[b]])
        if n[b]:
            _, h = recurrence_c(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["log_alpha"]),
                                s0[b:b + 1].astype(np.float64), w.beta_per_key_head)
            h = h[0]
        else:
            h = s0[b].astype(np.float64)
        assert rel_err(got_state[b], h) <= 1e-5, b
        assert rel_err(o_com[b, :n[b]], o_ver[b, :n[b]]) <= 1e-5 if n[b] else True
        assert np.all(np.isnan(o_com[b, n[b]:]))


def test_step_with_resets():
    w = Workload("step_resets", 2, 40, 2, 4, 128, 64, 64, 128, "bf16", seed=506)
    raw, x = draw(w)
    dev = device_inputs(raw)
    rs = make_resets(w.B, w.T, 12, seed=7, extra=[(0, 0), (1, 17)])
    rs[:, w.T - 8:] = 0            # the final state then carries several writes, not one exact one
    s0 = natural_state(w, 6)
    state = to_torch(s0)
    o = gb.gdr_recurrent_step_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], state,
                                 reset=torch.from_numpy(rs).cuda())
    o_ref, h_ref, _ = layer_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], s0.astype(np.float64), reset=rs)
    eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(state.cpu().numpy(), h_ref)
    print(f"[case] step with resets: err o={eo:.3e} state={eh:.3e}", flush=True)
    assert eo <= 1e-5 and eh <= 1e-5


# --------------------------------------------------------------- E4M3 state
def random_state(shape, seed):
    """Rows spanning several orders of magnitude, one zero row, some -0."""
    r = np.random.default_rng(seed)
    x = r.standard_normal(shape) * 10.0 ** r.uniform(-4, 1, shape[:-1] + (1,))
    x = x.astype(np.float32)
    x[0, 0, 1] = 0.0
    x[0, 0, 2, :5] = -0.0
    return x


@pytest.mark.parametrize("d_v", [32, 64, 128, 256])
def test_state_conversions_bit_exact(d_v):
    x = random_state((2, 3, 64, d_v), d_v)
    codes, scale = gb.gdr_state_quantize(to_torch(x))
    c_ref, s_ref = quantize_rows(x)
    codes, scale = codes.cpu().numpy(), scale.cpu().numpy()
    print(f"[case] E4M3 quantize d_v={d_v}: codes differing {int(np.sum(codes != c_ref))} of {codes.size}",
          flush=True)
    assert np.array_equal(scale, s_ref)
    assert np.array_equal(codes, c_ref)
    back = gb.gdr_state_dequantize(torch.from_numpy(c_ref).cuda(), torch.from_numpy(s_ref).cuda())
    assert np.array_equal(back.cpu().numpy(), dequantize_rows(c_ref, s_ref))


@pytest.mark.parametrize("d_v,dk,T", [(128, 128, 16), (64, 256, 8), (32, 64, 1)])
def test_step_over_e4m3_state(d_v, dk, T):
    """One call over T tokens from an E4M3 state: the outputs equal the fp64
    recurrence from the dequantised state within the fp32 bar; the new codes
    are the E4M3 rounding of the oracle's final state, exactly or by one code
    where the fp32 and fp64 states fall on either side of a rounding
    boundary, and the scales agree to fp32 rounding."""
    w = Workload("e4m3", 2, T, 2, 4, dk, d_v, 64, dk, "bf16", seed=507 + d_v)
    raw, x = draw(w)
    dev = device_inputs(raw)
    s_f32 = natural_state(w, 8)
    c0, sc0 = quantize_rows(s_f32)
    s_deq = dequantize_rows(c0, sc0)
    codes, scale = torch.from_numpy(c0).cuda(), torch.from_numpy(sc0).cuda()
    o = gb.gdr_recurrent_step_ex(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], codes,
                                 state_scale=scale)
    torch.cuda.synchronize()
    o_ref, h_ref = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], s_deq.astype(np.float64))
    eo = rel_err(o.cpu().numpy(), o_ref)
    c_ref, s_ref = quantize_rows(h_ref.astype(np.float32))
    got_c, got_s = codes.cpu().numpy(), scale.cpu().numpy()
    vg, vr = e4m3_value(got_c), e4m3_value(c_ref)
    same = got_c == c_ref
    # adjacent codes: no E4M3 value lies strictly between the two
    ulp = np.abs(vg - vr) <= np.maximum(np.abs(vr), np.abs(vg)) * 2.0 ** -3 + 2.0 ** -9
    print(f"[case] E4M3 step d_v={d_v} d_k={dk} T={T}: err o={eo:.3e}, codes equal {same.mean():.4f}, "
          f"scales max rel diff {np.max(np.abs(got_s - s_ref) / np.maximum(s_ref, 1e-30)):.2e}", flush=True)
    assert eo <= 1e-5
    assert np.all(same | ulp) and same.mean() >= 0.99
    assert np.allclose(got_s, s_ref, rtol=1e-5, atol=0)

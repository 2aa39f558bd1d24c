"""The C-ABI entry points under HIP graph capture: a captured sequence of
launches, replayed several times with eager work and synchronisations in
between, gives bit-identical results to the same calls made eagerly.  The
library issues only kernel launches on the caller's stream (no memset, no
allocation, no synchronisation), so its calls can be captured."""
import pytest
import torch

from gated_delta_rule_87_amd import binding as gb
from gated_delta_rule_87_amd.inputs import Workload
from gpu_common import device_inputs, draw, need_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _eager_noise():
    # unrelated eager work between replays
    x = torch.randn(1 << 16, device="cuda")
    (x * 2.0 + 1.0).sum().item()
    torch.cuda.synchronize()


def test_recurrent_steps_in_a_graph():
    need_gpu()
    w = Workload("graph_kda", 2, 12, 2, 4, 128, 64, 64, 128, "bf16", seed=41)
    raw, _ = draw(w)
    dev = device_inputs(raw)
    toks = [tuple(dev[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "beta", "log_alpha"))
            for t in range(w.T)]
    state = torch.zeros(w.B, w.H_v, w.d_k, w.d_v, device="cuda")
    o = torch.empty(w.B, 1, w.H_v, w.d_v, device="cuda")

    def steps():
        for tq, tk, tv, tb, tl in toks:
            gb.gdr_recurrent_step(tq, tk, tv, tb, tl, state, o=o)

    print("[case] recurrent steps, eager then captured", flush=True)
    steps()
    torch.cuda.synchronize()
    ref_state, ref_o = state.clone(), o.clone()
    state.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    for r in range(REPLAYS):
        state.zero_()
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), r
        assert torch.equal(o, ref_o), r
        _eager_noise()


@pytest.mark.parametrize("solve", ["exact", "neumann"])
def test_chunk_forward_in_a_graph(solve):
    need_gpu()
    w = Workload("graph_chunk", 1, 300, 2, 2, 128, 64, 64, 128, "bf16", seed=42)
    raw, _ = draw(w)
    dev = device_inputs(raw)
    p = gb.make_problem(dev["q"], dev["v"], dev["log_alpha"], dev["beta"], chunk=w.chunk, solve=solve)
    ws = torch.empty(gb.gdr_chunk_fwd_workspace_size(p) // 4, dtype=torch.float32, device="cuda")
    o = torch.empty(w.B, w.T, w.H_v, w.d_v, device="cuda")
    hT = torch.empty(w.B, w.H_v, w.d_k, w.d_v, device="cuda")
    kw = dict(chunk=w.chunk, solve=solve)

    def fwd():
        gb.gdr_chunk_prepare(dev["q"], dev["k"], dev["beta"], dev["log_alpha"], H_v=w.H_v, workspace=ws, **kw)
        gb.gdr_chunk_scan(dev["q"], dev["k"], dev["v"], dev["beta"], dev["log_alpha"], None, workspace=ws,
                          o=o, hT=hT, **kw)

    print(f"[case] chunk forward ({solve}), eager then captured", flush=True)
    fwd()
    torch.cuda.synchronize()
    ref_o, ref_h = o.clone(), hT.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    for r in range(REPLAYS):
        o.fill_(float("nan"))
        hT.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), r
        assert torch.equal(hT, ref_h), r
        _eager_noise()

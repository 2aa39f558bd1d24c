#!/usr/bin/env python3
"""Chunkwise gated delta-rule forward on one MI355X: throughput, roofline,
and the fp64 CPU oracle timed beside it.

    python bench.py [--steps K] [--warmup W] [--config 2] [--solve exact|neumann|block_neumann]   (defaults 200, 400, 2)
    python bench.py --copy-calibration BYTES      # plain copy, for rocprofv3 --pmc scaling
    python bench.py --decode [--config 2] [--state-format e4m3]   # the recurrent step, one token per sequence
    python bench.py --verify 16 [--config 2]      # speculative verify of 16 drafted tokens + commit

One step is one full forward over the workload's synthetic batch, inputs
already resident in HBM: the chunk-prep kernel then the scan/output kernel
(exactly the launches of gdr_chunk_fwd, issued as gdr_chunk_prepare +
gdr_chunk_scan so that HIP events on the launch stream time each kernel).
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec and MFMA TFLOP/s (% of peak) for chunkwise gated-delta fwd, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA peaks
KERNEL_SOURCES = {
    "prep": ["gated_delta_rule_87_amd/csrc/prep.hip", "gated_delta_rule_87_amd/csrc/common.hpp"],
    "scan": ["gated_delta_rule_87_amd/csrc/scan.hip", "gated_delta_rule_87_amd/csrc/common.hpp"],
}


def source_sha(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def work_model(w):
    """Algorithmic FLOPs and HBM bytes per launch of each kernel.

    prep: Gram and L (2 C d_k per key-head token, causal halves) and the solve
    (C^2/3 per value-head token); it must read the key side (q, k, beta, log
    alpha) once.  scan: W/U, L E and the three state products per value-head
    token; it must read v and write o (fp32) and hT once.  The workspace that
    carries prepared chunks from prep to scan is not algorithmic traffic: it
    shows up in the measured ``traffic``."""
    C, dk, dv = w.chunk, w.d_k, w.d_v
    R = w.H_v // w.H_k
    token_heads = w.B * w.T * w.H_v
    es = 2 if w.dtype == "bf16" else 4
    flops_prep = token_heads * (2.0 * C * dk / R + C * C / 3.0)
    flops_scan = token_heads * ((C + 1.0) * (dk + 2.0 * dv) + 6.0 * dk * dv)
    bt = w.B * w.T
    bytes_prep = es * bt * (2 * w.H_k * dk + w.H_k * w.G + w.H_beta)     # q, k, log_alpha, beta
    bytes_scan = es * bt * w.H_v * dv + 4 * bt * w.H_v * dv + 4 * w.B * w.H_v * dk * dv   # v, o, hT
    return {"prep": (flops_prep, bytes_prep), "scan": (flops_scan, bytes_scan)}


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    e = data.get(f"{kernel}:{workload}")
    if not e or e.get("source_sha") != source_sha(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


def host_cpu():
    """The host's logical CPUs, physical cores and CPU model (from /proc/cpuinfo)."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None:
            cores.add((phys, core))
    except OSError:
        pass
    return {"logical_cpus": os.cpu_count(), "physical_cores": len(cores) or None, "model": model}


def cpu_baseline(w, x, o_gpu, target_s=10.0, target_1t_s=3.0):
    """The fp64 oracle on a bounded sample of (batch, value head) units over the
    full sequence, on this host's cores (at most 16 threads, the CPU share of
    one GPU), and on one thread; also the GPU's error on the sample."""
    import numpy as np
    from oracle.recurrence import recurrence_c   # test infrastructure: baseline leg only

    threads = max(1, min(os.cpu_count() or 1, 16))
    units_all = w.B * w.H_v
    # calibrate: one unit over a short prefix
    Tc = min(w.T, 256)
    sl = lambda a: np.ascontiguousarray(a[:1, :Tc])
    t = time.perf_counter()
    recurrence_c(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["log_alpha"]),
                 beta_per_key_head=w.beta_per_key_head, units=[0], nthreads=1)
    per_token_head = (time.perf_counter() - t) / Tc
    n_units = int(target_s * threads / max(per_token_head * w.T, 1e-9))
    n_units = max(1, min(units_all, (n_units // threads) * threads or threads))
    rng = np.random.default_rng(12345)
    units = sorted(rng.choice(units_all, size=n_units, replace=False).tolist())
    t = time.perf_counter()
    o_ref, _ = recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"],
                            beta_per_key_head=w.beta_per_key_head, units=units, nthreads=threads)
    dt = time.perf_counter() - t
    tokens_equiv = n_units * w.T / w.H_v          # whole-job tokens (all heads) the sample is worth
    # one thread, on the first units of the same sample
    n1 = max(1, min(len(units), int(target_1t_s / max(per_token_head * w.T, 1e-9))))
    t = time.perf_counter()
    recurrence_c(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], beta_per_key_head=w.beta_per_key_head,
                 units=units[:n1], nthreads=1)
    dt1 = time.perf_counter() - t
    err = None
    if o_gpu is not None:
        num, den = 0.0, 0.0
        for u in units:
            b, h = divmod(u, w.H_v)
            ref = o_ref[b, :, h]
            num = max(num, float(np.max(np.abs(o_gpu[b, :, h] - ref))))
            den += float(np.sum(ref ** 2))
        err = num / (den / (n_units * w.T * w.d_v)) ** 0.5
    host = host_cpu()
    return {
        "value": tokens_equiv / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": f"{n_units} of {units_all} (batch, value head) units x all {w.T} tokens, "
                  f"fp64 token recurrence in C on {threads} threads, {dt:.2f} s; one thread: {n1} units, "
                  f"{dt1:.2f} s",
        "value_1thread": n1 * w.T / w.H_v / dt1,
        "host_logical_cpus": host["logical_cpus"], "host_physical_cores": host["physical_cores"],
        "cpu_model": host["model"],
    }, err


def copy_calibration(nbytes, steps):
    import torch
    n = nbytes // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / steps
    print(json.dumps({"copy_bytes": n * 4, "steps": steps, "ms_per_copy": dt * 1e3,
                      "GBs_read_plus_write": 2 * n * 4 / dt / 1e9}), flush=True)


def decode_bench(w, args, q, k, v, beta, la):
    """Decoding: gdr_recurrent_step on token t of every sequence (t runs over
    the workload's first 64 tokens), the fp32 state [B, H_v, d_k, d_v]
    resident and updated in place.  A step is one launch, short enough that
    the host's call overhead would be what the wall clock measures, so the
    64 steps are captured once in a HIP graph and the graph is replayed; one
    replay is checked against the same steps run eagerly.  The step reads and
    writes the state once; that dominates its HBM traffic."""
    import torch
    from gated_delta_rule_87_amd import binding as gb

    n_tok = min(w.T, 64)
    toks = [tuple(x[:, t:t + 1].contiguous() for x in (q, k, v, beta, la)) for t in range(n_tok)]
    e4m3 = args.state_format == "e4m3"
    state = torch.zeros((w.B, w.H_v, w.d_k, w.d_v), dtype=torch.uint8 if e4m3 else torch.float32, device="cuda")
    scale = torch.zeros((w.B, w.H_v, w.d_k), dtype=torch.float32, device="cuda") if e4m3 else None
    o = torch.empty((w.B, 1, w.H_v, w.d_v), dtype=torch.float32, device="cuda")

    def steps():
        for tq, tk, tv, tb, tl in toks:
            if e4m3:
                gb.gdr_recurrent_step_ex(tq, tk, tv, tb, tl, state, state_scale=scale, o=o)
            else:
                gb.gdr_recurrent_step(tq, tk, tv, tb, tl, state, o=o)

    def reset_state():
        state.zero_()
        if e4m3:
            scale.zero_()

    steps()                                     # eager reference from the zero state
    torch.cuda.synchronize()
    ref = state.clone()
    reset_state()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    reset_state()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replay_diff = float((state.float() - ref.float()).abs().max().item())
    reps = max(1, args.steps // n_tok)
    for _ in range(max(1, args.warmup // n_tok)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (reps * n_tok)
    es = 2 if w.dtype == "bf16" else 4
    state_bytes = (1 if e4m3 else 4) * w.B * w.H_v * w.d_k * w.d_v + (4 * w.B * w.H_v * w.d_k if e4m3 else 0)
    io_bytes = w.B * (es * (2 * w.H_k * w.d_k + w.H_v * w.d_v + w.H_beta + w.H_k * w.G) + 4 * w.H_v * w.d_v)
    achieved = (2 * state_bytes + io_bytes) / (ms_step * 1e-3) / 1e9
    print(json.dumps({
        "metric": "decode tokens/s (recurrent step, one token per sequence), 1 GPU",
        "value": w.B / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": reps * n_tok,
        "warmup": max(1, args.warmup // n_tok) * n_tok, "ms_per_step": ms_step, "higher_is_better": True,
        "dtype": ("row-scaled E4M3 state, " if e4m3 else "f32 state, ") + w.dtype + " inputs", "data": "synthetic",
        "timing": "HIP graph of 64 steps", "graph_replay_max_abs_diff_vs_eager": replay_diff,
        "config": {"workload": w.name + "_decode", "B": w.B, "T": 1, "H_k": w.H_k, "H_v": w.H_v,
                   "d_k": w.d_k, "d_v": w.d_v, "gate_groups": w.G, "state": args.state_format},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "kernel": "step", "traffic": None},
    }), flush=True)


def verify_bench(w, args, q, k, v, beta, la):
    """Speculative decoding step: verify T_ver drafted tokens of every
    sequence from its state (gdr_verify), then commit an accepted prefix of
    each (gdr_recurrent_step_ex with per-sequence token counts; here half of
    the drafted tokens).  Both launches are captured in a HIP graph and
    replayed; tokens/s counts the accepted tokens."""
    import torch
    from gated_delta_rule_87_amd import binding as gb

    tv = args.verify
    draft = tuple(x[:, :tv].contiguous() for x in (q, k, v, beta, la))
    state = torch.zeros((w.B, w.H_v, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((w.B, tv, w.H_v, w.d_v), dtype=torch.float32, device="cuda")
    oc = torch.empty_like(o)
    n_acc = torch.full((w.B,), tv // 2, dtype=torch.int32, device="cuda")

    def step():
        gb.gdr_verify(*draft, state, o=o)
        gb.gdr_recurrent_step_ex(*draft, state, n_tokens=n_acc, o=oc)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(max(1, args.warmup)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({
        "metric": "speculative decoding: verify T_ver drafted tokens + commit accepted prefix, 1 GPU",
        "value": w.B * (tv // 2) / (ms * 1e-3), "unit": "accepted tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "f32 state, " + w.dtype,
        "data": "synthetic", "timing": "HIP graph of verify + commit",
        "config": {"workload": w.name + "_verify", "B": w.B, "T_ver": tv, "accepted": tv // 2, "H_k": w.H_k,
                   "H_v": w.H_v, "d_k": w.d_k, "d_v": w.d_v, "gate_groups": w.G},
    }), flush=True)


def train_bench(w, args, q, k, v, beta, la):
    """Training step: the forward that keeps every chunk-entry state
    (gdr_chunk_fwd_train) and the backward pass (gdr_chunk_bwd) with a
    seeded upstream gradient of o; tokens/s of forward + backward."""
    import torch
    from gated_delta_rule_87_amd import binding as gb

    p = gb.make_problem(q, v, la, beta, chunk=w.chunk)
    ws_f = torch.empty(gb.gdr_chunk_fwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(gb.gdr_chunk_bwd_workspace_size(p), dtype=torch.uint8, device="cuda")
    nc = -(-w.T // w.chunk)
    states = torch.empty((w.B, w.H_v, nc, w.d_k, w.d_v), device="cuda",
                         dtype=torch.float16 if q.dtype == torch.bfloat16 else torch.float32)
    o = torch.empty((w.B, w.T, w.H_v, w.d_v), dtype=torch.float32, device="cuda")
    hT = torch.empty((w.B, w.H_v, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 7)
    d_o = torch.randn(o.shape, generator=gen, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(k.shape, **f32), "dv": torch.empty(v.shape, **f32),
           "dbeta": torch.empty(beta.shape, **f32), "dlog_alpha": torch.empty(la.shape, **f32),
           "dh0": torch.empty(hT.shape, **f32)}

    def step(evs=None):
        if evs:
            evs[0].record()
        gb.gdr_chunk_fwd_train(q, k, v, beta, la, None, chunk=w.chunk, o=o, hT=hT, states=states, workspace=ws_f)
        if evs:
            evs[1].record()
        gb.gdr_chunk_bwd(q, k, v, beta, la, states, d_o, None, chunk=w.chunk, workspace=ws_b, out=out)
        if evs:
            evs[2].record()

    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(5):
            step()
        n_warm += 5
        torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    print(json.dumps({
        "metric": "training step (chunkwise forward keeping chunk states + backward), 1 GPU",
        "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": w.dtype,
        "data": "synthetic", "kernel_ms": {"forward_train": fwd_ms, "backward": bwd_ms},
        "config": {"workload": w.name + "_train", "B": w.B, "T": w.T, "H_k": w.H_k, "H_v": w.H_v, "d_k": w.d_k,
                   "d_v": w.d_v, "chunk": w.chunk, "gate_groups": w.G, "grad_dtype": "f32"},
    }), flush=True)


def layer_bench(w, args, q, k, v, beta, la):
    """The SLA layer's forward (Systolic Linear Attention, Table 2 and
    section 2.1): packed documents (resets, geometric lengths of mean
    --doc-len tokens), chunk-boundary momentum mu = 0.25, then the gated
    RMSNorm epilogue sigma(z) * RMSNorm(o) with a seeded bf16 gate input;
    tokens/s of the whole layer forward."""
    import torch
    from gated_delta_rule_87_amd import binding as gb
    from gated_delta_rule_87_amd.inputs import make_resets

    reset = torch.from_numpy(make_resets(w.B, w.T, args.doc_len, seed=w.seed + 11)).cuda()
    p = gb.make_problem(q, v, la, beta, chunk=w.chunk)
    ws = torch.empty(max(gb.gdr_chunk_fwd_workspace_size(p), 256), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    o = torch.empty((w.B, w.T, w.H_v, w.d_v), **f32)
    y = torch.empty_like(o)
    hT = torch.empty((w.B, w.H_v, w.d_k, w.d_v), **f32)
    zT = torch.empty_like(hT)
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 13)
    z = torch.randn(o.shape, generator=gen, device="cuda").to(torch.bfloat16)
    weight = torch.ones(w.d_v, **f32)

    def step(evs=None):
        if evs:
            evs[0].record()
        gb.gdr_chunk_fwd_ex(q, k, v, beta, la, None, reset=reset, momentum=0.25, zT=zT, chunk=w.chunk, o=o, hT=hT,
                            workspace=ws)
        if evs:
            evs[1].record()
        gb.gdr_gated_rmsnorm(o, z, weight=weight, y=y)
        if evs:
            evs[2].record()

    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(5):
            step()
        n_warm += 5
        torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    epi_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    # the epilogue reads o (fp32) and z (bf16) and writes y (fp32) once
    epi_bytes = w.B * w.T * w.H_v * w.d_v * (4 + 2 + 4)
    print(json.dumps({
        "metric": "SLA layer forward (resets + chunk-boundary momentum + gated RMSNorm epilogue), 1 GPU",
        "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": w.dtype,
        "data": "synthetic", "kernel_ms": {"forward_ex": fwd_ms, "epilogue": epi_ms},
        "epilogue_roofline": {"bound": "hbm", "achieved": epi_bytes / (epi_ms * 1e-3) / 1e9, "peak": 8000.0,
                              "unit": "GB/s", "frac": epi_bytes / (epi_ms * 1e-3) / 1e9 / 8000.0},
        "config": {"workload": w.name + "_layer", "B": w.B, "T": w.T, "H_k": w.H_k, "H_v": w.H_v, "d_k": w.d_k,
                   "d_v": w.d_v, "chunk": w.chunk, "gate_groups": w.G, "momentum": 0.25,
                   "mean_doc_len": args.doc_len, "documents": int(reset.sum().item()) + w.B},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU needs a few tenths of a second of sustained work before its
    # clocks settle (timings of the first few hundred steps drift down by
    # 10-25 %): warm-up runs at least --warmup steps and at least
    # --warmup-seconds of work, whichever is longer.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--warmup-seconds", type=float, default=0.6)
    ap.add_argument("--config", type=int, default=2, help="workload index (default: per-channel-gate KDA)")
    ap.add_argument("--solve", default=None, choices=["exact", "neumann", "block_neumann"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--decode", action="store_true",
                    help="time gdr_recurrent_step on one token per sequence (its own metric)")
    ap.add_argument("--state-format", default="f32", choices=["f32", "e4m3"], help="decode state format")
    ap.add_argument("--layer", action="store_true",
                    help="time the SLA layer forward: resets, momentum 0.25, gated RMSNorm epilogue (its own metric)")
    ap.add_argument("--doc-len", type=int, default=2048, help="--layer: mean document length (geometric)")
    ap.add_argument("--batch", type=int, default=0, help="decode / verify: sequences in the batch (default: workload's)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step: forward keeping chunk states + backward (its own metric)")
    ap.add_argument("--verify", type=int, default=0, metavar="T_VER",
                    help="time verify of T_VER drafted tokens + commit of half of them (its own metric)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here.  Every "
              "(batch, value head) unit is independent, so B * H_v would be split across GPUs "
              "with no communication; run one process per GPU on its slice.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    import numpy as np
    import torch

    from gated_delta_rule_87_amd import binding as gb
    from gated_delta_rule_87_amd.inputs import WORKLOADS, decoded, make_inputs

    w = WORKLOADS[args.config]
    solve = args.solve or w.solves[0]
    if solve == "block_neumann":
        w = w.with_(neumann_order=1, neumann_residual=0)   # the pages' 1-Step Neumann
    serving = args.decode or args.verify
    if serving:
        # decode and verification read only the first 64 tokens of each sequence
        w = w.with_(T=64, B=args.batch or w.B)
    print(f"[bench] workload {w.name}: {w.description}; solve={solve}", file=sys.stderr, flush=True)
    raw = make_inputs(w)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    q, k, v, beta, la = (dev(raw[n]) for n in ("q", "k", "v", "beta", "log_alpha"))
    if args.decode:
        decode_bench(w, args, q, k, v, beta, la)
        return
    if args.verify:
        verify_bench(w, args, q, k, v, beta, la)
        return
    if args.train:
        train_bench(w, args, q, k, v, beta, la)
        return
    if args.layer:
        layer_bench(w, args, q, k, v, beta, la)
        return
    p = gb.make_problem(q, v, la, beta, chunk=w.chunk, solve=solve, neumann_order=w.neumann_order,
                        neumann_residual_steps=w.neumann_residual)
    ws = torch.empty(gb.gdr_chunk_fwd_workspace_size(p) // 4, dtype=torch.float32, device="cuda")
    o = torch.empty((w.B, w.T, w.H_v, w.d_v), dtype=torch.float32, device="cuda")
    hT = torch.empty((w.B, w.H_v, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    kw = dict(chunk=w.chunk, solve=solve, neumann_order=w.neumann_order,
              neumann_residual_steps=w.neumann_residual)

    def step(evs=None):
        if evs:
            evs[0].record()
        gb.gdr_chunk_prepare(q, k, beta, la, H_v=w.H_v, workspace=ws, **kw)
        if evs:
            evs[1].record()
        gb.gdr_chunk_scan(q, k, v, beta, la, None, workspace=ws, o=o, hT=hT, **kw)
        if evs:
            evs[2].record()

    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(10):
            step()
        n_warm += 10
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    prep_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    tokens = w.B * w.T
    model = work_model(w)
    flops_total = model["prep"][0] + model["scan"][0]
    tflops = flops_total / (ms_step * 1e-3) / 1e12
    dtype = "bf16" if w.dtype == "bf16" else "f32"

    dom = "scan" if scan_ms >= prep_ms else "prep"
    dom_ms = scan_ms if dom == "scan" else prep_ms
    f_dom, b_dom = model[dom]
    hbm_bound = b_dom / (HBM_PEAK_GBS * 1e9) >= f_dom / (MFMA_PEAK_TFS[dtype] * 1e12)
    if hbm_bound:
        achieved = b_dom / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = f_dom / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFS[dtype], "unit": "TFLOP/s",
                "frac": achieved / MFMA_PEAK_TFS[dtype]}
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(dom, w.name)

    result = {
        "metric": METRIC, "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "warmup_steps_run": n_warm, "warmup_s": round(warm_s, 3),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H_k": w.H_k, "H_v": w.H_v, "d_k": w.d_k,
                   "d_v": w.d_v, "chunk": w.chunk, "gate_groups": w.G, "solve": solve,
                   "solve_order": None if solve == "exact" else w.neumann_order,
                   "in_dtype": w.dtype, "out_dtype": "f32", "parallelism": "single-gpu"},
        "tflops_useful": tflops, "mfma_frac_useful": tflops / MFMA_PEAK_TFS[dtype],
        "kernel_ms": {"prep": prep_ms, "scan": scan_ms},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        o_np = o.cpu().numpy()
        cb, err = cpu_baseline(w, decoded(raw), o_np)
        result["cpu_baseline"] = cb
        result["parity_sample_max_err_over_rms"] = err
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

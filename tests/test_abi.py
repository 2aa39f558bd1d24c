"""The C ABI on the host (no GPU): libgdr.so loads, exports every entry point
include/gdr.h declares, sizes its workspace, and rejects every malformed call
with its documented status before anything is launched.

Every call here fails validation; none is a well-formed problem with real
device pointers, so nothing reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_87_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gb.LIB_PATH), reason="libgdr.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = gb.load()
    names = declared_functions()
    assert set(names) == set(gb.EXPORTS)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings():
    assert gb.status_string(gb.GDR_OK) == "GDR_OK"
    assert gb.status_string(gb.GDR_ERR_INVALID_ARG) == "GDR_ERR_INVALID_ARG"
    assert gb.status_string(gb.GDR_ERR_UNSUPPORTED) == "GDR_ERR_UNSUPPORTED"
    assert gb.status_string(gb.GDR_ERR_WORKSPACE) == "GDR_ERR_WORKSPACE"
    assert gb.status_string(gb.GDR_ERR_HIP) == "GDR_ERR_HIP"


def problem(**kw):
    p = gb.GdrProblem()
    base = dict(B=2, T=8192, H_k=32, H_v=32, d_k=128, d_v=128, chunk=64, gate_groups=128,
                beta_per_key_head=0, in_dtype=gb.GDR_BF16, out_dtype=gb.GDR_F32, solve=0,
                neumann_order=4, neumann_residual_steps=1)
    base.update(kw)
    for k_, v_ in base.items():
        setattr(p, k_, v_)
    return p


def expected_regions(B, T, H_k, H_v, d_k, chunk, bf16=True, beta_per_key_head=0):
    """Region sizes as documented in include/gdr.h (each region padded to 256 B)."""
    nc = -(-T // chunk)
    hb = H_k if beta_per_key_head else H_v
    pb = 2 if bf16 else 4                      # fp16 tiles for bf16 inputs, fp32 otherwise
    tiles = [("A", hb, pb * chunk * chunk), ("L", H_k, pb * chunk * chunk), ("KB", H_k, pb * chunk * d_k),
             ("QB", H_k, pb * chunk * d_k), ("KH", H_k, pb * d_k * chunk), ("GM", H_k, 4 * d_k)]
    out, at = {}, 0
    for name, heads, tile in tiles:
        out[name] = at
        at += B * heads * nc * tile
        at = -(-at // 256) * 256
    out["total"] = at
    return out


def test_workspace_size():
    lib = gb.load()
    p = problem()
    exp = expected_regions(2, 8192, 32, 32, 128, 64)
    assert exp["total"] == 541_065_216
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(p)) == exp["total"]
    assert gb.gdr_chunk_workspace_layout(p) == exp
    p = problem(H_k=8, H_v=32, d_k=256, gate_groups=4, T=100)
    assert gb.gdr_chunk_workspace_layout(p) == expected_regions(2, 100, 8, 32, 256, 64)
    p = problem(H_k=8, H_v=32, d_k=256, gate_groups=4, T=100, beta_per_key_head=1)
    assert gb.gdr_chunk_workspace_layout(p) == expected_regions(2, 100, 8, 32, 256, 64, beta_per_key_head=1)
    p = problem(T=333, chunk=128, in_dtype=gb.GDR_F32, d_v=32)
    assert gb.gdr_chunk_workspace_layout(p) == expected_regions(2, 333, 32, 32, 128, 128, bf16=False)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(problem(H_v=30))) == 0
    assert lib.gdr_chunk_fwd_workspace_size(None) == 0
    with pytest.raises(gb.GdrError):
        gb.gdr_chunk_workspace_layout(problem(H_v=30))


def test_workspace_size_chunk16():
    """Chunk 16 runs as chunk 32 on T' = 32 ceil(T / 16) tokens: its
    workspace is that padded problem's, followed by padded copies of q, k, v,
    beta, log alpha, the reset flags and o (each 256-byte aligned)."""
    lib = gb.load()
    B, T, Hk, Hv, dk, dv, G = 2, 300, 2, 4, 128, 64, 128
    p = problem(B=B, T=T, H_k=Hk, H_v=Hv, d_k=dk, d_v=dv, chunk=16, gate_groups=G)
    Tp = 32 * -(-T // 16)
    pp = problem(B=B, T=Tp, H_k=Hk, H_v=Hv, d_k=dk, d_v=dv, chunk=32, gate_groups=G)
    base = lib.gdr_chunk_fwd_workspace_size(ctypes.byref(pp))   # with the segment-parallel scan's region
    assert base >= expected_regions(B, Tp, Hk, Hv, dk, 32)["total"]
    up = lambda n: -(-n // 256) * 256
    rows = B * Tp
    extra = sum(up(n) for n in (rows * Hk * dk * 2, rows * Hk * dk * 2, rows * Hv * dv * 2, rows * Hv * 2,
                                rows * Hk * G * 2, rows, rows * Hv * dv * 4))
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(p)) == base + extra
    assert gb.gdr_chunk_workspace_layout(p)["KB"] == expected_regions(B, Tp, Hk, Hv, dk, 32)["KB"]


FAKE = 0x10000          # 64 KiB-aligned non-null address, never dereferenced
MIS = 0x10004           # misaligned


def call_fwd(p, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, la=FAKE, h0=None, o=FAKE, hT=None, ws=FAKE, ws_bytes=None):
    lib = gb.load()
    if ws_bytes is None:
        ws_bytes = 1 << 40
    vp = ctypes.c_void_p
    return lib.gdr_chunk_fwd(None if p is None else ctypes.byref(p), vp(q), vp(k), vp(v), vp(beta), vp(la),
                             vp(h0), vp(o), vp(hT), vp(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H_v=30), gb.GDR_ERR_INVALID_ARG),
    (dict(H_k=0), gb.GDR_ERR_INVALID_ARG),
    (dict(B=-1), gb.GDR_ERR_INVALID_ARG),
    (dict(T=-5), gb.GDR_ERR_INVALID_ARG),
    (dict(d_v=0), gb.GDR_ERR_INVALID_ARG),
    (dict(gate_groups=3), gb.GDR_ERR_INVALID_ARG),
    (dict(gate_groups=0), gb.GDR_ERR_INVALID_ARG),
    (dict(in_dtype=7), gb.GDR_ERR_INVALID_ARG),
    (dict(out_dtype=-1), gb.GDR_ERR_INVALID_ARG),
    (dict(beta_per_key_head=2), gb.GDR_ERR_INVALID_ARG),
    (dict(chunk=0), gb.GDR_ERR_INVALID_ARG),
    (dict(solve=5), gb.GDR_ERR_INVALID_ARG),
    (dict(solve=1, neumann_order=-1), gb.GDR_ERR_INVALID_ARG),
    (dict(solve=1, neumann_residual_steps=-2), gb.GDR_ERR_INVALID_ARG),
    (dict(d_k=96, gate_groups=96), gb.GDR_ERR_UNSUPPORTED),
    (dict(d_v=72), gb.GDR_ERR_UNSUPPORTED),
    (dict(chunk=48), gb.GDR_ERR_UNSUPPORTED),
    (dict(chunk=16, d_v=48), gb.GDR_ERR_UNSUPPORTED),
    (dict(chunk=24), gb.GDR_ERR_UNSUPPORTED),
    (dict(chunk=32, d_v=48), gb.GDR_ERR_UNSUPPORTED),
    (dict(solve=2, neumann_order=-1), gb.GDR_ERR_INVALID_ARG),
    (dict(chunk=128, d_k=256, gate_groups=256), gb.GDR_ERR_UNSUPPORTED),
    (dict(B=1 << 20, T=1 << 20), gb.GDR_ERR_INVALID_ARG),
    (dict(B=70000), gb.GDR_ERR_UNSUPPORTED),
    (dict(H_k=70000, H_v=70000), gb.GDR_ERR_UNSUPPORTED),
    (dict(B=1, T=(1 << 30) + 1), gb.GDR_ERR_UNSUPPORTED),
    (dict(B=128, H_k=4096, H_v=4096, d_v=256), gb.GDR_ERR_UNSUPPORTED),
])
def test_invalid_problems(kw, status):
    assert call_fwd(problem(**kw)) == status
    assert gb.last_error() != ""


@pytest.mark.parametrize("kw", [
    dict(B=1, T=256, chunk=128, H_k=256, H_v=32768, d_v=256, beta_per_key_head=1),
    dict(B=1, T=256, chunk=64, H_k=1024, H_v=32768, d_v=512, beta_per_key_head=1),
])
def test_chunk_of_v_or_o_beyond_4gib(kw):
    """The scan addresses the rows of one chunk of v and o with 32-bit byte
    offsets: C * H_v * d_v * 4 bytes must stay below 2^32."""
    p = problem(**kw)
    assert p.chunk * p.H_v * p.d_v * 4 >= 1 << 32
    assert call_fwd(p) == gb.GDR_ERR_UNSUPPORTED
    assert "2^30" in gb.last_error()
    # the same heads at half the value width pass this check
    assert (p.chunk * p.H_v * (p.d_v // 2) * 4) < 1 << 32


def test_null_problem():
    assert call_fwd(None) == gb.GDR_ERR_INVALID_ARG


@pytest.mark.parametrize("arg", ["q", "k", "v", "beta", "la", "o", "ws"])
def test_null_pointer(arg):
    assert call_fwd(problem(), **{arg: 0}) == gb.GDR_ERR_INVALID_ARG
    assert "NULL" in gb.last_error()


@pytest.mark.parametrize("arg", ["q", "k", "v", "beta", "la", "o", "h0", "hT", "ws"])
def test_misaligned_pointer(arg):
    assert call_fwd(problem(), **{arg: MIS}) == gb.GDR_ERR_INVALID_ARG
    assert "aligned" in gb.last_error()


def test_workspace_too_small():
    p = problem()
    need = gb.load().gdr_chunk_fwd_workspace_size(ctypes.byref(p))
    assert call_fwd(p, ws_bytes=need - 1) == gb.GDR_ERR_WORKSPACE
    assert str(need) in gb.last_error()


def test_prepare_and_step_validate():
    lib = gb.load()
    vp = ctypes.c_void_p
    p = problem(H_v=30)
    assert lib.gdr_chunk_prepare(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1 << 40,
                                 None) == gb.GDR_ERR_INVALID_ARG
    p = problem()
    assert lib.gdr_chunk_prepare(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 16,
                                 None) == gb.GDR_ERR_WORKSPACE
    # the recurrent path ignores chunk/solve but checks the rest
    p = problem(chunk=0, solve=9)
    assert lib.gdr_recurrent_step(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(0),
                                  vp(FAKE), None) == gb.GDR_ERR_INVALID_ARG
    assert "state" in gb.last_error()
    # the scan reads only v, h0 and the workspace
    p = problem()
    assert lib.gdr_chunk_scan(ctypes.byref(p), vp(0), None, vp(FAKE), None, vp(FAKE), 1 << 40,
                              None) == gb.GDR_ERR_INVALID_ARG
    assert "v is NULL" in gb.last_error()
    assert lib.gdr_chunk_scan(ctypes.byref(p), vp(FAKE), None, vp(FAKE), None, vp(FAKE), 1024,
                              None) == gb.GDR_ERR_WORKSPACE
    assert lib.gdr_chunk_scan(ctypes.byref(p), vp(FAKE), None, vp(FAKE), None, vp(MIS), 1 << 40,
                              None) == gb.GDR_ERR_INVALID_ARG
    p = problem(d_k=32, gate_groups=32)
    assert lib.gdr_recurrent_step(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                  vp(FAKE), None) == gb.GDR_ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        gb.gdr_chunk_fwd(q, q, q, torch.zeros(1, 64, 1), torch.zeros(1, 64, 1, 1))

"""ctypes binding of libgdr.so with the C ABI's names (include/gdr.h).

Argument marshalling only: torch tensors provide device memory and the
current stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if libgdr.so is missing or a tensor is not on
the GPU, the call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_WORKSPACE, GDR_ERR_HIP = range(5)
GDR_F32, GDR_BF16 = 0, 1
GDR_SOLVE_EXACT, GDR_SOLVE_NEUMANN, GDR_SOLVE_BLOCK_NEUMANN = 0, 1, 2

EXPORTS = ("gdr_chunk_fwd", "gdr_chunk_fwd_workspace_size", "gdr_chunk_workspace_layout", "gdr_chunk_prepare",
           "gdr_chunk_scan", "gdr_chunk_fwd_noalloc", "gdr_chunk_fwd_ex", "gdr_gated_rmsnorm", "gdr_recurrent_step",
           "gdr_verify", "gdr_recurrent_step_ex", "gdr_state_quantize", "gdr_state_dequantize",
           "gdr_chunk_states_size", "gdr_chunk_fwd_train", "gdr_chunk_bwd_workspace_size", "gdr_chunk_bwd",
           "gdr_status_string", "gdr_last_error")
GDR_STATE_F32, GDR_STATE_E4M3 = 0, 1
NOALLOC_SCRATCH_BYTES = 128 << 20   # GDR_NOALLOC_SCRATCH_BYTES
# Workspace regions, in order (include/gdr.h, gdr_chunk_fwd_workspace_size).
WS_REGIONS = ("A", "L", "KB", "QB", "KH", "GM")


class GdrProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "T", "H_k", "H_v", "d_k", "d_v", "chunk", "gate_groups", "beta_per_key_head",
        "in_dtype", "out_dtype", "solve", "neumann_order", "neumann_residual_steps")]


class GdrLayerOpts(ctypes.Structure):
    _fields_ = [("reset", ctypes.c_void_p), ("momentum", ctypes.c_float), ("z0", ctypes.c_void_p),
                ("zT", ctypes.c_void_p)]


class GdrStepOpts(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_void_p), ("reset", ctypes.c_void_p), ("state_format", ctypes.c_int32),
                ("state_scale", ctypes.c_void_p)]


class GdrError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


_lib = None


def load():
    """Load libgdr.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_87_amd._build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GdrProblem)
        vp = ctypes.c_void_p
        lib.gdr_chunk_fwd_workspace_size.restype = ctypes.c_size_t
        lib.gdr_chunk_fwd_workspace_size.argtypes = [P]
        lib.gdr_chunk_fwd.restype = ctypes.c_int
        lib.gdr_chunk_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_scan.restype = ctypes.c_int
        lib.gdr_chunk_scan.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_workspace_layout.restype = ctypes.c_int
        lib.gdr_chunk_workspace_layout.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.gdr_chunk_prepare.restype = ctypes.c_int
        lib.gdr_chunk_prepare.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_fwd_ex.restype = ctypes.c_int
        lib.gdr_chunk_fwd_ex.argtypes = [P, ctypes.POINTER(GdrLayerOpts), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        lib.gdr_gated_rmsnorm.restype = ctypes.c_int
        lib.gdr_gated_rmsnorm.argtypes = [P, vp, vp, vp, ctypes.c_float, vp, vp]
        lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.gdr_chunk_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_recurrent_step.restype = ctypes.c_int
        lib.gdr_recurrent_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_verify.restype = ctypes.c_int
        lib.gdr_verify.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_recurrent_step_ex.restype = ctypes.c_int
        lib.gdr_recurrent_step_ex.argtypes = [P, ctypes.POINTER(GdrStepOpts), vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdr_state_quantize.restype = ctypes.c_int
        lib.gdr_state_quantize.argtypes = [P, vp, vp, vp, vp]
        lib.gdr_state_dequantize.restype = ctypes.c_int
        lib.gdr_state_dequantize.argtypes = [P, vp, vp, vp, vp]
        lib.gdr_chunk_states_size.restype = ctypes.c_size_t
        lib.gdr_chunk_states_size.argtypes = [P]
        lib.gdr_chunk_fwd_train.restype = ctypes.c_int
        lib.gdr_chunk_fwd_train.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.gdr_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        lib.gdr_chunk_bwd_workspace_size.argtypes = [P]
        lib.gdr_chunk_bwd.restype = ctypes.c_int
        lib.gdr_chunk_bwd.argtypes = [P] + [vp] * 15 + [ctypes.c_size_t, vp]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_status_string.argtypes = [ctypes.c_int]
        lib.gdr_last_error.restype = ctypes.c_char_p
        lib.gdr_last_error.argtypes = []
        _lib = lib
    return _lib


def status_string(status):
    return load().gdr_status_string(int(status)).decode()


def last_error():
    return load().gdr_last_error().decode()


def _check(status):
    if status != GDR_OK:
        raise GdrError(status, last_error())


_DT = {torch.float32: GDR_F32, torch.bfloat16: GDR_BF16}


def make_problem(q, v, log_alpha, beta, *, chunk=64, solve="exact", neumann_order=4,
                 neumann_residual_steps=1, out_dtype=torch.float32):
    """A gdr_problem from tensor shapes (q [B,T,H_k,d_k], v [B,T,H_v,d_v],
    log_alpha [B,T,H_k,G], beta [B,T,H_v] or [B,T,H_k])."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if q.dtype not in _DT or out_dtype not in _DT:
        raise TypeError(f"dtypes must be float32 or bfloat16, got {q.dtype} / {out_dtype}")
    if beta.shape[2] not in (Hk, Hv):
        raise ValueError(f"beta has {beta.shape[2]} heads; expected H_v={Hv} or H_k={Hk}")
    p = GdrProblem()
    p.B, p.T, p.H_k, p.H_v, p.d_k, p.d_v = B, T, Hk, Hv, dk, dv
    p.chunk = chunk
    p.gate_groups = log_alpha.shape[3]
    p.beta_per_key_head = int(beta.shape[2] == Hk and Hk != Hv)
    p.in_dtype = _DT[q.dtype]
    p.out_dtype = _DT[out_dtype]
    p.solve = {"exact": GDR_SOLVE_EXACT, "neumann": GDR_SOLVE_NEUMANN, "block_neumann": GDR_SOLVE_BLOCK_NEUMANN}[solve]
    p.neumann_order = neumann_order
    p.neumann_residual_steps = neumann_residual_steps
    return p


def _ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_inputs(q, k, v, beta, log_alpha):
    dt = q.dtype
    B, T, Hk, dk = q.shape
    _ptr(q, "q", dt)
    _ptr(k, "k", dt, q.shape)
    if v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError(f"v has shape {tuple(v.shape)}; expected [B, T, H_v, d_v] with B={B}, T={T}")
    _ptr(v, "v", dt)
    if beta.dim() != 3 or beta.shape[:2] != q.shape[:2]:
        raise ValueError(f"beta has shape {tuple(beta.shape)}; expected [B, T, H]")
    _ptr(beta, "beta", dt)
    if log_alpha.dim() != 4 or log_alpha.shape[:3] != q.shape[:3]:
        raise ValueError(f"log_alpha has shape {tuple(log_alpha.shape)}; expected [B, T, H_k, G]")
    _ptr(log_alpha, "log_alpha", dt)


def gdr_chunk_fwd_workspace_size(problem):
    return int(load().gdr_chunk_fwd_workspace_size(ctypes.byref(problem)))


def gdr_chunk_workspace_layout(problem):
    """{region name: byte offset} for the six workspace regions, plus "total"."""
    out = (ctypes.c_size_t * 7)()
    _check(load().gdr_chunk_workspace_layout(ctypes.byref(problem), out))
    d = dict(zip(WS_REGIONS, (int(x) for x in out[:6])))
    d["total"] = int(out[6])
    return d


def _chunk_call(entry, q, k, v, beta, log_alpha, h0, chunk, solve, neumann_order, neumann_residual_steps,
                out_dtype, o, hT, return_final_state, workspace, stream):
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, chunk=chunk, solve=solve, neumann_order=neumann_order,
                     neumann_residual_steps=neumann_residual_steps, out_dtype=out_dtype)
    dev = q.device
    if o is None:
        o = torch.empty((p.B, p.T, p.H_v, p.d_v), dtype=out_dtype, device=dev)
    state_shape = (p.B, p.H_v, p.d_k, p.d_v)
    if hT is None and return_final_state:
        hT = torch.empty(state_shape, dtype=torch.float32, device=dev)
    ws_bytes = gdr_chunk_fwd_workspace_size(p)
    if ws_bytes == 0 and p.B * p.T > 0:
        _check(lib.gdr_chunk_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None, 0, None))
    if workspace is None:
        if entry == "gdr_chunk_scan":
            raise ValueError("gdr_chunk_scan needs the workspace gdr_chunk_prepare filled")
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    h0p, hTp = _ptr(h0, "h0", torch.float32, state_shape), _ptr(hT, "hT", torch.float32, state_shape)
    op = _ptr(o, "o", out_dtype, (p.B, p.T, p.H_v, p.d_v))
    wsp, wsn = _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    if entry == "gdr_chunk_scan":
        _check(lib.gdr_chunk_scan(ctypes.byref(p), _ptr(v, "v"), h0p, op, hTp, wsp, wsn, _stream(stream)))
    else:
        _check(lib.gdr_chunk_fwd(ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"),
                                 _ptr(log_alpha, "log_alpha"), h0p, op, hTp, wsp, wsn, _stream(stream)))
    return o, hT


def gdr_chunk_fwd(q, k, v, beta, log_alpha, h0=None, *, chunk=64, solve="exact", neumann_order=4,
                  neumann_residual_steps=1, out_dtype=torch.float32, o=None, hT=None,
                  return_final_state=True, workspace=None, stream=None):
    """Chunkwise forward.  Returns (o [B,T,H_v,d_v], hT [B,H_v,d_k,d_v] fp32 or None).

    ``workspace`` (a GPU tensor) may be passed to avoid an allocation; on
    return it holds the prepared chunk quantities (gdr_chunk_workspace_layout)."""
    return _chunk_call("gdr_chunk_fwd", q, k, v, beta, log_alpha, h0, chunk, solve, neumann_order,
                       neumann_residual_steps, out_dtype, o, hT, return_final_state, workspace, stream)


def gdr_chunk_fwd_ex(q, k, v, beta, log_alpha, h0=None, *, reset=None, momentum=0.0, z0=None, zT=None,
                     return_momentum_state=False, chunk=64, solve="exact", neumann_order=4, neumann_residual_steps=1,
                     out_dtype=torch.float32, o=None, hT=None, return_final_state=True, workspace=None, stream=None):
    """Chunk forward with the layer options: ``reset`` (uint8/bool [B, T],
    nonzero where a token starts a new document), chunk-boundary ``momentum``
    (mu) with buffer ``z0`` in and ``zT`` out (fp32 [B, H_v, d_k, d_v]).
    Returns (o, hT) or, with ``return_momentum_state`` (or a given zT),
    (o, hT, zT)."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, chunk=chunk, solve=solve, neumann_order=neumann_order,
                     neumann_residual_steps=neumann_residual_steps, out_dtype=out_dtype)
    dev = q.device
    state_shape = (p.B, p.H_v, p.d_k, p.d_v)
    if o is None:
        o = torch.empty((p.B, p.T, p.H_v, p.d_v), dtype=out_dtype, device=dev)
    if hT is None and return_final_state:
        hT = torch.empty(state_shape, dtype=torch.float32, device=dev)
    want_z = return_momentum_state or zT is not None
    if zT is None and want_z:
        zT = torch.empty(state_shape, dtype=torch.float32, device=dev)
    if reset is not None:
        if tuple(reset.shape) != (p.B, p.T):
            raise ValueError(f"reset has shape {tuple(reset.shape)}, expected {(p.B, p.T)}")
        reset = reset.to(torch.uint8) if reset.dtype != torch.uint8 else reset
    opts = GdrLayerOpts()
    opts.reset = _ptr(reset, "reset", torch.uint8)
    opts.momentum = float(momentum)
    opts.z0 = _ptr(z0, "z0", torch.float32, state_shape)
    opts.zT = _ptr(zT, "zT", torch.float32, state_shape)
    ws_bytes = gdr_chunk_fwd_workspace_size(p)
    if ws_bytes == 0 and p.B * p.T > 0:
        _check(lib.gdr_chunk_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None, 0, None))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _check(lib.gdr_chunk_fwd_ex(
        ctypes.byref(p), ctypes.byref(opts), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"),
        _ptr(log_alpha, "log_alpha"), _ptr(h0, "h0", torch.float32, state_shape),
        _ptr(o, "o", out_dtype, (p.B, p.T, p.H_v, p.d_v)), _ptr(hT, "hT", torch.float32, state_shape),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return (o, hT, zT) if want_z else (o, hT)


def gdr_gated_rmsnorm(o, z, *, weight=None, eps=1e-6, y=None, stream=None):
    """y = sigmoid(z) * o / sqrt(mean(o^2 over d_v) + eps) * weight, per
    (batch, token, value head) row; o, y [B, T, H_v, d_v] (fp32 or bf16, y
    like o unless given), z [B, T, H_v, d_v] (fp32 or bf16), weight fp32
    [d_v] or None.  y may be o itself."""
    lib = load()
    if o.dim() != 4 or tuple(z.shape) != tuple(o.shape):
        raise ValueError(f"o {tuple(o.shape)} and z {tuple(z.shape)} must both be [B, T, H_v, d_v]")
    if y is None:
        y = torch.empty_like(o)
    B, T, Hv, dv = o.shape
    p = GdrProblem()
    p.B, p.T, p.H_k, p.H_v, p.d_k, p.d_v = B, T, Hv, Hv, 64, dv
    p.chunk, p.gate_groups = 64, 1
    p.in_dtype = _DT[z.dtype]
    p.out_dtype = _DT[o.dtype]
    _check(lib.gdr_gated_rmsnorm(ctypes.byref(p), _ptr(o, "o"), _ptr(z, "z"),
                                 _ptr(weight, "weight", torch.float32, (dv,)), float(eps),
                                 _ptr(y, "y", o.dtype, tuple(o.shape)), _stream(stream)))
    return y


def gdr_chunk_fwd_noalloc(q, k, v, beta, log_alpha, h0, o, hT, *, chunk=64, solve="exact", neumann_order=4,
                          neumann_residual_steps=1, stream=None):
    """gdr_chunk_fwd into caller-provided ``o`` (and ``hT``, or None) with the
    library's static per-device scratch instead of a workspace: neither this
    call nor the library allocates.  Calls that overlap on one device race."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, chunk=chunk, solve=solve, neumann_order=neumann_order,
                     neumann_residual_steps=neumann_residual_steps, out_dtype=o.dtype)
    state_shape = (p.B, p.H_v, p.d_k, p.d_v)
    _check(lib.gdr_chunk_fwd_noalloc(
        ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"), _ptr(log_alpha, "log_alpha"),
        _ptr(h0, "h0", torch.float32, state_shape), _ptr(o, "o", o.dtype, (p.B, p.T, p.H_v, p.d_v)),
        _ptr(hT, "hT", torch.float32, state_shape), _stream(stream)))
    return o, hT


def gdr_chunk_scan(q, k, v, beta, log_alpha, h0=None, *, workspace, chunk=64, solve="exact", neumann_order=4,
                   neumann_residual_steps=1, out_dtype=torch.float32, o=None, hT=None,
                   return_final_state=True, stream=None):
    """State scan and output over a workspace filled by gdr_chunk_prepare.  The
    tensors q, k, beta and log_alpha only describe the problem (shapes and
    dtype); the library reads v, h0 and the workspace."""
    return _chunk_call("gdr_chunk_scan", q, k, v, beta, log_alpha, h0, chunk, solve, neumann_order,
                       neumann_residual_steps, out_dtype, o, hT, return_final_state, workspace, stream)


def gdr_chunk_prepare(q, k, beta, log_alpha, *, chunk=64, solve="exact", neumann_order=4,
                      neumann_residual_steps=1, H_v=None, d_v=None, workspace=None, stream=None):
    """The parallel half of the chunk forward.  Returns (workspace, problem):
    ``workspace`` (allocated as uint8 if not given) holds the prepared chunk
    quantities laid out as gdr_chunk_workspace_layout(problem) gives.  d_v:
    the value width of the scan that will read it (the workspace size depends
    on it through the segment-parallel scan's region and chunk 16's padded
    copies); by default the smallest width the chunk size takes."""
    lib = load()
    B, T, Hk, dk = q.shape
    Hv = beta.shape[2] if H_v is None else H_v
    dv = d_v if d_v is not None else (32 if chunk <= 32 else 16)
    fake_v = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    _check_inputs(q, k, fake_v, beta, log_alpha)
    p = make_problem(q, fake_v, log_alpha, beta, chunk=chunk, solve=solve, neumann_order=neumann_order,
                     neumann_residual_steps=neumann_residual_steps)
    ws_bytes = gdr_chunk_fwd_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=q.device)
    _check(lib.gdr_chunk_prepare(ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(beta, "beta"),
                                 _ptr(log_alpha, "log_alpha"), _ptr(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return workspace, p


def gdr_recurrent_step(q, k, v, beta, log_alpha, state, *, out_dtype=torch.float32, o=None, stream=None):
    """Token recurrence over q.shape[1] tokens; ``state`` (fp32 [B,H_v,d_k,d_v])
    is updated in place.  Returns o [B,T,H_v,d_v]."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, out_dtype=out_dtype)
    if o is None:
        o = torch.empty((p.B, p.T, p.H_v, p.d_v), dtype=out_dtype, device=q.device)
    _check(lib.gdr_recurrent_step(
        ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"), _ptr(log_alpha, "log_alpha"),
        _ptr(state, "state", torch.float32, (p.B, p.H_v, p.d_k, p.d_v)),
        _ptr(o, "o", out_dtype, (p.B, p.T, p.H_v, p.d_v)), _stream(stream)))
    return o


def gdr_verify(q, k, v, beta, log_alpha, state, *, out_dtype=torch.float32, o=None, stream=None):
    """Outputs of T <= 16 drafted tokens read from ``state`` (fp32
    [B, H_v, d_k, d_v], not modified).  Returns o [B, T, H_v, d_v]."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, out_dtype=out_dtype)
    if o is None:
        o = torch.empty((p.B, p.T, p.H_v, p.d_v), dtype=out_dtype, device=q.device)
    _check(lib.gdr_verify(
        ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"), _ptr(log_alpha, "log_alpha"),
        _ptr(state, "state", torch.float32, (p.B, p.H_v, p.d_k, p.d_v)),
        _ptr(o, "o", out_dtype, (p.B, p.T, p.H_v, p.d_v)), _stream(stream)))
    return o


def gdr_recurrent_step_ex(q, k, v, beta, log_alpha, state, *, n_tokens=None, reset=None, state_scale=None,
                          out_dtype=torch.float32, o=None, stream=None):
    """gdr_recurrent_step with per-sequence token counts ``n_tokens`` (int32
    [B]), document ``reset`` flags (uint8 [B, T]) and, when ``state`` is a
    uint8 tensor of E4M3 codes, the row-scaled FP8 state with its fp32
    ``state_scale`` [B, H_v, d_k] (both updated in place)."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, out_dtype=out_dtype)
    if o is None:
        o = torch.empty((p.B, p.T, p.H_v, p.d_v), dtype=out_dtype, device=q.device)
    opts = GdrStepOpts()
    shape = (p.B, p.H_v, p.d_k, p.d_v)
    if state.dtype == torch.uint8:
        opts.state_format = GDR_STATE_E4M3
        sp = _ptr(state, "state", torch.uint8, shape)
        opts.state_scale = _ptr(state_scale, "state_scale", torch.float32, shape[:3])
    else:
        opts.state_format = GDR_STATE_F32
        sp = _ptr(state, "state", torch.float32, shape)
    opts.n_tokens = _ptr(n_tokens, "n_tokens", torch.int32, (p.B,))
    opts.reset = _ptr(reset, "reset", torch.uint8, (p.B, p.T))
    _check(lib.gdr_recurrent_step_ex(
        ctypes.byref(p), ctypes.byref(opts), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"),
        _ptr(log_alpha, "log_alpha"), sp, _ptr(o, "o", out_dtype, (p.B, p.T, p.H_v, p.d_v)), _stream(stream)))
    return o


def _state_problem(shape):
    B, Hv, dk, dv = shape
    p = GdrProblem()
    p.B, p.T, p.H_k, p.H_v, p.d_k, p.d_v = B, 1, Hv, Hv, dk, dv
    p.chunk, p.gate_groups = 64, 1
    return p


def gdr_state_quantize(state, *, codes=None, scale=None, stream=None):
    """fp32 state [B, H_v, d_k, d_v] -> (E4M3 codes uint8, fp32 row scales [B, H_v, d_k])."""
    lib = load()
    p = _state_problem(tuple(state.shape))
    if codes is None:
        codes = torch.empty(state.shape, dtype=torch.uint8, device=state.device)
    if scale is None:
        scale = torch.empty(state.shape[:3], dtype=torch.float32, device=state.device)
    _check(lib.gdr_state_quantize(ctypes.byref(p), _ptr(state, "state", torch.float32),
                                  _ptr(codes, "codes", torch.uint8, tuple(state.shape)),
                                  _ptr(scale, "scale", torch.float32, tuple(state.shape[:3])), _stream(stream)))
    return codes, scale


def gdr_state_dequantize(codes, scale, *, state=None, stream=None):
    """(E4M3 codes, row scales) -> fp32 state [B, H_v, d_k, d_v]."""
    lib = load()
    p = _state_problem(tuple(codes.shape))
    if state is None:
        state = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib.gdr_state_dequantize(ctypes.byref(p), _ptr(codes, "codes", torch.uint8),
                                    _ptr(scale, "scale", torch.float32, tuple(codes.shape[:3])),
                                    _ptr(state, "state", torch.float32, tuple(codes.shape)), _stream(stream)))
    return state


# ------------------------------------------------------------------ training
def gdr_chunk_states_size(problem):
    return int(load().gdr_chunk_states_size(ctypes.byref(problem)))


def gdr_chunk_bwd_workspace_size(problem):
    return int(load().gdr_chunk_bwd_workspace_size(ctypes.byref(problem)))


def gdr_chunk_fwd_train(q, k, v, beta, log_alpha, h0=None, *, chunk=64, out_dtype=torch.float32, o=None,
                        hT=None, states=None, workspace=None, stream=None):
    """Training forward: gdr_chunk_fwd that also keeps the state entering
    every chunk.  Returns (o, hT, states) with states [B, H_v, N_c, d_k, d_v],
    float16 for bfloat16 inputs and float32 for float32 inputs."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    p = make_problem(q, v, log_alpha, beta, chunk=chunk, out_dtype=out_dtype)
    dev = q.device
    nc = (p.T + p.chunk - 1) // p.chunk
    state_shape = (p.B, p.H_v, p.d_k, p.d_v)
    if o is None:
        o = torch.empty((p.B, p.T, p.H_v, p.d_v), dtype=out_dtype, device=dev)
    if hT is None:
        hT = torch.empty(state_shape, dtype=torch.float32, device=dev)
    st_dtype = torch.float16 if q.dtype == torch.bfloat16 else torch.float32
    if states is None:
        states = torch.empty((p.B, p.H_v, nc, p.d_k, p.d_v), dtype=st_dtype, device=dev)
    ws_bytes = gdr_chunk_fwd_workspace_size(p)
    if gdr_chunk_states_size(p) == 0 and p.B * p.T > 0:
        _check(lib.gdr_chunk_fwd_train(ctypes.byref(p), *([None] * 10), 0, None))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _check(lib.gdr_chunk_fwd_train(
        ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"), _ptr(log_alpha, "log_alpha"),
        _ptr(h0, "h0", torch.float32, state_shape), _ptr(o, "o", out_dtype, (p.B, p.T, p.H_v, p.d_v)),
        _ptr(hT, "hT", torch.float32, state_shape),
        _ptr(states, "states", st_dtype, (p.B, p.H_v, nc, p.d_k, p.d_v)),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, hT, states


def gdr_chunk_bwd(q, k, v, beta, log_alpha, states, d_o, dhT=None, *, chunk=64, want_dh0=True, workspace=None,
                  out=None, stream=None):
    """Backward pass.  ``d_o`` has the forward's output dtype; ``states``
    comes from gdr_chunk_fwd_train.  Returns a dict of fp32 gradients dq, dk,
    dv, dbeta, dlog_alpha and dh0 (None unless ``want_dh0``); ``out`` may
    hold preallocated tensors for them."""
    lib = load()
    _check_inputs(q, k, v, beta, log_alpha)
    if d_o.dtype not in _DT:
        raise TypeError(f"d_o must be float32 or bfloat16, got {d_o.dtype}")
    p = make_problem(q, v, log_alpha, beta, chunk=chunk, out_dtype=d_o.dtype)
    dev = q.device
    nc = (p.T + p.chunk - 1) // p.chunk
    state_shape = (p.B, p.H_v, p.d_k, p.d_v)
    f32 = dict(dtype=torch.float32, device=dev)
    if out is None:
        out = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(k.shape, **f32),
               "dv": torch.empty(v.shape, **f32), "dbeta": torch.empty(beta.shape, **f32),
               "dlog_alpha": torch.empty(log_alpha.shape, **f32),
               "dh0": torch.empty(state_shape, **f32) if want_dh0 else None}
    for n, t in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta), ("dlog_alpha", log_alpha)):
        _ptr(out[n], n, torch.float32, t.shape)
    _ptr(out.get("dh0"), "dh0", torch.float32, state_shape)
    ws_bytes = gdr_chunk_bwd_workspace_size(p)
    if ws_bytes == 0:
        _check(lib.gdr_chunk_bwd(ctypes.byref(p), *([None] * 15), 0, None))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    _check(lib.gdr_chunk_bwd(
        ctypes.byref(p), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _ptr(beta, "beta"), _ptr(log_alpha, "log_alpha"),
        _ptr(states, "states", torch.float16 if q.dtype == torch.bfloat16 else torch.float32,
             (p.B, p.H_v, nc, p.d_k, p.d_v)),
        _ptr(d_o, "d_o", None, (p.B, p.T, p.H_v, p.d_v)), _ptr(dhT, "dhT", torch.float32, state_shape),
        _ptr(out["dq"], "dq"), _ptr(out["dk"], "dk"), _ptr(out["dv"], "dv"), _ptr(out["dbeta"], "dbeta"),
        _ptr(out["dlog_alpha"], "dlog_alpha"), _ptr(out["dh0"], "dh0"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out

"""Token-by-token fp64 gated delta rule -- TEST INFRASTRUCTURE ONLY.

Follows "Systolic Linear Attention: Co-Designing Tile-Grouped Gated Delta
Attention for TPUs", section 2.1,
Eq. (2): per token, decay the state by the diagonal gate F_t, take the
prediction error u_t = v_t - (F_t S_{t-1})^T k_t, write S_t = F_t S_{t-1} +
beta_t k_t u_t^T, and read out o_t = S_t^T q_t after the update.

Two independent implementations of the same definition:

* :func:`recurrence_c` calls ``liboracle.so`` (``gdr_oracle.c``), threaded over
  (batch, value head).  Used at large sizes.
* :func:`recurrence_np` is a numpy loop over tokens, vectorised over
  (batch, value head).  Used at small sizes and as the C code's twin.

Argument conventions (both functions):
  q, k       [B, T, H_k, d_k]  float32 (bf16 inputs are decoded to fp32 exactly)
  v          [B, T, H_v, d_v]
  beta       [B, T, H_v]  ([B, T, H_k] when beta_per_key_head)
  log_alpha  [B, T, H_k, G]  natural-log decay, channel i uses group i // (d_k // G)
  h0         [B, H_v, d_k, d_v] or None (zero state)
Returns (o [B, T, H_v, d_v], hT [B, H_v, d_k, d_v]) in float64.
Value head h_v reads key head h_v // (H_v // H_k) (contiguous value-head groups,
section 2.4.1 of the same paper).

:func:`layer_c` and :func:`layer_np` add the layer's sequence-level features
(same paper, Table 2: Z_c, mu, kappa_c; section 2.3, "Why chunk-level
momentum"): document resets (``reset`` [B, T], nonzero where a token starts a
new document: the state carried into it is discarded) and chunk-boundary
momentum with coefficient ``momentum`` over chunks of ``chunk`` tokens
counted from the first token:

    carry = kappa_c F_c S_{c-1},  Z_c = mu kappa_c Z_{c-1} + (S~_c - carry),
    S_c = carry + Z_c,

S~_c being the state after the chunk's last token, evolved token by token
from S_{c-1} (the outputs inside the chunk are read from that evolution),
F_c the product of the chunk's decays and kappa_c = 0 when a reset falls in
the chunk.  They return (o, hT, zT).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        f = lib.oracle_gdr_recurrence
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int] * 8 + [ctypes.c_void_p] * 8 + [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        g = lib.oracle_gdr_layer
        g.restype = ctypes.c_int
        g.argtypes = ([ctypes.c_int] * 8 + [ctypes.c_void_p] * 8 + [ctypes.c_int, ctypes.c_double] +
                      [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_int])
        _LIB = lib
    return _LIB


def _shapes(q, v, log_alpha):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = log_alpha.shape[3]
    return B, T, Hk, Hv, dk, dv, G


def recurrence_c(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False,
                 units=None, nthreads=None):
    """fp64 token recurrence in C.  ``units`` optionally lists b * H_v + h_v
    indices to evaluate; the rows of ``o``/``hT`` of other units stay zero."""
    B, T, Hk, Hv, dk, dv, G = _shapes(q, v, log_alpha)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    q, k, v, beta, log_alpha = f32(q), f32(k), f32(v), f32(beta), f32(log_alpha)
    h0a = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    o = np.zeros((B, T, Hv, dv), np.float64)
    hT = np.zeros((B, Hv, dk, dv), np.float64)
    ua = None if units is None else np.ascontiguousarray(units, dtype=np.int32)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = _lib().oracle_gdr_recurrence(
        B, T, Hk, Hv, dk, dv, G, int(bool(beta_per_key_head)),
        p(q), p(k), p(v), p(beta), p(log_alpha), p(h0a), p(o), p(hT),
        p(ua), 0 if ua is None else len(ua), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gdr_recurrence rejected the problem")
    return o, hT


def layer_c(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False, reset=None, momentum=0.0, chunk=0,
            z0=None, units=None, nthreads=None):
    """fp64 token recurrence with document resets and chunk-boundary momentum,
    in C.  Returns (o, hT, zT)."""
    B, T, Hk, Hv, dk, dv, G = _shapes(q, v, log_alpha)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    f64 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float64)
    q, k, v, beta, log_alpha = f32(q), f32(k), f32(v), f32(beta), f32(log_alpha)
    rs = None if reset is None else np.ascontiguousarray(np.asarray(reset) != 0, dtype=np.uint8)
    if rs is not None and rs.shape != (B, T):
        raise ValueError(f"reset has shape {rs.shape}, expected {(B, T)}")
    h0a, z0a = f64(h0), f64(z0)
    o = np.zeros((B, T, Hv, dv), np.float64)
    hT = np.zeros((B, Hv, dk, dv), np.float64)
    zT = np.zeros((B, Hv, dk, dv), np.float64)
    ua = None if units is None else np.ascontiguousarray(units, dtype=np.int32)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = _lib().oracle_gdr_layer(
        B, T, Hk, Hv, dk, dv, G, int(bool(beta_per_key_head)),
        p(q), p(k), p(v), p(beta), p(log_alpha), p(rs), p(h0a), p(z0a), int(chunk), float(momentum),
        p(o), p(hT), p(zT), p(ua), 0 if ua is None else len(ua), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gdr_layer rejected the problem")
    return o, hT, zT


def layer_np(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False, reset=None, momentum=0.0, chunk=0,
             z0=None):
    """fp64 token recurrence with document resets and chunk-boundary momentum,
    in numpy (small sizes).  Returns (o, hT, zT)."""
    B, T, Hk, Hv, dk, dv, G = _shapes(q, v, log_alpha)
    R = Hv // Hk
    key_of = np.arange(Hv) // R
    q = np.asarray(q, np.float64)[:, :, key_of]
    k = np.asarray(k, np.float64)[:, :, key_of]
    v = np.asarray(v, np.float64)
    la = np.repeat(np.asarray(log_alpha, np.float64)[:, :, key_of], dk // G, axis=3)
    beta = np.asarray(beta, np.float64)
    if beta_per_key_head:
        beta = beta[:, :, key_of]
    rs = np.zeros((B, T), bool) if reset is None else np.asarray(reset) != 0
    S = np.zeros((B, Hv, dk, dv)) if h0 is None else np.array(h0, np.float64)
    Z = np.zeros((B, Hv, dk, dv)) if z0 is None else np.array(z0, np.float64)
    o = np.zeros((B, T, Hv, dv))
    use_m = chunk > 0 and momentum != 0.0
    for c0 in range(0, T, chunk if use_m else max(T, 1)):
        c1 = min(c0 + chunk, T) if use_m else T
        S_in = S.copy()
        # kappa_c per batch row: no reset among the chunk's tokens
        kappa = ~rs[:, c0:c1].any(axis=1)
        for t in range(c0, c1):
            S = np.where(rs[:, t][:, None, None, None], 0.0, S)
            S = np.exp(la[:, t])[..., None] * S
            u = v[:, t] - np.einsum("bhij,bhi->bhj", S, k[:, t])
            S = S + beta[:, t, :, None, None] * k[:, t, :, :, None] * u[:, :, None, :]
            o[:, t] = np.einsum("bhij,bhi->bhj", S, q[:, t])
        if use_m:
            Fc = np.exp(la[:, c0:c1].sum(axis=1))                      # [B, Hv, dk]
            kap = kappa[:, None, None, None]
            carry = np.where(kap, Fc[..., None] * S_in, 0.0)
            Z = momentum * np.where(kap, Z, 0.0) + (S - carry)
            S = carry + Z
    return o, S, Z


def recurrence_np(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False):
    """fp64 token recurrence in numpy (small sizes)."""
    B, T, Hk, Hv, dk, dv, G = _shapes(q, v, log_alpha)
    R = Hv // Hk
    key_of = np.arange(Hv) // R
    q = np.asarray(q, np.float64)[:, :, key_of]          # [B, T, Hv, dk]
    k = np.asarray(k, np.float64)[:, :, key_of]
    v = np.asarray(v, np.float64)
    la = np.asarray(log_alpha, np.float64)[:, :, key_of]  # [B, T, Hv, G]
    la = np.repeat(la, dk // G, axis=3)                   # [B, T, Hv, dk]
    beta = np.asarray(beta, np.float64)
    if beta_per_key_head:
        beta = beta[:, :, key_of]
    S = np.zeros((B, Hv, dk, dv)) if h0 is None else np.array(h0, np.float64)
    o = np.zeros((B, T, Hv, dv))
    for t in range(T):
        S = np.exp(la[:, t])[..., None] * S                           # F_t S_{t-1}
        u = v[:, t] - np.einsum("bhij,bhi->bhj", S, k[:, t])          # v_t - (F_t S)^T k_t
        S = S + beta[:, t, :, None, None] * k[:, t, :, :, None] * u[:, :, None, :]
        o[:, t] = np.einsum("bhij,bhi->bhj", S, q[:, t])               # S_t^T q_t
    return o, S

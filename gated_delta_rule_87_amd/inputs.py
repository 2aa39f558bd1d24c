"""Seeded synthetic inputs and the workload registry.

This module only draws random numbers and encodes them; it holds none of the
gated-delta-rule arithmetic.  Both the GPU path and the CPU oracle consume
exactly the arrays it returns (the same bits), so neither side ever sees the
other's numbers.

Input recipe (one numpy ``Generator(PCG64(seed))`` per workload, full arrays in
C order, drawn in this order):

1. q_raw [B, T, H_k, d_k] ~ N(0, 1), then L2-normalised over d_k (fp64, no eps);
2. k_raw likewise;
3. v [B, T, H_v, d_v] ~ N(0, 1);
4. beta logits [B, T, H_beta] ~ N(0, 1), beta = s_beta * sigmoid(logit)
   (s_beta = 1 for the Gated DeltaNet / KDA gate; 2 for the Systolic Linear
   Attention write gate, section 2.3 and Table 2: beta in (0, 2));
5. decay logits [B, T, H_k, G] ~ N(mu, sigma) (sigma a standard deviation),
   log_alpha = logsigmoid(logit) = -log1p(exp(-logit)).

The fp64 values are cast fp64 -> fp32 (round to nearest even) and, for bf16
workloads, fp32 -> bf16 (round to nearest even).  bf16 arrays are returned as
``uint16`` bit patterns; :func:`decode` turns any returned array into fp32
(exact for bf16).  The unit-norm of q and k therefore holds up to the final
rounding only; nothing renormalises it.

The distributions are those of the Systolic Linear Attention paper's layer
(section 2.1: unit-norm queries and keys, sigmoid write gate, log-sigmoid
forget gate; section 2.3 for the four-tile grouped gate and grouped value
heads).  No public dataset is involved.
"""
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    chunk: int
    G: int                    # decay groups: 1 scalar, d_k per channel, else tiles
    dtype: str                # "f32" or "bf16" for q, k, v, beta, log_alpha
    alpha_mu: float = 3.0
    alpha_sigma: float = 1.0
    beta_per_key_head: bool = False
    beta_scale: float = 1.0   # s_beta: beta = s_beta * sigmoid(logit)
    solves: tuple = ("exact",)
    neumann_order: int = 4
    neumann_residual: int = 1
    seed: int = 20261203
    description: str = field(default="", compare=False)

    @property
    def H_beta(self):
        return self.H_k if self.beta_per_key_head else self.H_v

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    0: Workload("gdn_f32_tiny", 1, 256, 2, 2, 64, 64, 64, 1, "f32", seed=20261203,
                description="scalar-gate GDN, fp32, B1 T256 H2 d64 C64"),
    1: Workload("gdn_bf16", 4, 4096, 16, 16, 128, 128, 64, 1, "bf16", seed=20261204,
                description="scalar-gate GDN, bf16 in / fp32 out, B4 T4096 H16 d128 C64"),
    2: Workload("kda_bf16", 2, 8192, 32, 32, 128, 128, 64, 128, "bf16", seed=20261205,
                description="per-channel-gate KDA, bf16 in / fp32 out, B2 T8192 H32 d128 C64"),
    3: Workload("sla_gva_bf16", 2, 16384, 8, 32, 256, 128, 64, 4, "bf16", seed=20261206,
                description="widened keys d_k=256, 8 key heads x 4 value heads, G=4 tiles of 64, B2 T16384 C64"),
    4: Workload("kda_stress_c128", 1, 32768, 16, 16, 128, 128, 128, 128, "bf16",
                alpha_mu=1.0, alpha_sigma=2.0, solves=("exact", "neumann"), seed=20261207,
                description="per-channel strong decay logsigmoid(N(1,2)), B1 T32768 H16 d128 C128"),
}


def f64_to_bf16_bits(x):
    """fp64 -> fp32 (RNE) -> bf16 (RNE), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def decode(a):
    """fp32 view of an array returned by :func:`make_inputs` (exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return a.astype(np.float32, copy=False)


def encode(x, dtype):
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _unit(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def make_inputs(w: Workload, seed=None, T=None, B=None):
    """Draw one workload's inputs.  Returns a dict of arrays in the storage
    encoding (uint16 bf16 bits or float32): q, k, v, beta, log_alpha.
    ``T``/``B`` override the workload's sequence length / batch (the draw
    order is unchanged, so a shorter T is not a prefix of the longer one)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B = w.B if B is None else B
    T = w.T if T is None else T
    q = _unit(rng.standard_normal((B, T, w.H_k, w.d_k)))
    k = _unit(rng.standard_normal((B, T, w.H_k, w.d_k)))
    v = rng.standard_normal((B, T, w.H_v, w.d_v))
    beta_logit = rng.standard_normal((B, T, w.H_beta))
    alpha_logit = rng.normal(w.alpha_mu, w.alpha_sigma, (B, T, w.H_k, w.G))
    beta = w.beta_scale / (1.0 + np.exp(-beta_logit))
    log_alpha = -np.log1p(np.exp(-alpha_logit))
    return {
        "q": encode(q, w.dtype),
        "k": encode(k, w.dtype),
        "v": encode(v, w.dtype),
        "beta": encode(beta, w.dtype),
        "log_alpha": encode(log_alpha, w.dtype),
    }


def make_resets(B, T, mean_doc_len, seed, extra=()):
    """Document starts for packed sequences: uint8 [B, T], 1 where a token
    starts a new document.  Document lengths are drawn from a geometric
    distribution with the given mean (numpy Generator(PCG64(seed))); ``extra``
    lists (b, t) positions that are also marked (to place starts on chunk
    edges, on token 0 or twice in one 16-token block)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    r = np.zeros((B, T), np.uint8)
    for b in range(B):
        t = int(rng.geometric(1.0 / mean_doc_len))
        while t < T:
            r[b, t] = 1
            t += int(rng.geometric(1.0 / mean_doc_len))
    for b, t in extra:
        if 0 <= t < T:
            r[b, t] = 1
    return r


def decoded(inputs):
    """All five arrays as fp32 (exact decode)."""
    return {name: decode(a) for name, a in inputs.items()}

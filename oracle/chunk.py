"""Chunkwise WY form of the gated delta rule in fp64 -- TEST INFRASTRUCTURE ONLY.

Written from "Systolic Linear Attention: Co-Designing Tile-Grouped Gated Delta
Attention for TPUs":

* Table 2 (notation) defines, per chunk of C tokens and one key head:
  the in-chunk cumulative log-decay Lambda_{t,i} = sum_{s<=t} log f_{s,i};
  the decayed queries/keys Qbar = (P_{t<-0} q_t)^T, Kbar = (P_{t<-0} k_t)^T and
  carried keys Khat = (P_{C<-t} k_t)^T; the strictly lower-triangular Gram
  M_c, the lower-triangular (diagonal included) score matrix L_c and the WY
  inverse A_c = (I + M_c)^{-1}; the WY factors U_c = diag(beta) A_c V_c,
  W_c = diag(beta) A_c Kbar_c and the chunk writes E_c = U_c - W_c S_{c-1}.
* Section 2.2, "Bottleneck 2", gives the Gram entries
  (M_c)_{t,j} = 1[t > j] beta_j sum_i exp(Lambda_{t,i} - Lambda_{j,i}) k_{t,i} k_{j,i};
  L_c has the same form with q_t in place of k_t, 1[t >= j] and no beta
  (the tile masks Psi_g of Table 2, with one decay per channel).
* Section 2.3, the state increment Delta S_c = Khat_c^T E_c, so the next
  boundary state is S_c = F_c S_{c-1} + Khat_c^T E_c with F_c = diag(exp(Lambda_C)).
* Section 2.4.2, the unrolled intra-chunk state
  S~_t = P_{t<-0} S_{c-1} + sum_{j<=t} beta_j (P_{t<-j} k_j) u_j^T;  reading it
  out with o_t = S~_t^T q_t gives the chunk output O_c = Qbar_c S_{c-1} + L_c E_c.

In-chunk inverses:

* :func:`exact_inverse` is the plain definition, ``inv(I + M)``.
* :func:`block_doubling_inverse` is the recursive block-doubling of section
  2.4.3 (merge two diagonal-block inverses with two products per merge).
  Exact algebra, pinned against ``exact_inverse``.
* :func:`neumann_inverse` is the truncated Neumann series of the
  paper "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
  Approximation for Quantized Gated DeltaNet" (core claim and Fig. 5): X = sum_{s=0}^{m} (-M)^s ("order m" keeps powers 0..m, the reading
  under which ||A||^{m+1}/(1-||A||) bounds the tail), followed by r parallel
  residual corrections X <- X + X (I - (I + M) X).
* :func:`block_neumann_inverse` is the block-Jacobi form of section 2.4.3's
  block-Neumann factorisation, sum_{s<terms} (-N)^s D_blk^{-1}; with
  16-row blocks and two terms it is the 1-Step Neumann inverse
  A_N1 = (I - N) D_blk^{-1} (``solve="block_neumann"``, order 1).

Document resets and chunk-boundary momentum (Table 2: Z_c, mu, kappa_c;
section 2.3, "Why chunk-level momentum"): a reset at token t discards the
state carried into t.  Within a chunk the tokens then fall into segments
(segment of t = number of resets at or before t in the chunk); Lambda is
cumulated from the start of each token's segment; pairs (t, j) of different
segments get no decay factor (their Gram and score entries are zero); only
segment 0 sees the chunk-entry state (rows of Qbar and Kbar of later
segments are zero); only the last segment carries into the chunk's end (rows
of Khat before it are zero); F_c is zero when the chunk holds a reset, and
so is kappa_c.  Momentum then acts on the increment Delta S_c = Khat^T E_c:
Z_c = mu kappa_c Z_{c-1} + Delta S_c, S_c = F_c S_{c-1} + Z_c.

Everything is fp64 numpy; exponentials are only taken of Lambda_t - Lambda_j
on the causal side t >= j (masked before exp), i.e. of non-positive numbers.
"""
import numpy as np


# ----------------------------------------------------------------- inverses
def exact_inverse(M):
    """(I + M)^{-1} by the plain definition."""
    n = M.shape[0]
    return np.linalg.inv(np.eye(n) + M)


def block_doubling_inverse(M):
    """(I + M)^{-1} for strictly lower-triangular M by recursive block doubling:
    inv([[I+M11, 0], [M21, I+M22]]) = [[A11, 0], [-A22 M21 A11, A22]]."""
    n = M.shape[0]
    if n == 1:
        return np.ones((1, 1))
    h = n // 2
    A11 = block_doubling_inverse(M[:h, :h])
    A22 = block_doubling_inverse(M[h:, h:])
    out = np.zeros((n, n))
    out[:h, :h] = A11
    out[h:, h:] = A22
    out[h:, :h] = -A22 @ (M[h:, :h] @ A11)
    return out


def neumann_inverse(M, order, residual_steps=0):
    """Truncated Neumann series sum_{s=0}^{order} (-M)^s, then ``residual_steps``
    residual corrections X <- X + X (I - (I + M) X)."""
    n = M.shape[0]
    eye = np.eye(n)
    X = eye.copy()
    P = eye.copy()
    for _ in range(order):
        P = -(P @ M)
        X = X + P
    for _ in range(residual_steps):
        X = X + X @ (eye - (eye + M) @ X)
    return X


def block_neumann_inverse(M, block, terms):
    """sum_{s=0}^{terms-1} (-N)^s D^{-1} with D the block-diagonal part of I + M
    (blocks of ``block`` rows) and N = D^{-1} (I + M - D)."""
    n = M.shape[0]
    IM = np.eye(n) + M
    D = np.zeros_like(IM)
    for s in range(0, n, block):
        D[s:s + block, s:s + block] = IM[s:s + block, s:s + block]
    Dinv = np.linalg.inv(D)
    N = Dinv @ (IM - D)
    X = np.zeros_like(IM)
    P = np.eye(n)
    for _ in range(terms):
        X = X + P
        P = -(P @ N)
    return X @ Dinv


BLOCK_NEUMANN_ROWS = 16   # B_blk of the 1-Step Neumann setting in section 2.4.3


def invert(M, solve="exact", order=4, residual_steps=1):
    """``order`` m: the Neumann series keeps powers 0..m of -M (then
    ``residual_steps`` corrections); the block-Neumann form keeps powers 0..m
    of -N (m = 1 is the pages' 1-Step Neumann, (I - N) D^{-1}; no residual
    step)."""
    if solve == "exact":
        return exact_inverse(M)
    if solve == "neumann":
        return neumann_inverse(M, order, residual_steps)
    if solve == "block_neumann":
        return block_neumann_inverse(M, BLOCK_NEUMANN_ROWS, order + 1)
    if solve == "block_doubling":
        return block_doubling_inverse(M)
    raise ValueError(solve)


# ------------------------------------------------------------ chunk pieces
def chunk_pieces(q, k, beta, la, reset=None):
    """Per-chunk quantities of Table 2 for one key head and one chunk.

    q, k: [n, d_k]; beta: [n]; la: [n, d_k] per-channel log decay (groups
    already broadcast); reset: [n] or None, nonzero where a token starts a new
    document.  Returns a dict with Lambda, Qbar, Kbar, Khat, gamma (= diag of
    F_c), kappa, G (the beta-free strictly lower Gram), M = G diag(beta) and L.
    """
    n = q.shape[0]
    rs = np.zeros(n, bool) if reset is None else np.asarray(reset) != 0
    seg = np.cumsum(rs)                                         # segment of each token
    Lam = np.zeros_like(np.asarray(la, np.float64))
    run = np.zeros(la.shape[1])
    for t in range(n):                                          # cumulated within the segment
        run = (0.0 if rs[t] else run) + la[t]
        Lam[t] = run
    t_idx = np.arange(n)
    same = seg[:, None] == seg[None, :]
    causal = (t_idx[:, None] >= t_idx[None, :]) & same          # t >= j, same document
    diff = Lam[:, None, :] - Lam[None, :, :]                    # Lambda_t - Lambda_j
    P = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
    kk = np.einsum("ti,ji,tji->tj", k, k, P)
    qk = np.einsum("ti,ji,tji->tj", q, k, P)
    strict = (t_idx[:, None] > t_idx[None, :]) & same
    G = np.where(strict, kk, 0.0)
    first = (seg == 0)[:, None]                                 # tokens that see the chunk-entry state
    last = (seg == seg[-1])[:, None] if n else first           # tokens that carry into the chunk's end
    kappa = not rs.any()
    return {
        "Lambda": Lam,
        "Qbar": np.where(first, q * np.exp(np.where(first, Lam, 0.0)), 0.0),
        "Kbar": np.where(first, k * np.exp(np.where(first, Lam, 0.0)), 0.0),
        "Khat": np.where(last, k * np.exp(np.where(last, Lam[-1][None, :] - Lam, 0.0)), 0.0),
        "gamma": np.exp(Lam[-1]) if kappa else np.zeros(la.shape[1]),
        "kappa": kappa,
        "G": G,
        "M": G * beta[None, :],
        "L": np.where(causal, qk, 0.0),
    }


def _expand(q, k, log_alpha, beta, beta_per_key_head, b, hv, Hv, Hk):
    R = Hv // Hk
    hk = hv // R
    dk = q.shape[3]
    G = log_alpha.shape[3]
    qh = np.asarray(q[b, :, hk], np.float64)
    kh = np.asarray(k[b, :, hk], np.float64)
    la = np.repeat(np.asarray(log_alpha[b, :, hk], np.float64), dk // G, axis=1)
    bh = np.asarray(beta[b, :, hk] if beta_per_key_head else beta[b, :, hv], np.float64)
    return qh, kh, la, bh


def chunk_forward(q, k, v, beta, log_alpha, h0=None, chunk=64, solve="exact",
                  order=4, residual_steps=1, beta_per_key_head=False, units=None,
                  reset=None, momentum=0.0, z0=None, return_z=False):
    """Chunkwise WY forward in fp64 with the chosen in-chunk inverse.

    Shapes as in :mod:`oracle.recurrence`; a final chunk shorter than
    ``chunk`` is processed at its own length.  ``reset`` [B, T] marks tokens
    that start a new document; ``momentum`` is mu of the chunk-boundary
    momentum, ``z0`` its initial buffer.  Returns (o, hT), or (o, hT, zT) with
    ``return_z``, in float64; with ``units`` only those b * H_v + h_v entries
    are filled.
    """
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    o = np.zeros((B, T, Hv, dv))
    hT = np.zeros((B, Hv, dk, dv))
    zT = np.zeros((B, Hv, dk, dv))
    todo = range(B * Hv) if units is None else units
    for u in todo:
        b, hv = divmod(int(u), Hv)
        qh, kh, la, bh = _expand(q, k, log_alpha, beta, beta_per_key_head, b, hv, Hv, Hk)
        vh = np.asarray(v[b, :, hv], np.float64)
        rb = None if reset is None else np.asarray(reset[b])
        S = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, hv], np.float64)
        Z = np.zeros((dk, dv)) if z0 is None else np.array(z0[b, hv], np.float64)
        for s in range(0, T, chunk):
            e = min(s + chunk, T)
            pc = chunk_pieces(qh[s:e], kh[s:e], bh[s:e], la[s:e], None if rb is None else rb[s:e])
            A = invert(pc["M"], solve, order, residual_steps)
            Bd = bh[s:e][:, None]
            U = Bd * (A @ vh[s:e])                 # U_c = diag(beta) A_c V_c
            W = Bd * (A @ pc["Kbar"])              # W_c = diag(beta) A_c Kbar_c
            E = U - W @ S                          # E_c = U_c - W_c S_{c-1}
            o[b, s:e, hv] = pc["Qbar"] @ S + pc["L"] @ E
            dS = pc["Khat"].T @ E                  # Delta S_c
            if momentum != 0.0:
                Z = momentum * (Z if pc["kappa"] else 0.0) + dS
                S = pc["gamma"][:, None] * S + Z
            else:
                S = pc["gamma"][:, None] * S + dS
        hT[b, hv] = S
        zT[b, hv] = Z
    return (o, hT, zT) if return_z else (o, hT)


def chunk_stage_matrices(q, k, beta, log_alpha, chunk, solve="exact", order=4,
                         residual_steps=1, beta_per_key_head=False):
    """A_c per beta head and L_c per key head for every chunk, padded to C x C.

    Returns (A [B, H_beta, N_c, C, C], L [B, H_k, N_c, C, C]) where H_beta is
    the number of beta heads (H_v, or H_k when beta is per key head).  In a
    short final chunk the padded rows/columns hold the identity in A and zeros
    in L (what a zero-beta, zero-decay padding token produces).
    """
    B, T, Hk, dk = q.shape
    Hb = beta.shape[2]
    R = Hb // Hk
    G = log_alpha.shape[3]
    Nc = (T + chunk - 1) // chunk
    A_all = np.zeros((B, Hb, Nc, chunk, chunk))
    L_all = np.zeros((B, Hk, Nc, chunk, chunk))
    for b in range(B):
        for hk in range(Hk):
            qh = np.asarray(q[b, :, hk], np.float64)
            kh = np.asarray(k[b, :, hk], np.float64)
            la = np.repeat(np.asarray(log_alpha[b, :, hk], np.float64), dk // G, axis=1)
            for c in range(Nc):
                s, e = c * chunk, min(c * chunk + chunk, T)
                n = e - s
                pc = chunk_pieces(qh[s:e], kh[s:e], np.ones(n), la[s:e])
                L_all[b, hk, c, :n, :n] = pc["L"]
                for hb in range(hk * R, (hk + 1) * R):
                    bh = np.asarray(beta[b, s:e, hb], np.float64)
                    A_all[b, hb, c] = np.eye(chunk)
                    A_all[b, hb, c, :n, :n] = invert(pc["G"] * bh[None, :], solve, order, residual_steps)
    return A_all, L_all

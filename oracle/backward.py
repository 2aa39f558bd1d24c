"""Gradients of the gated delta rule in fp64 -- TEST INFRASTRUCTURE ONLY.

Two independent evaluations of the vector-Jacobian product of the forward
pass (Systolic Linear Attention, section 2.1, Eq. (2); backward pass,
section 2.5):

* :func:`vjp_autograd`: reverse-mode differentiation (torch autograd, fp64,
  CPU) of the plain token recurrence written out step by step -- decay,
  prediction error, rank-one write, readout -- as in oracle.recurrence.  This
  is *the* gradient oracle: the gradient of the definition itself.
* :func:`vjp_chunk`: the chunkwise backward the pages describe, written out
  in numpy: the forward keeps only the chunk-entry states S_{c-1}; the
  reverse pass over chunks recomputes M_c, L_c, A_c and the unscaled writes
  E~_c = A_c (V_c - Kbar_c S_{c-1}), and with dE_c the gradient of the chunk
  writes forms D_c = A_c^T diag(beta_c) dE_c and dM_c = -tril_{-1}(D_c E~_c^T)
  (section 2.5); every other adjoint follows by the chain rule through the
  chunk quantities of Table 2.  Pinned against vjp_autograd.

Arguments: q, k [B,T,H_k,d_k], v [B,T,H_v,d_v], beta [B,T,H_beta],
log_alpha [B,T,H_k,G], h0 [B,H_v,d_k,d_v] or None, do [B,T,H_v,d_v] (the
upstream gradient of o), dhT [B,H_v,d_k,d_v] or None (of the final state).
Returns a dict of fp64 arrays: dq, dk, dv, dbeta, dlog_alpha, dh0.
"""
import numpy as np
import torch


def _forward_torch(q, k, v, beta, la, h0, beta_per_key_head):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = la.shape[3]
    R = Hv // Hk
    key_of = torch.arange(Hv) // R
    qe, ke = q[:, :, key_of], k[:, :, key_of]                       # [B, T, Hv, dk]
    lae = la[:, :, key_of].repeat_interleave(dk // G, dim=3)        # [B, T, Hv, dk]
    be = beta[:, :, key_of] if beta_per_key_head else beta          # [B, T, Hv]
    S = torch.zeros(B, Hv, dk, dv, dtype=torch.float64) if h0 is None else h0
    outs = []
    for t in range(T):
        S = torch.exp(lae[:, t])[..., None] * S                      # decay
        u = v[:, t] - torch.einsum("bhij,bhi->bhj", S, ke[:, t])      # prediction error
        S = S + be[:, t, :, None, None] * ke[:, t, :, :, None] * u[:, :, None, :]   # rank-one write
        outs.append(torch.einsum("bhij,bhi->bhj", S, qe[:, t]))      # readout after the update
    return torch.stack(outs, dim=1), S


def vjp_autograd(q, k, v, beta, log_alpha, h0, do, dhT=None, beta_per_key_head=False):
    t64 = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    tq, tk, tv, tb, tl = (t64(a) for a in (q, k, v, beta, log_alpha))
    th = t64(h0) if h0 is not None else None
    o, hT = _forward_torch(tq, tk, tv, tb, tl, th, beta_per_key_head)
    loss = (o * torch.tensor(np.asarray(do, np.float64))).sum()
    if dhT is not None:
        loss = loss + (hT * torch.tensor(np.asarray(dhT, np.float64))).sum()
    leaves = [tq, tk, tv, tb, tl] + ([th] if th is not None else [])
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    names = ["dq", "dk", "dv", "dbeta", "dlog_alpha"] + (["dh0"] if th is not None else [])
    out = {n: (g.numpy() if g is not None else np.zeros(x.shape)) for n, g, x in zip(names, grads, leaves)}
    if th is None:
        out["dh0"] = None
    return out


def _chunk_quantities(q, k, beta, la):
    """Table 2's per-chunk quantities for one chunk, one value head."""
    n = q.shape[0]
    Lam = np.cumsum(la, axis=0)
    t = np.arange(n)
    causal = t[:, None] >= t[None, :]
    diff = np.where(causal[:, :, None], Lam[:, None, :] - Lam[None, :, :], 0.0)
    P = np.where(causal[:, :, None], np.exp(diff), 0.0)               # P[t, j, i] = e^{Lambda_ti - Lambda_ji}, t >= j
    strict = t[:, None] > t[None, :]
    G = np.where(strict, np.einsum("ti,ji,tji->tj", k, k, P), 0.0)
    L = np.where(causal, np.einsum("ti,ji,tji->tj", q, k, P), 0.0)
    M = G * beta[None, :]
    A = np.linalg.inv(np.eye(n) + M)
    return {"Lam": Lam, "P": P, "G": G, "L": L, "M": M, "A": A, "gamma": np.exp(Lam[-1]),
            "Qbar": q * np.exp(Lam), "Kbar": k * np.exp(Lam), "Khat": k * np.exp(Lam[-1][None, :] - Lam)}


def vjp_chunk(q, k, v, beta, log_alpha, h0, do, dhT=None, chunk=64, beta_per_key_head=False):
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    G = log_alpha.shape[3]
    R = Hv // Hk
    f = lambda a: np.asarray(a, np.float64)
    q, k, v, beta, log_alpha, do = f(q), f(k), f(v), f(beta), f(log_alpha), f(do)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dbeta": np.zeros_like(beta),
           "dlog_alpha": np.zeros_like(log_alpha), "dh0": np.zeros((B, Hv, dk, dv))}
    starts = list(range(0, T, chunk))
    for b in range(B):
        for hv in range(Hv):
            hk = hv // R
            hb = hk if beta_per_key_head else hv
            qh, kh, vh = q[b, :, hk], k[b, :, hk], v[b, :, hv]
            la = np.repeat(log_alpha[b, :, hk], dk // G, axis=1)
            bh = beta[b, :, hb]
            # forward, keeping the chunk-entry states only
            S = np.zeros((dk, dv)) if h0 is None else f(h0[b, hv]).copy()
            entry = []
            for s in starts:
                e = min(s + chunk, T)
                c = _chunk_quantities(qh[s:e], kh[s:e], bh[s:e], la[s:e])
                entry.append(S.copy())
                Et = c["A"] @ (vh[s:e] - c["Kbar"] @ S)                 # unscaled writes E~
                S = c["gamma"][:, None] * S + c["Khat"].T @ (bh[s:e][:, None] * Et)
            # reverse over chunks, recomputing each chunk
            dS = np.zeros((dk, dv)) if dhT is None else f(dhT[b, hv]).copy()
            for ci in reversed(range(len(starts))):
                s = starts[ci]
                e = min(s + chunk, T)
                qc, kc, bc = qh[s:e], kh[s:e], bh[s:e]
                c = _chunk_quantities(qc, kc, bc, la[s:e])
                Sp = entry[ci]
                Y = vh[s:e] - c["Kbar"] @ Sp
                Et = c["A"] @ Y
                E = bc[:, None] * Et
                dO = do[b, s:e, hv]
                # O = Qbar S + L E ; S' = diag(gamma) S + Khat^T E
                dE = c["L"].T @ dO + c["Khat"] @ dS
                dQbar = dO @ Sp.T
                dL = np.where(np.tril(np.ones_like(c["L"])) > 0, dO @ E.T, 0.0)
                dKhat = E @ dS.T
                dgamma = np.sum(Sp * dS, axis=1)
                dSp = c["gamma"][:, None] * dS + c["Qbar"].T @ dO
                # E = diag(beta) E~ ; E~ = A Y ; A = (I + M)^{-1}
                dbeta_c = np.sum(dE * Et, axis=1)
                D = c["A"].T @ (bc[:, None] * dE)                       # section 2.5: D = A^T diag(beta) dE
                dM = -np.tril(D @ Et.T, -1)                              # section 2.5: dM = -tril_{-1}(D E~^T)
                # Y = V - Kbar S
                out["dv"][b, s:e, hv] += D
                dKbar = -D @ Sp.T
                dSp -= c["Kbar"].T @ D
                # M = G diag(beta)
                dG = dM * bc[None, :]
                dbeta_c += np.sum(dM * c["G"], axis=0)
                out["dbeta"][b, s:e, hb] += dbeta_c
                # G, L, Qbar, Kbar, Khat, gamma -> q, k, Lambda
                P = c["P"]
                dq = dQbar * np.exp(c["Lam"]) + np.einsum("tj,ji,tji->ti", dL, kc, P)
                dkk = (dKbar * np.exp(c["Lam"]) + dKhat * np.exp(c["Lam"][-1][None, :] - c["Lam"])
                       + np.einsum("tj,ji,tji->ti", dG, kc, P)            # G: row side
                       + np.einsum("tj,ti,tji->ji", dG, kc, P)            # G: column side
                       + np.einsum("tj,ti,tji->ji", dL, qc, P))           # L: column side
                wG = np.einsum("tj,ti,ji,tji->tji", dG, kc, kc, P) + np.einsum("tj,ti,ji,tji->tji", dL, qc, kc, P)
                dLam = wG.sum(axis=1) - wG.sum(axis=0)                   # d/dLambda_t and -d/dLambda_j
                dLam += dQbar * c["Qbar"] + dKbar * c["Kbar"] - dKhat * c["Khat"]
                dLam[-1] += np.sum(dKhat * c["Khat"], axis=0) + dgamma * c["gamma"]
                out["dq"][b, s:e, hk] += dq
                out["dk"][b, s:e, hk] += dkk
                dla = np.cumsum(dLam[::-1], axis=0)[::-1]                 # Lambda_t = sum_{s<=t} log alpha_s
                out["dlog_alpha"][b, s:e, hk] += dla.reshape(e - s, G, dk // G).sum(axis=2)
                dS = dSp
            out["dh0"][b, hv] = dS
    if h0 is None:
        out["dh0"] = None
    return out

"""Pins for the token-recurrence oracle (helper module, imported by tests).

Every pin takes a recurrence implementation
``fn(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False) -> (o, hT)``
and raises AssertionError when it disagrees with something the pages or the
mathematics fix independently of the recurrence loop: hand-worked examples,
closed forms, invariants.  The recurrence is Systolic Linear Attention,
section 2.1, Eq. (2); the invariants and closed forms below are derived from
it by hand (derivations in each docstring).

The same pins run against the C oracle, the numpy twin, and deliberately
broken copies of the recurrence (tests/test_oracle_mutations.py), which must
each fail at least one pin.
"""
import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_problem(seed, B=1, T=5, Hk=1, Hv=1, dk=4, dv=3, G=None, h0=False, bkh=False):
    r = _rng(seed)
    G = dk if G is None else G
    q = _f32(_unit(r.standard_normal((B, T, Hk, dk))))
    k = _f32(_unit(r.standard_normal((B, T, Hk, dk))))
    v = _f32(r.standard_normal((B, T, Hv, dv)))
    beta = _f32(r.uniform(0.1, 1.9, (B, T, Hk if bkh else Hv)))
    la = _f32(-np.log1p(np.exp(-r.normal(1.0, 1.0, (B, T, Hk, G)))))
    s0 = _f32(r.standard_normal((B, Hv, dk, dv))).astype(np.float64) if h0 else None
    return q, k, v, beta, la, s0


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------- hand-worked
def pin_hand_worked(fn):
    """Three tokens, d_k = d_v = 2, worked by hand from Eq. (2).

    k = (1,0), (0.6,0.8), (0,1); q = (1,0), (0,1), (0.6,0.8);
    v = (2,0), (0,4), (1,1); beta = 1/2, 1, 1/4; S_0 = 0.
    Scalar gate alpha_2 = alpha_3 = 1/2 (alpha_1 acts on the zero state):
      t=1: u=(2,0), S_1=[[1,0],[0,0]], o_1=(1,0)
      t=2: F S_1=[[.5,0],[0,0]], (F S)^T k_2=(.3,0), u=(-.3,4),
           S_2=[[.32,2.4],[-.24,3.2]], o_2=S_2[1]=(-.24,3.2)
      t=3: F S_2=[[.16,1.2],[-.12,1.6]], u=(1.12,-.6),
           S_3=[[.16,1.2],[.16,1.45]], o_3=.6*S_3[0]+.8*S_3[1]=(.224,1.88)
    Per-channel gate f_2=(1/2,1/4), f_3=(1,1/2): t=1,2 as above (row 1 of
    S_1 is zero); t=3: F S_2=[[.32,2.4],[-.12,1.6]], u=(1.12,-.6),
    S_3=[[.32,2.4],[.16,1.45]], o_3=(.32,2.6).
    Inputs are fp32, so 0.6, 0.8 and log(1/2) carry ~1e-8 rounding: tol 1e-6.
    """
    k = _f32([[1, 0], [0.6, 0.8], [0, 1]]).reshape(1, 3, 1, 2)
    q = _f32([[1, 0], [0, 1], [0.6, 0.8]]).reshape(1, 3, 1, 2)
    v = _f32([[2, 0], [0, 4], [1, 1]]).reshape(1, 3, 1, 2)
    beta = _f32([0.5, 1.0, 0.25]).reshape(1, 3, 1)
    la = _f32(np.log([1.0, 0.5, 0.5])).reshape(1, 3, 1, 1)
    o, hT = fn(q, k, v, beta, la)
    _close(o[0, :, 0], [[1, 0], [-0.24, 3.2], [0.224, 1.88]], 1e-6, "hand scalar o")
    _close(hT[0, 0], [[0.16, 1.2], [0.16, 1.45]], 1e-6, "hand scalar hT")
    la = _f32(np.log([[1.0, 1.0], [0.5, 0.25], [1.0, 0.5]])).reshape(1, 3, 1, 2)
    o, hT = fn(q, k, v, beta, la)
    _close(o[0, :, 0], [[1, 0], [-0.24, 3.2], [0.32, 2.6]], 1e-6, "hand per-channel o")
    _close(hT[0, 0], [[0.32, 2.4], [0.16, 1.45]], 1e-6, "hand per-channel hT")


# --------------------------------------------------------------- closed forms
def pin_two_token(fn):
    """S_0 = 0, two tokens, D_2 = diag(f_2) (f_1 acts on the zero state):
    o_1 = beta_1 (q_1.k_1) v_1;  u_2 = v_2 - beta_1 (k_2^T D_2 k_1) v_1;
    S_2 = beta_1 D_2 k_1 v_1^T + beta_2 k_2 u_2^T;
    o_2 = beta_1 (q_2^T D_2 k_1) v_1 + beta_2 (q_2.k_2) u_2.
    Checked for G in {1, 2, d_k}, with two value heads per key head."""
    dk = 6
    for G in (1, 2, dk):
        q, k, v, beta, la, _ = random_problem(11 + G, T=2, Hk=1, Hv=2, dk=dk, dv=3, G=G)
        o, hT = fn(q, k, v, beta, la)
        f2 = np.repeat(np.exp(la[0, 1, 0].astype(np.float64)), dk // G)
        q1, q2 = q[0, 0, 0].astype(np.float64), q[0, 1, 0].astype(np.float64)
        k1, k2 = k[0, 0, 0].astype(np.float64), k[0, 1, 0].astype(np.float64)
        for hv in range(2):
            v1, v2 = v[0, 0, hv].astype(np.float64), v[0, 1, hv].astype(np.float64)
            b1, b2 = float(beta[0, 0, hv]), float(beta[0, 1, hv])
            o1 = b1 * (q1 @ k1) * v1
            u2 = v2 - b1 * (k2 @ (f2 * k1)) * v1
            S2 = b1 * np.outer(f2 * k1, v1) + b2 * np.outer(k2, u2)
            o2 = b1 * (q2 @ (f2 * k1)) * v1 + b2 * (q2 @ k2) * u2
            _close(o[0, 0, hv], o1, TOL, f"two-token o1 G={G}")
            _close(o[0, 1, hv], o2, TOL, f"two-token o2 G={G}")
            _close(hT[0, hv], S2, TOL, f"two-token S2 G={G}")


def pin_one_token_h0(fn):
    """One token from a nonzero state: S_1 = F_1 h0 + beta k (v - (F_1 h0)^T k)^T,
    o_1 = S_1^T q."""
    dk = 5
    q, k, v, beta, la, h0 = random_problem(3, T=1, dk=dk, dv=4, G=dk, h0=True)
    o, hT = fn(q, k, v, beta, la, h0)
    f = np.exp(la[0, 0, 0].astype(np.float64))
    Fh = f[:, None] * h0[0, 0]
    kk = k[0, 0, 0].astype(np.float64)
    u = v[0, 0, 0] - Fh.T @ kk
    S1 = Fh + float(beta[0, 0, 0]) * np.outer(kk, u)
    _close(hT[0, 0], S1, TOL, "one-token S1")
    _close(o[0, 0, 0], S1.T @ q[0, 0, 0].astype(np.float64), TOL, "one-token o1")


# ----------------------------------------------------------------- invariants
def pin_orthonormal_recall(fn):
    """beta = 1, alpha = 1, orthonormal keys: every stored value is recalled
    exactly (S_T^T k_j = v_j), reading with q_t = k_t returns v_t, and writing
    an already-used key again recalls the newest value.  Keys are the rows of
    a 4x4 Hadamard matrix / 2 (exact in fp32)."""
    H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]) / 2.0
    order = [0, 2, 3, 1, 2]          # key 2 is rewritten last
    k = _f32(H4[order]).reshape(1, 5, 1, 4)
    q = k.copy()
    v = _f32(_rng(5).standard_normal((1, 5, 1, 3)))
    beta = np.ones((1, 5, 1), np.float32)
    la = np.zeros((1, 5, 1, 1), np.float32)
    o, hT = fn(q, k, v, beta, la)
    _close(o[0, :, 0], v[0, :, 0], 1e-12, "recall o_t = v_t")
    S = hT[0, 0]
    newest = {}
    for t, key in enumerate(order):
        newest[key] = t
    for key, t in newest.items():
        _close(S.T @ H4[key], v[0, t, 0], 1e-12, f"recall key {key}")


def pin_no_write(fn):
    """beta = 0 and alpha = 1: the state never changes, S_t = S_0 and
    o_t = S_0^T q_t."""
    q, k, v, beta, la, h0 = random_problem(7, T=4, dk=4, dv=3, h0=True)
    beta = np.zeros_like(beta)
    la = np.zeros_like(la)
    o, hT = fn(q, k, v, beta, la, h0)
    _close(hT, h0, TOL, "no-write hT")
    for t in range(4):
        _close(o[0, t, 0], h0[0, 0].T @ q[0, t, 0].astype(np.float64), TOL, "no-write o")


def pin_full_decay(fn):
    """alpha -> 0 (log alpha = -1e4, so exp underflows to exactly 0): each
    token sees an empty state, S_t = beta_t k_t v_t^T, o_t = beta_t (q_t.k_t) v_t,
    whatever S_0 was.  Division by the decay would overflow here."""
    q, k, v, beta, la, h0 = random_problem(9, T=4, dk=4, dv=3, h0=True)
    la = np.full_like(la, -1e4)
    o, hT = fn(q, k, v, beta, la, h0)
    for t in range(4):
        kt, qt, vt, bt = (k[0, t, 0].astype(np.float64), q[0, t, 0].astype(np.float64),
                          v[0, t, 0].astype(np.float64), float(beta[0, t, 0]))
        _close(o[0, t, 0], bt * (qt @ kt) * vt, TOL, "full-decay o")
    want = float(beta[0, 3, 0]) * np.outer(k[0, 3, 0].astype(np.float64), v[0, 3, 0].astype(np.float64))
    _close(hT[0, 0], want, TOL, "full-decay hT")


def pin_one_hot_linear_attention(fn):
    """S_0 = 0 and one-hot keys e_{i_j} on distinct channels, per-channel gate:
    no key is ever predicted (u_t = v_t), so the rule reduces to gated linear
    attention, row i_j of S_T = beta_j prod_{s>j} f_{s,i_j} v_j^T and
    o_t = sum_{j<=t} beta_j q_{t,i_j} prod_{j<s<=t} f_{s,i_j} v_j."""
    dk, T = 6, 4
    chan = [4, 1, 5, 2]
    r = _rng(13)
    k = np.zeros((1, T, 1, dk), np.float32)
    for t, i in enumerate(chan):
        k[0, t, 0, i] = 1.0
    q = _f32(r.standard_normal((1, T, 1, dk)))
    v = _f32(r.standard_normal((1, T, 1, 3)))
    beta = _f32(r.uniform(0.2, 1.0, (1, T, 1)))
    la = _f32(-r.uniform(0.05, 0.9, (1, T, 1, dk)))
    o, hT = fn(q, k, v, beta, la)
    f = np.exp(la[0, :, 0].astype(np.float64))
    for t in range(T):
        want = np.zeros(3)
        for j in range(t + 1):
            i = chan[j]
            want += float(beta[0, j, 0]) * float(q[0, t, 0, i]) * np.prod(f[j + 1:t + 1, i]) * v[0, j, 0]
        _close(o[0, t, 0], want, TOL, "one-hot o")
    S = np.zeros((dk, 3))
    for j, i in enumerate(chan):
        S[i] = float(beta[0, j, 0]) * np.prod(f[j + 1:, i]) * v[0, j, 0]
    _close(hT[0, 0], S, TOL, "one-hot hT")


def pin_tied_channels(fn):
    """A per-channel gate whose channels are all equal is the scalar gate; a
    G-tile gate equals the per-channel gate with the tile's value repeated."""
    dk = 8
    q, k, v, beta, la1, h0 = random_problem(17, T=6, dk=dk, dv=3, G=1, h0=True)
    o1, h1 = fn(q, k, v, beta, la1, h0)
    od, hd = fn(q, k, v, beta, np.repeat(la1, dk, axis=3), h0)
    _close(o1, od, TOL, "scalar vs tied per-channel o")
    _close(h1, hd, TOL, "scalar vs tied per-channel hT")
    _, _, _, _, la4, _ = random_problem(18, T=6, dk=dk, dv=3, G=4)
    o4, h4 = fn(q, k, v, beta, la4, h0)
    oe, he = fn(q, k, v, beta, np.repeat(la4, dk // 4, axis=3), h0)
    _close(o4, oe, TOL, "4-tile vs expanded o")
    _close(h4, he, TOL, "4-tile vs expanded hT")


def pin_grouped_value_heads(fn):
    """H_k = 2 key heads shared by R = 2 value heads each equals H_k = H_v = 4
    with q, k and log alpha replicated to the value heads (value heads of one
    key head are contiguous)."""
    q, k, v, beta, la, h0 = random_problem(21, B=2, T=5, Hk=2, Hv=4, dk=4, dv=3, G=2, h0=True)
    o, hT = fn(q, k, v, beta, la, h0)
    rep = lambda a: np.repeat(a, 2, axis=2)
    o2, h2 = fn(rep(q), rep(k), v, beta, rep(la), h0)
    _close(o, o2, TOL, "GVA o")
    _close(hT, h2, TOL, "GVA hT")


def pin_beta_per_key_head(fn):
    """beta given per key head equals the same beta repeated to its value heads."""
    q, k, v, beta, la, h0 = random_problem(22, T=5, Hk=2, Hv=4, dk=4, dv=3, G=4, h0=True, bkh=True)
    o, hT = fn(q, k, v, beta, la, h0, beta_per_key_head=True)
    o2, h2 = fn(q, k, v, np.repeat(beta, 2, axis=2), la, h0)
    _close(o, o2, TOL, "beta per key head o")
    _close(hT, h2, TOL, "beta per key head hT")


def pin_column_separability(fn):
    """Value columns evolve independently: running d_v in two pieces gives the
    same o and hT columns as running it whole."""
    q, k, v, beta, la, h0 = random_problem(23, T=6, dk=4, dv=6, h0=True)
    o, hT = fn(q, k, v, beta, la, h0)
    oa, ha = fn(q, k, np.ascontiguousarray(v[..., :2]), beta, la, np.ascontiguousarray(h0[..., :2]))
    ob, hb = fn(q, k, np.ascontiguousarray(v[..., 2:]), beta, la, np.ascontiguousarray(h0[..., 2:]))
    _close(o, np.concatenate([oa, ob], -1), TOL, "column split o")
    _close(hT, np.concatenate([ha, hb], -1), TOL, "column split hT")


def pin_resume(fn):
    """Running T tokens equals running the first T1, then the rest from hT
    (the affine chunk map of the paper's section 3.3 holds at any cut)."""
    q, k, v, beta, la, h0 = random_problem(29, B=2, T=9, Hk=1, Hv=2, dk=4, dv=3, G=4, h0=True)
    o, hT = fn(q, k, v, beta, la, h0)
    c = lambda a, s: np.ascontiguousarray(a[:, s])
    oa, ha = fn(c(q, slice(0, 4)), c(k, slice(0, 4)), c(v, slice(0, 4)), c(beta, slice(0, 4)),
                c(la, slice(0, 4)), h0)
    ob, hb = fn(c(q, slice(4, 9)), c(k, slice(4, 9)), c(v, slice(4, 9)), c(beta, slice(4, 9)),
                c(la, slice(4, 9)), ha)
    _close(o, np.concatenate([oa, ob], 1), TOL, "resume o")
    _close(hT, hb, TOL, "resume hT")


ALL_PINS = [
    pin_hand_worked, pin_two_token, pin_one_token_h0, pin_orthonormal_recall,
    pin_no_write, pin_full_decay, pin_one_hot_linear_attention, pin_tied_channels,
    pin_grouped_value_heads, pin_beta_per_key_head, pin_column_separability, pin_resume,
]

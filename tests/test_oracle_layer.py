"""Pins of the layer-level oracle (no GPU): document resets, chunk-boundary
momentum (Systolic Linear Attention, Table 2: Z_c, mu, kappa_c; section 2.3,
"Why chunk-level momentum") and the gated RMSNorm output epilogue (section
2.3, the token-level recurrence box).

Three implementations of resets and momentum are held to each other (the C
token recurrence, its numpy twin, and the fp64 WY chunk form, which shares no
code with either), and all of them to hand-worked values and to invariants
that the definition fixes: mu = 0 is the plain recurrence; a reset equals
starting the document as a separate sequence; a reset at a chunk boundary
with momentum equals a fresh start of both state and momentum buffer;
resuming from (hT, zT) at a chunk boundary equals one run.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import chunk as och
from oracle.epilogue import gated_rmsnorm
from oracle.recurrence import layer_c, layer_np, recurrence_c, recurrence_np


def _layer_c(*a, **kw):
    return layer_c(*a, nthreads=2, **kw)


def _layer_chunk(q, k, v, beta, la, h0=None, beta_per_key_head=False, reset=None, momentum=0.0, chunk=0,
                 z0=None):
    C = chunk if chunk > 0 else max(q.shape[1], 1)
    return och.chunk_forward(q, k, v, beta, la, h0, chunk=C, beta_per_key_head=beta_per_key_head, reset=reset,
                             momentum=momentum, z0=z0, return_z=True)


IMPLS = {"c": _layer_c, "numpy": layer_np, "chunk_form": _layer_chunk}


def _scalar_case(v, reset=None):
    """d_k = d_v = 1, k = q = 1, beta = 1/2, alpha = 1/2 (log alpha rounded to
    fp32, so values carry ~1e-8 relative rounding)."""
    T = len(v)
    one = np.ones((1, T, 1, 1), np.float32)
    beta = np.full((1, T, 1), 0.5, np.float32)
    la = np.full((1, T, 1, 1), np.log(0.5), np.float32)
    vv = np.asarray(v, np.float32).reshape(1, T, 1, 1)
    rs = None if reset is None else np.asarray(reset, np.uint8).reshape(1, T)
    return one, one, vv, beta, la, rs


def pin_momentum_hand_worked(fn):
    """C = 2, mu = 1/4, v = (2, 4, -2, 6, 1, -1), S_0 = Z_0 = 0.  Per token
    S <- S/2, u = v - S, S <- S + u/2, o = S; at each chunk end
    carry = F_c S_{c-1} (F_c = 1/4), Z_c = Z_{c-1}/4 + (S~_c - carry),
    S_c = carry + Z_c.  By hand:
      chunk 1: o = 1, 2.25; carry 0; Z_1 = 2.25; S_1 = 2.25
      chunk 2: o = -0.4375, 2.890625; carry 0.5625; Delta = 2.328125;
               Z_2 = 0.5625 + 2.328125 = 2.890625; S_2 = 3.453125
      chunk 3: o = 1.36328125, -0.1591796875; carry 0.86328125;
               Delta = -1.0224609375; Z_3 = 0.72265625 - 1.0224609375
               = -0.2998046875; S_3 = 0.5634765625
    With a reset at token 4 (inside chunk 2): t4 starts from S = 0, so
    o_4 = 3; kappa_2 = 0, carry 0, Z_2 = 3, S_2 = 3; chunk 3 then gives
    t5: S = 1.5, u = -0.5, o_5 = 1.25; t6: S = 0.625, u = -1.625,
    o_6 = -0.1875; carry 0.75, Delta = -0.9375, Z_3 = 0.75 - 0.9375 =
    -0.1875, S_3 = 0.5625."""
    q, k, v, beta, la, _ = _scalar_case([2, 4, -2, 6, 1, -1])
    o, hT, zT = fn(q, k, v, beta, la, momentum=0.25, chunk=2)
    oracle_pins._close(o.ravel(), [1, 2.25, -0.4375, 2.890625, 1.36328125, -0.1591796875], 1e-6, "momentum o")
    oracle_pins._close(hT.ravel(), [0.5634765625], 1e-6, "momentum hT")
    oracle_pins._close(zT.ravel(), [-0.2998046875], 1e-6, "momentum zT")
    q, k, v, beta, la, rs = _scalar_case([2, 4, -2, 6, 1, -1], reset=[0, 0, 0, 1, 0, 0])
    o, hT, zT = fn(q, k, v, beta, la, reset=rs, momentum=0.25, chunk=2)
    oracle_pins._close(o.ravel(), [1, 2.25, -0.4375, 3, 1.25, -0.1875], 1e-6, "reset+momentum o")
    oracle_pins._close(hT.ravel(), [0.5625], 1e-6, "reset+momentum hT")
    oracle_pins._close(zT.ravel(), [-0.1875], 1e-6, "reset+momentum zT")


def pin_zero_momentum_is_plain(fn):
    q, k, v, beta, la, h0 = oracle_pins.random_problem(5, B=2, T=29, Hk=2, Hv=4, dk=8, dv=5, G=8, h0=True)
    o_ref, h_ref = recurrence_np(q, k, v, beta, la, h0)
    o, hT, _ = fn(q, k, v, beta, la, h0, momentum=0.0, chunk=4)
    oracle_pins._close(o, o_ref, 1e-12, "mu=0 o")
    oracle_pins._close(hT, h_ref, 1e-12, "mu=0 hT")


def _docs(T, starts):
    rs = np.zeros(T, np.uint8)
    rs[list(starts)] = 1
    return rs


def pin_reset_equals_separate_documents(fn):
    """Without momentum, a reset at token t makes tokens t.. a sequence of
    their own starting from the zero state: concatenating the separate runs
    gives the packed run (the first document starts from h0), and hT is the
    last document's final state.  Resets fall inside chunks, on chunk
    boundaries and on the first token."""
    T = 41
    q, k, v, beta, la, h0 = oracle_pins.random_problem(9, B=2, T=T, Hk=1, Hv=2, dk=8, dv=4, G=2, h0=True)
    starts = {0: [7, 16, 17, 33], 1: [0, 5, 30]}
    rs = np.stack([_docs(T, starts[0]), _docs(T, starts[1])])
    o, hT, _ = fn(q, k, v, beta, la, h0, reset=rs, chunk=8)
    for b in range(2):
        bounds = [0] + [s for s in starts[b] if s > 0] + [T]
        for i in range(len(bounds) - 1):
            s, e = bounds[i], bounds[i + 1]
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, s:e])
            init = h0[b:b + 1] if (s == 0 and 0 not in starts[b]) else None
            od, hd = recurrence_c(sl(q), sl(k), sl(v), sl(beta), sl(la), init, nthreads=1)
            oracle_pins._close(o[b, s:e], od[0], 1e-12, f"doc {b}:{s}-{e} o")
        oracle_pins._close(hT[b], hd[0], 1e-12, f"doc {b} last hT")


def pin_reset_at_chunk_boundary_is_fresh_start(fn):
    """With momentum, a reset on the first token of chunk c discards both the
    state and the momentum buffer, so chunks c.. equal a separate run from
    S = 0, Z = 0."""
    C, T = 4, 26
    q, k, v, beta, la, h0 = oracle_pins.random_problem(13, B=1, T=T, Hk=2, Hv=4, dk=8, dv=3, G=8, h0=True)
    z0 = np.random.default_rng(2).standard_normal(h0.shape)
    rs = _docs(T, [12]).reshape(1, T)
    o, hT, zT = fn(q, k, v, beta, la, h0, reset=rs, momentum=0.25, chunk=C, z0=z0)
    sl = lambda a: np.ascontiguousarray(a[:, 12:])
    o2, h2, z2 = layer_np(sl(q), sl(k), sl(v), sl(beta), sl(la), momentum=0.25, chunk=C)
    oracle_pins._close(o[:, 12:], o2, 1e-12, "fresh start o")
    oracle_pins._close(hT, h2, 1e-12, "fresh start hT")
    oracle_pins._close(zT, z2, 1e-12, "fresh start zT")


def pin_resume_at_chunk_boundary(fn):
    """Running the first 3 chunks, then the rest from (hT, zT), equals one run
    with momentum and resets."""
    C, T = 4, 30
    q, k, v, beta, la, h0 = oracle_pins.random_problem(17, B=2, T=T, Hk=1, Hv=2, dk=6, dv=4, G=3, h0=True)
    rs = np.stack([_docs(T, [5, 13]), _docs(T, [22])])
    o, hT, zT = fn(q, k, v, beta, la, h0, reset=rs, momentum=0.25, chunk=C)
    cut = 3 * C
    a = lambda x: np.ascontiguousarray(x[:, :cut])
    b = lambda x: np.ascontiguousarray(x[:, cut:])
    oa, ha, za = fn(a(q), a(k), a(v), a(beta), a(la), h0, reset=a(rs), momentum=0.25, chunk=C)
    ob, hb, zb = fn(b(q), b(k), b(v), b(beta), b(la), ha, reset=b(rs), momentum=0.25, chunk=C, z0=za)
    oracle_pins._close(np.concatenate([oa, ob], 1), o, 1e-12, "resume o")
    oracle_pins._close(hb, hT, 1e-12, "resume hT")
    oracle_pins._close(zb, zT, 1e-12, "resume zT")


LAYER_PINS = [pin_momentum_hand_worked, pin_zero_momentum_is_plain, pin_reset_equals_separate_documents,
              pin_reset_at_chunk_boundary_is_fresh_start, pin_resume_at_chunk_boundary]


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("pin", LAYER_PINS, ids=lambda p: p.__name__)
def test_pin(impl, pin):
    pin(IMPLS[impl])


def mutant_layer(mutation):
    """The numpy layer recurrence with one deliberate mistake."""

    def fn(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False, reset=None, momentum=0.0, chunk=0,
           z0=None):
        B, T, Hk, dk = q.shape
        Hv, dv = v.shape[2], v.shape[3]
        G = log_alpha.shape[3]
        key_of = np.arange(Hv) // (Hv // Hk)
        qe = np.asarray(q, np.float64)[:, :, key_of]
        ke = np.asarray(k, np.float64)[:, :, key_of]
        la = np.repeat(np.asarray(log_alpha, np.float64)[:, :, key_of], dk // G, axis=3)
        be = np.asarray(beta, np.float64)
        if beta_per_key_head:
            be = be[:, :, key_of]
        vv = np.asarray(v, np.float64)
        rs = np.zeros((B, T), bool) if reset is None else np.asarray(reset) != 0
        S = np.zeros((B, Hv, dk, dv)) if h0 is None else np.array(h0, np.float64)
        Z = np.zeros((B, Hv, dk, dv)) if z0 is None else np.array(z0, np.float64)
        o = np.zeros((B, T, Hv, dv))
        use_m = chunk > 0 and momentum != 0.0
        off = 1 if mutation == "chunks_offset_by_one" else 0
        edges = [0] + list(range(off or chunk, T, chunk)) + [T] if use_m else [0, T]
        for c0, c1 in zip(edges[:-1], edges[1:]):
            if c1 <= c0:
                continue
            S_in = S.copy()
            kappa = ~rs[:, c0:c1].any(axis=1)
            for t in range(c0, c1):
                if mutation != "reset_keeps_state":
                    S = np.where(rs[:, t][:, None, None, None], 0.0, S)
                S = np.exp(la[:, t])[..., None] * S
                u = vv[:, t] - np.einsum("bhij,bhi->bhj", S, ke[:, t])
                S = S + be[:, t, :, None, None] * ke[:, t, :, :, None] * u[:, :, None, :]
                o[:, t] = np.einsum("bhij,bhi->bhj", S, qe[:, t])
            if use_m:
                Fc = np.exp(la[:, c0:c1].sum(axis=1))
                kap = kappa[:, None, None, None]
                if mutation == "carry_kept_on_reset":
                    carry = Fc[..., None] * S_in
                else:
                    carry = np.where(kap, Fc[..., None] * S_in, 0.0)
                Zp = Z if mutation == "momentum_kept_on_reset" else np.where(kap, Z, 0.0)
                if mutation == "velocity_is_whole_state":
                    Z = momentum * Zp + S
                else:
                    Z = momentum * Zp + (S - carry)
                if mutation == "momentum_on_state":
                    S = S + momentum * S_in
                elif mutation == "state_is_velocity":
                    S = Z
                else:
                    S = carry + Z
        return o, S, Z

    return fn


MUTATIONS = ["reset_keeps_state", "carry_kept_on_reset", "momentum_kept_on_reset", "velocity_is_whole_state",
             "momentum_on_state", "state_is_velocity", "chunks_offset_by_one"]


def test_unmutated_copy_passes():
    for pin in LAYER_PINS:
        pin(mutant_layer(None))


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_pins_catch_mutation(mutation):
    fn = mutant_layer(mutation)
    caught = []
    for pin in LAYER_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutation}"


def test_three_implementations_agree():
    """C token recurrence, numpy twin and the WY chunk form with segment
    masks: every gate kind, grouped value heads, beta per key head up to 2,
    resets inside and on chunk boundaries, momentum with z0."""
    cases = [
        dict(B=2, T=37, Hk=2, Hv=4, dk=8, dv=5, G=8, h0=True),
        dict(B=1, T=50, Hk=1, Hv=4, dk=16, dv=4, G=4, h0=True, bkh=True),
        dict(B=2, T=19, Hk=2, Hv=2, dk=8, dv=3, G=1),
    ]
    for i, cs in enumerate(cases):
        bkh = cs.get("bkh", False)
        q, k, v, beta, la, h0 = oracle_pins.random_problem(300 + i, **cs)
        B, T = q.shape[:2]
        r = np.random.default_rng(i)
        rs = (r.random((B, T)) < 0.12).astype(np.uint8)
        z0 = r.standard_normal((B, v.shape[2], q.shape[3], v.shape[3]))
        for C in (4, 8):
            res = [fn(q, k, v, beta, la, h0, bkh, reset=rs, momentum=0.25, chunk=C, z0=z0)
                   for fn in (_layer_c, layer_np, _layer_chunk)]
            for other in res[1:]:
                for x, y, n in zip(res[0], other, ("o", "hT", "zT")):
                    oracle_pins._close(x, y, 1e-12 * max(1.0, np.max(np.abs(x))), f"case {i} C={C} {n}")


def test_layer_c_plain_matches_recurrence_bitwise():
    q, k, v, beta, la, h0 = oracle_pins.random_problem(21, B=1, T=33, Hk=1, Hv=2, dk=8, dv=4, G=8, h0=True)
    o1, h1 = recurrence_c(q, k, v, beta, la, h0, nthreads=1)
    o2, h2, _ = layer_c(q, k, v, beta, la, h0, nthreads=1)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


# ------------------------------------------------------------------ epilogue
def test_gated_rmsnorm_hand_worked():
    """o = (3, 4): mean square 12.5; z = (0, ln 3): gates (1/2, 3/4);
    w = (2, 1), eps = 0: y = (1/2 * 3 / sqrt(12.5) * 2, 3/4 * 4 / sqrt(12.5))."""
    r = np.sqrt(12.5)
    y = gated_rmsnorm([3.0, 4.0], [0.0, np.log(3.0)], weight=[2.0, 1.0], eps=0.0)
    oracle_pins._close(y, [3.0 / r, 3.0 / r], 1e-15, "gated rmsnorm")
    y = gated_rmsnorm([3.0, 4.0], [0.0, 0.0], eps=12.5)
    oracle_pins._close(y, [0.5 * 3.0 / 5.0, 0.5 * 4.0 / 5.0], 1e-15, "gated rmsnorm eps")


def test_gated_rmsnorm_invariants():
    """Per head: scaling o by c > 0 leaves y unchanged at eps = 0; with the
    gate fully open (z -> +inf) and w = 1 each head's output has unit rms."""
    r = np.random.default_rng(3)
    o = r.standard_normal((2, 5, 3, 16))
    z = r.standard_normal((2, 5, 3, 16))
    y = gated_rmsnorm(o, z, eps=0.0)
    oracle_pins._close(gated_rmsnorm(7.5 * o, z, eps=0.0), y, 1e-14, "scale invariance")
    y1 = gated_rmsnorm(o, np.full_like(z, 50.0), eps=0.0)
    oracle_pins._close(np.sqrt(np.mean(y1 ** 2, axis=-1)), np.ones((2, 5, 3)), 1e-12, "unit rms")
    # heads are normalised separately: changing one head leaves the others
    o2 = o.copy()
    o2[..., 1, :] *= 100.0
    y2 = gated_rmsnorm(o2, z, eps=1e-3)
    yb = gated_rmsnorm(o, z, eps=1e-3)
    oracle_pins._close(y2[..., 0, :], yb[..., 0, :], 0.0, "head independence")

"""Pins of the gradient oracle (no GPU).

vjp_autograd (reverse-mode differentiation of the plain token recurrence)
is held to central finite differences of the pinned numpy recurrence and to
a hand-worked two-token gradient; vjp_chunk (the chunkwise backward of
Systolic Linear Attention section 2.5, written out independently) is held
to vjp_autograd at several chunk sizes, and planted mistakes in it are each
caught."""
import numpy as np
import pytest

import oracle_pins
from oracle import backward as ob
from oracle.recurrence import recurrence_np


def _loss(q, k, v, beta, la, h0, do, dhT, bkh):
    o, hT = recurrence_np(q, k, v, beta, la, h0, bkh)
    return float(np.sum(o * do) + (np.sum(hT * dhT) if dhT is not None else 0.0))


@pytest.mark.parametrize("bkh", [False, True])
def test_autograd_matches_finite_differences(bkh):
    q, k, v, beta, la, h0 = oracle_pins.random_problem(41, B=1, T=6, Hk=1, Hv=2, dk=3, dv=2, G=3, h0=True, bkh=bkh)
    f64 = lambda a: np.asarray(a, np.float64)
    q, k, v, beta, la = (f64(a) for a in (q, k, v, beta, la))
    r = np.random.default_rng(2)
    do = r.standard_normal(v.shape)
    dhT = r.standard_normal(h0.shape)
    g = ob.vjp_autograd(q, k, v, beta, la, h0, do, dhT, bkh)
    args = {"dq": q, "dk": k, "dv": v, "dbeta": beta, "dlog_alpha": la, "dh0": h0}
    eps = 1e-6
    for name, x in args.items():
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            fp = _loss(q, k, v, beta, la, h0, do, dhT, bkh)
            x[idx] = keep - eps
            fm = _loss(q, k, v, beta, la, h0, do, dhT, bkh)
            x[idx] = keep
            num[idx] = (fp - fm) / (2 * eps)
        scale = max(1.0, np.max(np.abs(num)))
        assert np.max(np.abs(g[name] - num)) <= 1e-6 * scale, name


def test_two_token_gradient_by_hand():
    """d_k = d_v = 1, k = q = 1, S_0 = 0, beta = (1/2, 1/4), alpha_2 = 1/2,
    v = (2, 4), do = (1, 1).  S_1 = b1 k1 v1 = 1, o_1 = q1 S_1;
    S_2 = a2 S_1 + b2 k2 (v2 - k2 a2 S_1), o_2 = q2 S_2 = 1.375:
      dv1 = b1 + a2 b1 (1 - b2) = 0.6875,  dv2 = b2 = 0.25,
      db1 = v1 + a2 v1 (1 - b2) = 2.75,    db2 = v2 - a2 b1 v1 = 3.5,
      dlog a2 = a2 b1 v1 (1 - b2) = 0.375, dlog a1 = 0 (it decays S_0 = 0),
      dq = (S_1, S_2) = (1, 1.375),
      dk1 = b1 v1 + a2 (1 - b2) b1 v1 = 1.375,  dk2 = b2 (v2 - 2 a2 S_1) = 0.75."""
    one = np.ones((1, 2, 1, 1))
    beta = np.array([0.5, 0.25]).reshape(1, 2, 1)
    la = np.array([0.0, np.log(0.5)]).reshape(1, 2, 1, 1)
    v = np.array([2.0, 4.0]).reshape(1, 2, 1, 1)
    do = np.ones((1, 2, 1, 1))
    g = ob.vjp_autograd(one, one, v, beta, la, None, do)
    oracle_pins._close(g["dv"].ravel(), [0.6875, 0.25], 1e-12, "dv")
    oracle_pins._close(g["dbeta"].ravel(), [2.75, 3.5], 1e-12, "dbeta")
    oracle_pins._close(g["dlog_alpha"].ravel(), [0.0, 0.375], 1e-12, "dlog_alpha")
    oracle_pins._close(g["dq"].ravel(), [1.0, 1.375], 1e-12, "dq")
    oracle_pins._close(g["dk"].ravel(), [1.375, 0.75], 1e-12, "dk")


CASES = [dict(B=1, T=11, Hk=1, Hv=1, dk=4, dv=3, G=4, h0=True),
         dict(B=2, T=13, Hk=2, Hv=4, dk=6, dv=3, G=2, h0=True, bkh=True),
         dict(B=1, T=9, Hk=1, Hv=2, dk=4, dv=2, G=1)]


@pytest.mark.parametrize("chunk", [1, 3, 4, 16])
def test_chunk_backward_matches_autograd(chunk):
    for i, cs in enumerate(CASES):
        cs = dict(cs)
        bkh = cs.pop("bkh", False)
        q, k, v, beta, la, h0 = oracle_pins.random_problem(60 + i, bkh=bkh, **cs)
        r = np.random.default_rng(i)
        do = r.standard_normal(v.shape)
        dhT = r.standard_normal((q.shape[0], v.shape[2], q.shape[3], v.shape[3]))
        a = ob.vjp_autograd(q, k, v, beta, la, h0, do, dhT, bkh)
        c = ob.vjp_chunk(q, k, v, beta, la, h0, do, dhT, chunk=chunk, beta_per_key_head=bkh)
        for n in a:
            if a[n] is None:
                continue
            assert np.max(np.abs(a[n] - c[n])) <= 1e-12 * max(1.0, np.max(np.abs(a[n]))), (i, n)


def _mutated_chunk_vjp(monkeypatch, mutation):
    orig = ob._chunk_quantities

    def pieces(q, k, beta, la):
        c = orig(q, k, beta, la)
        if mutation == "L_without_diagonal":
            c["L"] = np.tril(c["L"], -1)
        elif mutation == "gamma_first_token":
            c["gamma"] = np.exp(c["Lam"][0])
        elif mutation == "A_transposed":
            c["A"] = c["A"].T
        elif mutation == "Khat_from_start":
            c["Khat"] = k * np.exp(c["Lam"])
        return c

    monkeypatch.setattr(ob, "_chunk_quantities", pieces)


@pytest.mark.parametrize("mutation", ["L_without_diagonal", "gamma_first_token", "A_transposed", "Khat_from_start"])
def test_planted_mistakes_in_the_chunk_backward_are_caught(monkeypatch, mutation):
    q, k, v, beta, la, h0 = oracle_pins.random_problem(77, B=1, T=12, dk=4, dv=3, G=4, h0=True)
    r = np.random.default_rng(5)
    do = r.standard_normal(v.shape)
    a = ob.vjp_autograd(q, k, v, beta, la, h0, do)
    _mutated_chunk_vjp(monkeypatch, mutation)
    c = ob.vjp_chunk(q, k, v, beta, la, h0, do, chunk=4)
    worst = max(np.max(np.abs(a[n] - c[n])) for n in a if a[n] is not None)
    assert worst > 1e-6

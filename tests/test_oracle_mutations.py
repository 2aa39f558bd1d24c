"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pins catch every one.  This is what makes the pins worth trusting: a
dropped term, a wrong sign or index, a transposed operand or a misplaced
step must fail at least one of them."""
import numpy as np
import pytest

import oracle_pins
from oracle import chunk as ch
from oracle.recurrence import recurrence_np


def mutant_recurrence(mutation):
    """numpy token recurrence with one deliberate mistake."""

    def fn(q, k, v, beta, log_alpha, h0=None, beta_per_key_head=False):
        B, T, Hk, dk = q.shape
        Hv, dv = v.shape[2], v.shape[3]
        G = log_alpha.shape[3]
        R = Hv // Hk
        key_of = np.arange(Hv) % Hk if mutation == "key_head_modulo" else np.arange(Hv) // R
        qe = np.asarray(q, np.float64)[:, :, key_of]
        ke = np.asarray(k, np.float64)[:, :, key_of]
        la = np.asarray(log_alpha, np.float64)[:, :, key_of]
        if mutation == "group_interleaved":
            la = la[..., np.arange(dk) % G]
        else:
            la = np.repeat(la, dk // G, axis=3)
        if mutation == "decay_sign":
            la = -la
        be = np.asarray(beta, np.float64)
        if beta_per_key_head:
            be = be[:, :, key_of]
        vv = np.asarray(v, np.float64)
        S = np.zeros((B, Hv, dk, dv)) if h0 is None else np.array(h0, np.float64)
        o = np.zeros((B, T, Hv, dv))
        for t in range(T):
            f = np.exp(la[:, t])[..., None]
            bt = be[:, max(t - 1, 0)] if mutation == "beta_previous_token" else be[:, t]
            Sd = f * S
            if mutation == "erase_undecayed":
                u = vv[:, t] - np.einsum("bhij,bhi->bhj", S, ke[:, t])
            elif mutation == "error_sign":
                u = vv[:, t] + np.einsum("bhij,bhi->bhj", Sd, ke[:, t])
            else:
                u = vv[:, t] - np.einsum("bhij,bhi->bhj", Sd, ke[:, t])
            if mutation == "readout_before_write":
                o[:, t] = np.einsum("bhij,bhi->bhj", Sd, qe[:, t])
            scale = np.ones_like(bt) if mutation == "drop_beta" else bt
            write = scale[..., None, None] * ke[:, t, :, :, None] * u[:, :, None, :]
            if mutation == "decay_after_write":
                S = f * (S + write)
            elif mutation == "no_decay_in_state":
                S = S + write
            else:
                S = Sd + write
            if mutation == "transposed_readout":
                o[:, t] = np.einsum("bhij,bhj->bhi", S, qe[:, t])
            elif mutation == "readout_with_key":
                o[:, t] = np.einsum("bhij,bhi->bhj", S, ke[:, t])
            elif mutation != "readout_before_write":
                o[:, t] = np.einsum("bhij,bhi->bhj", S, qe[:, t])
        return o, S

    return fn


MUTATIONS = [
    "key_head_modulo", "group_interleaved", "decay_sign", "beta_previous_token",
    "erase_undecayed", "error_sign", "readout_before_write", "drop_beta",
    "decay_after_write", "no_decay_in_state", "transposed_readout", "readout_with_key",
]


def _fails_some_pin(fn):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError, IndexError) as e:  # shape errors count as caught
            failed.append((pin.__name__, str(e)[:60]))
    return failed


def test_unmutated_copy_passes():
    assert _fails_some_pin(mutant_recurrence("none")) == []


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutation_is_caught(mutation):
    assert _fails_some_pin(mutant_recurrence(mutation)), f"no pin catches {mutation}"


# ------------------------------------------------------------ chunk form
def _chunk_with(mutation):
    orig = ch.chunk_pieces

    def pieces(q, k, beta, la, reset=None):
        pc = orig(q, k, beta, la, reset)
        n = q.shape[0]
        if mutation == "L_without_diagonal":
            pc["L"] = np.tril(pc["L"], -1)
        elif mutation == "M_row_beta":
            pc["M"] = beta[:, None] * pc["G"]
        elif mutation == "Khat_from_start":
            pc["Khat"] = k * np.exp(pc["Lambda"])
        elif mutation == "gamma_first_token":
            pc["gamma"] = np.exp(pc["Lambda"][0])
        elif mutation == "M_with_diagonal":
            pc["M"] = pc["M"] + np.diag(beta * np.sum(k * k, axis=1))
        del n
        return pc

    return pieces


@pytest.mark.parametrize("mutation", ["L_without_diagonal", "M_row_beta", "Khat_from_start",
                                      "gamma_first_token", "M_with_diagonal"])
def test_chunk_mutation_is_caught(mutation, monkeypatch):
    """The chunk form is pinned by agreement with the recurrence; each planted
    error in a Table 2 quantity breaks that agreement."""
    monkeypatch.setattr(ch, "chunk_pieces", _chunk_with(mutation))
    q, k, v, beta, la, h0 = oracle_pins.random_problem(77, T=24, dk=6, dv=3, G=6, h0=True)
    o_r, h_r = recurrence_np(q, k, v, beta, la, h0)
    o_c, h_c = ch.chunk_forward(q, k, v, beta, la, h0, chunk=8)
    assert max(np.max(np.abs(o_c - o_r)), np.max(np.abs(h_c - h_r))) > 1e-6

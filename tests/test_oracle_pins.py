"""The token-recurrence oracle against hand-worked examples, closed forms and
invariants (no GPU)."""
import numpy as np
import pytest

import oracle_pins
from oracle.recurrence import recurrence_c, recurrence_np


def _c(q, k, v, beta, la, h0=None, beta_per_key_head=False):
    return recurrence_c(q, k, v, beta, la, h0, beta_per_key_head, nthreads=2)


IMPLS = {"c": _c, "numpy": recurrence_np}


@pytest.mark.parametrize("impl", sorted(IMPLS))
@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(impl, pin):
    pin(IMPLS[impl])


def test_c_matches_numpy_twin():
    """Two implementations with no shared code agree to 1e-12 on random
    problems covering every gate kind, GVA, beta per key head and h0."""
    cases = [
        dict(B=2, T=37, Hk=2, Hv=2, dk=8, dv=5, G=1),
        dict(B=1, T=50, Hk=2, Hv=4, dk=16, dv=8, G=16, h0=True),
        dict(B=2, T=23, Hk=1, Hv=4, dk=16, dv=4, G=4, h0=True),
        dict(B=1, T=19, Hk=2, Hv=4, dk=8, dv=3, G=2, bkh=True),
    ]
    for i, cs in enumerate(cases):
        bkh = cs.get("bkh", False)
        q, k, v, beta, la, h0 = oracle_pins.random_problem(100 + i, **cs)
        oc, hc = recurrence_c(q, k, v, beta, la, h0, bkh, nthreads=3)
        on, hn = recurrence_np(q, k, v, beta, la, h0, bkh)
        assert np.max(np.abs(oc - on)) <= 1e-12 * max(1.0, np.max(np.abs(on)))
        assert np.max(np.abs(hc - hn)) <= 1e-12 * max(1.0, np.max(np.abs(hn)))


def test_c_units_subset_and_threads():
    """Evaluating a subset of (b, h_v) units, with any thread count, gives the
    same rows as the full run and leaves the other rows zero."""
    q, k, v, beta, la, h0 = oracle_pins.random_problem(7, B=2, T=20, Hk=2, Hv=4, dk=8, dv=4, G=8, h0=True)
    o, hT = recurrence_c(q, k, v, beta, la, h0, nthreads=1)
    units = [5, 0, 3]
    os_, hs = recurrence_c(q, k, v, beta, la, h0, units=units, nthreads=4)
    for u in range(8):
        b, h = divmod(u, 4)
        if u in units:
            assert np.array_equal(os_[b, :, h], o[b, :, h])
            assert np.array_equal(hs[b, h], hT[b, h])
        else:
            assert not os_[b, :, h].any() and not hs[b, h].any()


def test_c_rejects_malformed():
    q, k, v, beta, la, _ = oracle_pins.random_problem(1, Hk=2, Hv=3)
    with pytest.raises(ValueError):
        recurrence_c(q, k, v, beta, la)

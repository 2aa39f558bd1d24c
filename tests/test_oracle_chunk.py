"""The fp64 chunkwise form and the in-chunk inverses of the oracle (no GPU).

Pins: the chunk form with the exact inverse reproduces the (separately
pinned) token recurrence; block doubling equals the explicit inverse; the
Neumann series obeys the nilpotency, tail and bound statements of the
multiplication-only inversion paper (Lemma 3.1, Fig. 5); the block-Neumann
identity of Systolic Linear Attention section 2.4.3 is exact for 8 block rows.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import chunk as ch
from oracle.recurrence import recurrence_np


def _strict_lower(seed, n, scale=0.3):
    r = np.random.default_rng(seed)
    return np.tril(r.standard_normal((n, n)) * scale, -1)


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16])
def test_chunk_exact_equals_recurrence(C):
    """Chunk sizes 1..16 (chunk-size invariance), T not a multiple of C,
    grouped value heads, nonzero h0 and every gate kind."""
    for G in (1, 4, 8):
        q, k, v, beta, la, h0 = oracle_pins.random_problem(40 + G, B=2, T=37, Hk=2, Hv=4, dk=8, dv=5, G=G, h0=True)
        o_r, h_r = recurrence_np(q, k, v, beta, la, h0)
        o_c, h_c = ch.chunk_forward(q, k, v, beta, la, h0, chunk=C, solve="exact")
        assert np.max(np.abs(o_c - o_r)) < 1e-12
        assert np.max(np.abs(h_c - h_r)) < 1e-12


def test_chunk_exact_beta_per_key_head_and_strong_decay():
    q, k, v, beta, la, h0 = oracle_pins.random_problem(3, B=1, T=40, Hk=2, Hv=4, dk=8, dv=3, G=8, h0=True, bkh=True)
    la = (la * 30).astype(np.float32)          # |Lambda| over a chunk well past 88.7
    o_r, h_r = recurrence_np(q, k, v, beta, la, h0, beta_per_key_head=True)
    o_c, h_c = ch.chunk_forward(q, k, v, beta, la, h0, chunk=16, beta_per_key_head=True)
    assert np.all(np.isfinite(o_c))
    assert np.max(np.abs(o_c - o_r)) < 1e-12
    assert np.max(np.abs(h_c - h_r)) < 1e-12


def test_block_doubling_is_exact():
    for n in (2, 4, 16, 64, 128):
        M = _strict_lower(n, n)
        X = ch.block_doubling_inverse(M)
        scale = np.max(np.abs(X))
        assert np.max(np.abs(X - ch.exact_inverse(M))) < 1e-13 * scale
        assert np.max(np.abs((np.eye(n) + M) @ X - np.eye(n))) < 1e-13 * scale


def test_lemma_band_structure():
    """Multiplication-only inversion paper, Lemma 3.1: powers of a strictly
    lower-triangular matrix are banded, (M^n)_{ij} = 0 whenever i - j < n."""
    M = _strict_lower(1, 12)
    P = np.eye(12)
    i, j = np.indices((12, 12))
    for n in range(1, 13):
        P = P @ M
        assert np.all(P[(i - j) < n] == 0.0)
    assert np.all(P == 0.0)          # nilpotent: M^C = 0


@pytest.mark.parametrize("C,m,r", [(64, 4, 4), (64, 7, 3), (128, 4, 5), (16, 15, 0), (32, 3, 3)])
def test_neumann_exact_when_long_enough(C, m, r):
    """(m + 1) 2^r >= C terms make the truncated series with r residual
    corrections exact (the corrections double the number of kept powers and
    M^C = 0 by the band structure)."""
    assert (m + 1) * 2 ** r >= C
    M = _strict_lower(C, C, 0.2)
    X = ch.neumann_inverse(M, m, r)
    assert np.max(np.abs(X - ch.exact_inverse(M))) < 1e-12


def test_neumann_truncation_tail_and_bound():
    """With no correction, the error is exactly the tail sum_{s>m} (-M)^s, and
    ||E_m||_2 <= ||M||_2^{m+1} / (1 - ||M||_2) when ||M||_2 < 1 (the geometric
    bound plotted in the inversion paper's Fig. 5)."""
    C = 64
    M = _strict_lower(5, C, 0.02)
    norm = np.linalg.norm(M, 2)
    assert norm < 1
    A = ch.exact_inverse(M)
    for m in range(0, 8):
        X = ch.neumann_inverse(M, m, 0)
        tail = np.zeros((C, C))
        P = np.linalg.matrix_power(-M, m + 1)
        for _ in range(m + 1, C):
            tail += P
            P = P @ (-M)
        assert np.max(np.abs((A - X) - tail)) < 1e-13
        assert np.linalg.norm(A - X, 2) <= norm ** (m + 1) / (1 - norm) * (1 + 1e-12)


def test_neumann_residual_doubles_terms():
    """One residual correction of the order-m series equals the order
    2(m+1)-1 series exactly (fp64)."""
    M = _strict_lower(8, 32, 0.3)
    for m in (1, 2, 4):
        assert np.max(np.abs(ch.neumann_inverse(M, m, 1) - ch.neumann_inverse(M, 2 * m + 1, 0))) < 1e-12


def test_block_neumann_identity():
    """Systolic Linear Attention section 2.4.3: with 8 block rows,
    sum_{s=0}^{7} (-N)^s D^{-1} = (I + N^4)(I + N^2)(I - N) D^{-1} is the exact
    inverse; one term less is not."""
    C, blk = 128, 16
    M = _strict_lower(9, C, 0.3)
    X = ch.block_neumann_inverse(M, blk, C // blk)
    assert np.max(np.abs(X - ch.exact_inverse(M))) < 1e-10
    IM = np.eye(C) + M
    D = np.zeros_like(IM)
    for s in range(0, C, blk):
        D[s:s + blk, s:s + blk] = IM[s:s + blk, s:s + blk]
    Dinv = np.linalg.inv(D)
    N = Dinv @ (IM - D)
    I = np.eye(C)
    prod = (I + np.linalg.matrix_power(N, 4)) @ (I + N @ N) @ (I - N) @ Dinv
    assert np.max(np.abs(prod - X)) < 1e-10
    assert np.max(np.abs(ch.block_neumann_inverse(M, blk, C // blk - 1) - X)) > 1e-6


def _blocks_inv(IM, blk):
    return [np.linalg.inv(IM[s:s + blk, s:s + blk]) for s in range(0, IM.shape[0], blk)]


def test_one_step_block_neumann_closed_forms():
    """Systolic Linear Attention section 2.4.3, 1-Step Neumann A_N1 = (I - N) D^{-1}:
    written block by block it is D_I^{-1} on the diagonal and
    -D_I^{-1} M_IJ D_J^{-1} below it (every pair of block rows, not only
    neighbours); with two block rows N^2 = 0 and it is the exact inverse; and
    the truncation property exact - A_N1 = sum_{s>=2} (-N)^s D^{-1} holds."""
    blk = 16
    for C in (32, 64, 128):
        M = _strict_lower(20 + C, C, 0.4)
        IM = np.eye(C) + M
        A1 = ch.invert(M, "block_neumann", order=1)
        assert np.max(np.abs(A1 - ch.block_neumann_inverse(M, blk, 2))) == 0.0
        Di = _blocks_inv(IM, blk)
        want = np.zeros((C, C))
        for I in range(C // blk):
            rI = slice(I * blk, I * blk + blk)
            want[rI, rI] = Di[I]
            for J in range(I):
                rJ = slice(J * blk, J * blk + blk)
                want[rI, rJ] = -Di[I] @ M[rI, rJ] @ Di[J]
        assert np.max(np.abs(A1 - want)) < 1e-12 * max(1.0, np.max(np.abs(want)))
        if C == 2 * blk:
            assert np.max(np.abs(A1 - ch.exact_inverse(M))) < 1e-12
        else:
            assert np.max(np.abs(A1 - ch.exact_inverse(M))) > 1e-6
        D = np.zeros_like(IM)
        for I, d in enumerate(Di):
            D[I * blk:(I + 1) * blk, I * blk:(I + 1) * blk] = np.linalg.inv(d)
        N = np.linalg.inv(D) @ (IM - D)
        tail = sum((np.linalg.matrix_power(-N, s) for s in range(2, C // blk)), np.zeros((C, C))) @ np.linalg.inv(D)
        ex = ch.exact_inverse(M)
        assert np.max(np.abs(ex - A1 - tail)) < 1e-12 * np.max(np.abs(ex))
        # a transposed order, (I - O D^{-1}) D^{-1}, is a different matrix
        wrong = (np.eye(C) - (IM - D) @ np.linalg.inv(D)) @ np.linalg.inv(D)
        assert C == 2 * blk or np.max(np.abs(wrong - A1)) > 1e-6


def test_block_neumann_order_in_chunk_form():
    """The chunk form with the block-Neumann solve of order m >= C/16 - 1 is
    the exact chunk form (the series ends); order 1 departs from it."""
    q, k, v, beta, la, h0 = oracle_pins.random_problem(5, B=1, T=70, Hk=1, Hv=2, dk=8, dv=4, G=8, h0=True)
    o_e, h_e = ch.chunk_forward(q, k, v, beta, la, h0, chunk=64, solve="exact")
    o_b, h_b = ch.chunk_forward(q, k, v, beta, la, h0, chunk=64, solve="block_neumann", order=3)
    assert np.max(np.abs(o_b - o_e)) < 1e-10 and np.max(np.abs(h_b - h_e)) < 1e-10
    o_1, _ = ch.chunk_forward(q, k, v, beta, la, h0, chunk=64, solve="block_neumann", order=1)
    assert np.max(np.abs(o_1 - o_e)) > 1e-8


def test_chunk_pieces_brute_force():
    """Each Table 2 quantity of one chunk against a brute-force evaluation of its
    definition with explicit products of the per-token gates."""
    q, k, v, beta, la, _ = oracle_pins.random_problem(4, T=7, dk=5, dv=2, G=5)
    q0, k0, b0 = q[0, :, 0].astype(float), k[0, :, 0].astype(float), beta[0, :, 0].astype(float)
    f = np.exp(la[0, :, 0].astype(float))              # f_{s,i}
    pc = ch.chunk_pieces(q0, k0, b0, la[0, :, 0].astype(float))
    n = 7
    P = lambda t, j: np.prod(f[j + 1:t + 1], axis=0)   # diag of P_{t<-j}, 0-based tokens
    for t in range(n):
        into = np.prod(f[:t + 1], axis=0)              # P_{t<-0}: all gates up to t
        carry = np.prod(f[t + 1:], axis=0)             # P_{C<-t}
        assert np.allclose(pc["Qbar"][t], into * q0[t], rtol=1e-13, atol=0)
        assert np.allclose(pc["Kbar"][t], into * k0[t], rtol=1e-13, atol=0)
        assert np.allclose(pc["Khat"][t], carry * k0[t], rtol=1e-13, atol=0)
        for j in range(n):
            m = b0[j] * np.sum(k0[t] * P(t, j) * k0[j]) if t > j else 0.0
            l_ = np.sum(q0[t] * P(t, j) * k0[j]) if t >= j else 0.0
            assert abs(pc["M"][t, j] - m) < 1e-14
            assert abs(pc["L"][t, j] - l_) < 1e-14
    assert np.allclose(pc["gamma"], np.prod(f, axis=0), rtol=1e-13, atol=0)


def test_wy_system_holds():
    """The prediction errors of the recurrence solve the chunk's triangular
    system, (I + M) u = V - Kbar S_0 (the packed WY equivalence proof of
    section 2.4.2), with u_t = v_t - (F_t S_{t-1})^T k_t from a token loop."""
    q, k, v, beta, la, h0 = oracle_pins.random_problem(6, T=9, dk=6, dv=3, G=6, h0=True)
    S = h0[0, 0].copy()
    us = []
    for t in range(9):
        S = np.exp(la[0, t, 0].astype(float))[:, None] * S
        u = v[0, t, 0] - S.T @ k[0, t, 0]
        S = S + float(beta[0, t, 0]) * np.outer(k[0, t, 0], u)
        us.append(u)
    U = np.array(us)
    pc = ch.chunk_pieces(q[0, :, 0].astype(float), k[0, :, 0].astype(float),
                         beta[0, :, 0].astype(float), la[0, :, 0].astype(float))
    lhs = (np.eye(9) + pc["M"]) @ U
    rhs = v[0, :, 0] - pc["Kbar"] @ h0[0, 0]
    assert np.max(np.abs(lhs - rhs)) < 1e-12


def test_stage_matrices_padding():
    q, k, v, beta, la, _ = oracle_pins.random_problem(8, B=1, T=20, Hk=1, Hv=2, dk=4, dv=2, G=4)
    A, L = ch.chunk_stage_matrices(q, k, beta, la, chunk=8)
    assert A.shape == (1, 2, 3, 8, 8) and L.shape == (1, 1, 3, 8, 8)
    # last chunk has 4 real tokens: identity / zero padding beyond them
    assert np.array_equal(A[0, 1, 2, 4:, 4:], np.eye(4))
    assert not A[0, 1, 2, 4:, :4].any() and not L[0, 0, 2, 4:].any() and not L[0, 0, 2, :, 4:].any()
    pc = ch.chunk_pieces(q[0, 8:16, 0].astype(float), k[0, 8:16, 0].astype(float),
                         beta[0, 8:16, 1].astype(float), la[0, 8:16, 0].astype(float))
    assert np.max(np.abs(A[0, 1, 1] - ch.exact_inverse(pc["M"]))) < 1e-13
    assert np.max(np.abs(L[0, 0, 1] - pc["L"])) < 1e-15


def test_fp32_exp_overflow_threshold():
    """Systolic Linear Attention section 2.4.2: exp(+-Lambda) leaves the fp32
    range once |Lambda| > 88.7, which is why the decay must only ever be
    exponentiated as a non-positive difference."""
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float32(88.8)))
        assert np.isfinite(np.exp(np.float32(88.6)))

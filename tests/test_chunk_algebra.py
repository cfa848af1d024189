"""The chunkwise (WY) form that the GPU kernels evaluate, written in numpy
fp64, against the oracle's token recurrence.  This checks the derivation the
kernels rely on, independently of any kernel:

* decay absorption ("Gated DeltaNet-2 Review" §3-2 item 5; Gated DeltaNet-2
  Q&A page Q4): within a chunk with in-chunk cumulative log-decay g_r and
  chunk total g_C, the operands E = b*k*exp(g - g_C), Qs = q*exp(g - g_C),
  Kh = k*exp(g_C - g) turn the chunk into a decay-free asymmetric delta
  recurrence on the pre-scaled state S' = diag(exp(g_C)) S;
* WY / UT form: (I + A) U = X - E S' with A = strict_lower(E Kh^T), so
  U = T (X - E S'), T = (I + A)^-1; outputs O = Qs S' + lower(Qs Kh^T) U and
  the carried state S_next = S' + Kh^T U.
* T by blocked doubling: invert the 16x16 diagonal blocks, then combine
  adjacent blocks with T_21 = -T_22 A_21 T_11 at sizes 16, 32, ...
"""
import numpy as np
import pytest

import oracle


def _inv_unit_lower_blocked(A):
    C = A.shape[0]
    T = np.zeros_like(A)
    nb = 16 if C >= 16 else C
    for s in range(0, C, nb):                      # diagonal blocks, forward substitution
        for j in range(nb):
            x = np.zeros(nb)
            for r in range(nb):
                x[r] = (1.0 if r == j else 0.0) - A[s + r, s:s + r] @ x[:r]
            T[s:s + nb, s + j] = x
    size = nb
    while size < C:
        for p in range(0, C, 2 * size):
            a, bb = slice(p, p + size), slice(p + size, p + 2 * size)
            T[bb, a] = -T[bb, bb] @ (A[bb, a] @ T[a, a])
        size *= 2
    return T


def chunk_forward(q, k, v, la, b, w, S0, C):
    BH, Tn, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((BH, Tn, dv))
    Sf = np.zeros((BH, dk, dv))
    for h in range(BH):
        S = S0[h].copy()
        for c0 in range(0, Tn, C):
            sl = slice(c0, c0 + C)
            g = np.cumsum(la[h, sl], axis=0)
            gC = g[-1]
            E = b[h, sl] * k[h, sl] * np.exp(g - gC)
            Qs = q[h, sl] * np.exp(g - gC)
            Kh = k[h, sl] * np.exp(gC - g)
            X = w[h, sl] * v[h, sl]
            A = np.tril(E @ Kh.T, -1)
            P = np.tril(Qs @ Kh.T, 0)
            T = _inv_unit_lower_blocked(A)
            Sp = np.exp(gC)[:, None] * S
            U = T @ (X - E @ Sp)
            o[h, sl] = Qs @ Sp + P @ U
            S = Sp + Kh.T @ U
        Sf[h] = S
    return o, Sf


def _case(T, dk, dv, seed, decay=0.05):
    r = np.random.default_rng(seed)
    q = r.standard_normal((2, T, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((2, T, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((2, T, dv))
    la = -np.logaddexp(0, r.standard_normal((2, T, dk))) * decay
    b = 1 / (1 + np.exp(-r.standard_normal((2, T, dk))))
    w = 1 / (1 + np.exp(-r.standard_normal((2, T, dv))))
    S0 = r.standard_normal((2, dk, dv)) * 0.02
    return q, k, v, la, b, w, S0


def test_blocked_inverse():
    r = np.random.default_rng(0)
    for C in (16, 32, 64):
        A = np.tril(r.standard_normal((C, C)) * 0.1, -1)
        np.testing.assert_allclose(_inv_unit_lower_blocked(A), np.linalg.inv(np.eye(C) + A),
                                   rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C,T,dk,dv", [(16, 64, 16, 16), (32, 96, 32, 16), (64, 192, 64, 32),
                                       (64, 128, 128, 128)])
def test_chunk_form_matches_token_recurrence(C, T, dk, dv):
    args = _case(T, dk, dv, seed=C + T)
    o, sf = oracle.fwd(*args)
    o2, s2 = chunk_forward(*args, C=C)
    np.testing.assert_allclose(o2, o, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(s2, sf, rtol=1e-9, atol=1e-11)


def test_chunk_form_strong_decay_fp64():
    """With strong decay the pre-scaled operands span a wide range; fp64 still
    reproduces the recurrence (the kernels bound the range per precision)."""
    args = _case(64, 16, 8, seed=5, decay=0.15)
    o, sf = oracle.fwd(*args)
    o2, s2 = chunk_forward(*args, C=64)
    np.testing.assert_allclose(o2, o, rtol=1e-8, atol=1e-10)

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


# ---------------------------------------------------------------------------
# Chunkwise backward: the blocking the backward kernels use, against the
# oracle's token-level reverse mode.
#
# Per chunk, with S the chunk-start state, D the gradient of the chunk-end
# state and the forward quantities above (S' = diag(e^{g_C}) S, R = X - E S',
# U = T R, O = Qs S' + P U, S_next = S' + Kh^T U):
#   dU  = Kh D + P^T dO          dR = T^T dU            dX = dR
#   dP  = lower(dO U^T)          dA = strict_lower(-dR U^T)
#   dQs = dO S'^T + dP Kh        dE = -dR S'^T + dA Kh
#   dKh = U D^T + dA^T E + dP^T Qs
#   dS' = D + Qs^T dO - E^T dR   and the chunk-start gradient is diag(e^{g_C}) dS'
# Through E, Qs, Kh the in-chunk prefix g enters as g_r - g_C; with
# dg_r = dE_r*E_r + dQs_r*Qs_r - dKh_r*Kh_r and Phi = rowsum(dS' * S'),
# the log-decay gradient is d log alpha_i = Phi - sum_{r<i} dg_r.
# ---------------------------------------------------------------------------


def chunk_backward(q, k, v, la, b, w, S0, dO, dSf, C):
    BH, Tn, dk = q.shape
    dv = v.shape[-1]
    NC = Tn // C
    g = {n: np.zeros((BH, Tn, dk)) for n in ("dq", "dk", "dlog_alpha", "db")}
    g.update({n: np.zeros((BH, Tn, dv)) for n in ("dv", "dw")})
    g["dS0"] = np.zeros((BH, dk, dv))

    def prep(h, c):
        sl = slice(c * C, (c + 1) * C)
        gg = np.cumsum(la[h, sl], axis=0)
        gC = gg[-1]
        E = b[h, sl] * k[h, sl] * np.exp(gg - gC)
        Qs = q[h, sl] * np.exp(gg - gC)
        Kh = k[h, sl] * np.exp(gC - gg)
        A = np.tril(E @ Kh.T, -1)
        P = np.tril(Qs @ Kh.T, 0)
        return sl, gg, gC, E, Qs, Kh, _inv_unit_lower_blocked(A), P

    for h in range(BH):
        # 1. chunk-start states (forward recompute)
        states = np.zeros((NC, dk, dv))
        S = S0[h].copy()
        for c in range(NC):
            states[c] = S
            sl, gg, gC, E, Qs, Kh, T, P = prep(h, c)
            Sp = np.exp(gC)[:, None] * S
            U = T @ (w[h, sl] * v[h, sl] - E @ Sp)
            S = Sp + Kh.T @ U
        # 2. reverse pass over chunks: gradient of each chunk-end state
        dstates = np.zeros((NC, dk, dv))
        D = dSf[h].copy() if dSf is not None else np.zeros((dk, dv))
        for c in reversed(range(NC)):
            dstates[c] = D
            sl, gg, gC, E, Qs, Kh, T, P = prep(h, c)
            dR = T.T @ (Kh @ D + P.T @ dO[h, sl])
            D = np.exp(gC)[:, None] * (D + Qs.T @ dO[h, sl] - E.T @ dR)
        g["dS0"][h] = D
        # 3. per-chunk gradients, independent across chunks
        for c in range(NC):
            sl, gg, gC, E, Qs, Kh, T, P = prep(h, c)
            D, dOc = dstates[c], dO[h, sl]
            Sp = np.exp(gC)[:, None] * states[c]
            X = w[h, sl] * v[h, sl]
            U = T @ (X - E @ Sp)
            dR = T.T @ (Kh @ D + P.T @ dOc)
            dP = np.tril(dOc @ U.T, 0)
            dA = np.tril(-dR @ U.T, -1)
            dQs = dOc @ Sp.T + dP @ Kh
            dE = -dR @ Sp.T + dA @ Kh
            dKh = U @ D.T + dA.T @ E + dP.T @ Qs
            dSp = D + Qs.T @ dOc - E.T @ dR
            phi = np.sum(dSp * Sp, axis=1)
            dg = dE * E + dQs * Qs - dKh * Kh
            excl = np.cumsum(dg, axis=0) - dg
            eg, ek = np.exp(gg - gC), np.exp(gC - gg)
            g["dq"][h, sl] = dQs * eg
            g["dk"][h, sl] = dE * b[h, sl] * eg + dKh * ek
            g["db"][h, sl] = dE * k[h, sl] * eg
            g["dv"][h, sl] = dR * w[h, sl]
            g["dw"][h, sl] = dR * v[h, sl]
            g["dlog_alpha"][h, sl] = phi[None, :] - excl
    return g


@pytest.mark.parametrize("C,T,dk,dv,with_dsf", [(16, 64, 16, 16, False), (32, 96, 32, 16, True),
                                                (64, 128, 64, 32, True), (16, 48, 8, 24, True)])
def test_chunk_backward_matches_reverse_mode(C, T, dk, dv, with_dsf):
    q, k, v, la, b, w, S0 = _case(T, dk, dv, seed=3 * C + T)
    r = np.random.default_rng(C)
    dO = r.standard_normal(v.shape)
    dSf = r.standard_normal(S0.shape) if with_dsf else None
    ref = oracle.bwd(q, k, v, la, b, w, S0, dO, dSf)
    got = chunk_backward(q, k, v, la, b, w, S0, dO, dSf, C)
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        np.testing.assert_allclose(got[n], ref[n], rtol=1e-8, atol=1e-10, err_msg=n)

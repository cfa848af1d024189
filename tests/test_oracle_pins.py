"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test computes its expected value by a route that shares nothing with the
oracle's token loop: hand-worked fixtures, closed forms of special cases, a
brute-force product of materialised transition matrices, the Gated DeltaNet
form of the update written as the explainer page states it, linearity and
symmetry invariants, and finite differences for the reverse mode.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng


def _rand_case(T=12, dk=5, dv=4, seed=0, BH=2, decay=0.3, gate_hi=1.0):
    r = rng0(seed)
    q = r.standard_normal((BH, T, dk))
    k = r.standard_normal((BH, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((BH, T, dv))
    la = -r.random((BH, T, dk)) * decay
    b = r.random((BH, T, dk)) * gate_hi
    w = r.random((BH, T, dv)) * gate_hi
    S0 = r.standard_normal((BH, dk, dv))
    return q, k, v, la, b, w, S0


# ---------------------------------------------------------------- fixtures


def test_hand_worked_two_tokens():
    g = json.load(open(os.path.join(GOLD, "hand_fwd_two_tokens.json")))
    la = np.log(np.array(g["alpha"], dtype=np.float64))
    o, sf = oracle.fwd(np.array(g["q"], float)[None], np.array(g["k"], float)[None],
                       np.array(g["v"], float)[None], la[None], np.array(g["b"], float)[None],
                       np.array(g["w"], float)[None], np.array(g["S0"], float)[None])
    np.testing.assert_allclose(o[0], np.array(g["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf[0], np.array(g["S_final"]), rtol=0, atol=1e-13)


def test_hand_worked_scalar_backward():
    g = json.load(open(os.path.join(GOLD, "hand_bwd_scalar_step.json")))
    x = g["inputs"]
    a1 = lambda s: np.array([[[s]]], dtype=np.float64)  # [BH=1, T=1, 1]
    o, sf = oracle.fwd(a1(x["q"]), a1(x["k"]), a1(x["v"]), a1(np.log(x["alpha"])),
                       a1(x["b"]), a1(x["w"]), np.array([[[x["S0"]]]]))
    assert abs(o[0, 0, 0] - g["o"]) < 1e-13 and abs(sf[0, 0, 0] - g["S_final"]) < 1e-13
    gr = oracle.bwd(a1(x["q"]), a1(x["k"]), a1(x["v"]), a1(np.log(x["alpha"])), a1(x["b"]),
                    a1(x["w"]), np.array([[[x["S0"]]]]), a1(x["dO"]))
    for n, val in g["grads"].items():
        assert abs(float(gr[n].ravel()[0]) - val) < 1e-12, n


# ---------------------------------------------------------------- closed forms


def test_pure_decay_closed_form():
    """b = w = 0: only the decay acts, S_t = diag(exp(sum_{s<=t} log a_s)) S0."""
    q, k, v, la, b, w, S0 = _rand_case(T=20, dk=6, dv=3)
    z = np.zeros_like(b)
    o, sf = oracle.fwd(q, k, v, la, z, np.zeros_like(w), S0)
    g = np.cumsum(la, axis=1)                                   # [BH, T, dk]
    S_t = np.exp(g)[..., None] * S0[:, None]                    # [BH, T, dk, dv]
    np.testing.assert_allclose(o, np.einsum("htij,hti->htj", S_t, q), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sf, S_t[:, -1], rtol=1e-12, atol=1e-12)


def test_write_only_is_decayed_linear_attention():
    """b = 0: no erase; S_T = G_T S0 + sum_s diag(exp(g_T - g_s)) k_s (w_s*v_s)^T."""
    q, k, v, la, b, w, S0 = _rand_case(T=15, dk=4, dv=5, seed=3)
    o, sf = oracle.fwd(q, k, v, la, np.zeros_like(b), w, S0)
    g = np.cumsum(la, axis=1)
    T = q.shape[1]
    exp_o = np.zeros_like(o)
    for t in range(T):
        St = np.exp(g[:, t])[..., None] * S0
        for s in range(t + 1):
            St = St + np.einsum("hi,hj->hij", np.exp(g[:, t] - g[:, s]) * k[:, s], w[:, s] * v[:, s])
        exp_o[:, t] = np.einsum("hij,hi->hj", St, q[:, t])
        if t == T - 1:
            np.testing.assert_allclose(sf, St, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-12)


def test_delta_rule_overwrite():
    """alpha = 1, b = w = 1, |k| = 1: after the write S_t^T k_t = v_t exactly."""
    q, k, v, la, b, w, S0 = _rand_case(T=10, dk=8, dv=6, seed=5)
    o, _ = oracle.fwd(k, k, v, np.zeros_like(la), np.ones_like(b), np.ones_like(w), S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_overwrite_with_decay_and_write_gate():
    """b = 1, |k| = 1, any decay: S_t^T k_t = w_t * v_t (erase removes the whole read)."""
    q, k, v, la, b, w, S0 = _rand_case(T=10, dk=8, dv=6, seed=6)
    o, _ = oracle.fwd(k, k, v, la, np.ones_like(b), w, S0)
    np.testing.assert_allclose(o, w * v, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- reductions


def _gdn_form(q, k, v, alpha, beta, S0):
    """Gated DeltaNet as the explainer page writes it:
    S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T,  o_t = S_t^T q_t."""
    BH, T, dk = q.shape
    o = np.zeros(v.shape)
    S = S0.copy()
    for h in range(BH):
        for t in range(T):
            kk = k[h, t][:, None]
            M = alpha[h, t] * (np.eye(dk) - beta[h, t] * kk @ kk.T)
            S[h] = M @ S[h] + beta[h, t] * kk @ v[h, t][None, :]
            o[h, t] = S[h].T @ q[h, t]
    return o, S


def _kda_form(q, k, v, la, beta, S0):
    """KDA: channel decay, one scalar gate for erase and write:
    S_t = (I - beta k k^T) diag(alpha_t) S + beta k v^T."""
    BH, T, dk = q.shape
    o = np.zeros(v.shape)
    S = S0.copy()
    for h in range(BH):
        for t in range(T):
            kk = k[h, t][:, None]
            S[h] = (np.eye(dk) - beta[h, t] * kk @ kk.T) @ (np.exp(la[h, t])[:, None] * S[h]) \
                + beta[h, t] * kk @ v[h, t][None, :]
            o[h, t] = S[h].T @ q[h, t]
    return o, S


def _prefix_states(q, k, v, la, b, w, S0):
    """S_t after each token t = 1..T (the oracle run on every prefix)."""
    T = q.shape[-2]
    return [oracle.fwd(q[:, :t], k[:, :t], v[:, :t], la[:, :t], b[:, :t], w[:, :t], S0)[1]
            for t in range(1, T + 1)]


def test_full_erase_is_a_reflection():
    """Expanded erase range ("Gated DeltaNet-2 Review" §5; sungsoo commentary):
    with b = 2, no write, no decay and |k| = 1 the transition is the
    reflection I - 2 k k^T, which has eigenvalue -1 along k.  So every step
    keeps the Frobenius norm of the state and flips the sign of k_t^T S."""
    q, k, v, la, b, w, S0 = _rand_case(T=9, dk=8, dv=5, seed=21)
    two = np.full_like(b, 2.0)
    Ss = _prefix_states(q, k, v, np.zeros_like(la), two, np.zeros_like(w), S0)
    prev = S0
    for t, St in enumerate(Ss):
        np.testing.assert_allclose(np.linalg.norm(St, axis=(1, 2)), np.linalg.norm(S0, axis=(1, 2)),
                                   rtol=1e-12)
        kt = k[:, t]
        np.testing.assert_allclose(np.einsum("bi,bij->bj", kt, St),
                                   -np.einsum("bi,bij->bj", kt, prev), rtol=0, atol=1e-12)
        prev = St


def test_full_erase_twice_restores_the_state():
    """The same key twice at b = 2 (no write, no decay) is a reflection
    applied twice: the state comes back unchanged."""
    q, k, v, la, b, w, S0 = _rand_case(T=6, dk=7, dv=4, seed=22)
    k = np.repeat(k[:, :3], 2, axis=1)             # k1 k1 k2 k2 k3 k3
    _, Sf = oracle.fwd(q, k, v, np.zeros_like(la), np.full_like(b, 2.0), np.zeros_like(w), S0)
    np.testing.assert_allclose(Sf, S0, rtol=0, atol=1e-12)


def test_erase_gates_up_to_two_never_grow_the_state():
    """With |k| = 1, decay <= 1 and a per-token erase gate b in [0, 2] (the
    same for every channel), the transition (I - b k k^T) D is a contraction
    (eigenvalues 1 and 1 - b of the symmetric erase factor, times a decay of
    at most 1), so with no write the state's norm never increases."""
    q, k, v, la, b, w, S0 = _rand_case(T=16, dk=6, dv=5, seed=23, decay=0.5)
    bt = rng0(24).random((b.shape[0], b.shape[1], 1)) * 2.0
    Ss = _prefix_states(q, k, v, la, np.broadcast_to(bt, b.shape).copy(), np.zeros_like(w), S0)
    norms = [np.linalg.norm(S0, axis=(1, 2))] + [np.linalg.norm(St, axis=(1, 2)) for St in Ss]
    for a0, a1 in zip(norms, norms[1:]):
        assert np.all(a1 <= a0 * (1 + 1e-12))
    assert np.all(norms[-1] < norms[0] * 0.99)     # and it does shrink


def test_tied_scalar_gates_give_gated_deltanet():
    q, k, v, la, b, w, S0 = _rand_case(T=16, dk=6, dv=5, seed=7)
    r = rng0(70)
    alpha = r.uniform(0.8, 1.0, size=q.shape[:2])
    beta = r.random(q.shape[:2])
    o, sf = oracle.fwd(q, k, v, np.log(alpha), beta, beta, S0)        # scalar gates broadcast
    o2, s2 = _gdn_form(q, k, v, alpha, beta, S0)
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sf, s2, rtol=1e-11, atol=1e-12)


def test_tied_gates_with_channel_decay_give_kda():
    q, k, v, la, b, w, S0 = _rand_case(T=16, dk=6, dv=5, seed=8)
    beta = rng0(80).random(q.shape[:2])
    o, sf = oracle.fwd(q, k, v, la, beta, beta, S0)
    o2, s2 = _kda_form(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sf, s2, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- brute force


def _brute_force(q, k, v, la, b, w, S0):
    """Materialise M_t = (I - k_t (b_t*k_t)^T) diag(exp(la_t)) and expand
    S_t = M_t...M_1 S0 + sum_s M_t...M_{s+1} k_s (w_s*v_s)^T for every t."""
    BH, T, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((BH, T, dv))
    Sf = np.zeros((BH, dk, dv))
    for h in range(BH):
        M = [(np.eye(dk) - np.outer(k[h, t], b[h, t] * k[h, t])) @ np.diag(np.exp(la[h, t]))
             for t in range(T)]
        for t in range(T):
            prod = np.eye(dk)
            for s in range(t, -1, -1):
                prod = prod @ M[s]
            St = prod @ S0[h]
            for s in range(t + 1):
                P = np.eye(dk)
                for u in range(t, s, -1):
                    P = P @ M[u]
                St = St + P @ np.outer(k[h, s], w[h, s] * v[h, s])
            o[h, t] = St.T @ q[h, t]
            if t == T - 1:
                Sf[h] = St
    return o, Sf


@pytest.mark.parametrize("T,dk,dv,hi", [(16, 5, 3, 1.0), (9, 3, 7, 2.0), (16, 8, 8, 1.0)])
def test_brute_force_transition_products(T, dk, dv, hi):
    q, k, v, la, b, w, S0 = _rand_case(T=T, dk=dk, dv=dv, seed=T + dk, gate_hi=hi, decay=0.5)
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    o2, s2 = _brute_force(q, k, v, la, b, w, S0)
    np.testing.assert_allclose(o, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sf, s2, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- invariants


def test_linear_in_state_and_values():
    q, k, v, la, b, w, S0 = _rand_case(T=14, dk=5, dv=4, seed=11)
    f = lambda s0, vv: oracle.fwd(q, k, vv, la, b, w, s0)
    o_full, s_full = f(S0, v)
    o_a, s_a = f(S0, np.zeros_like(v))
    o_b, s_b = f(np.zeros_like(S0), v)
    np.testing.assert_allclose(o_full, o_a + o_b, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s_full, s_a + s_b, rtol=1e-11, atol=1e-12)
    o_l, s_l = f(2.5 * S0, 2.5 * v)
    np.testing.assert_allclose(o_l, 2.5 * o_full, rtol=1e-11, atol=1e-12)


def test_channel_permutation_symmetry():
    q, k, v, la, b, w, S0 = _rand_case(T=14, dk=6, dv=5, seed=12)
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    pv = rng0(1).permutation(5)
    o2, s2 = oracle.fwd(q, k, v[..., pv], la, b, w[..., pv], S0[..., pv])
    np.testing.assert_allclose(o2, o[..., pv], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, sf[..., pv], rtol=1e-12, atol=1e-13)
    pk = rng0(2).permutation(6)
    o3, s3 = oracle.fwd(q[..., pk], k[..., pk], v, la[..., pk], b[..., pk], w, S0[:, pk, :])
    np.testing.assert_allclose(o3, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, sf[:, pk, :], rtol=1e-11, atol=1e-12)


def test_split_sequence_continuity_and_decode():
    """fwd(T) = fwd(T1) then fwd(T-T1) from the carried state = T single steps."""
    q, k, v, la, b, w, S0 = _rand_case(T=13, dk=4, dv=3, seed=13)
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    o1, s1 = oracle.fwd(q[:, :5], k[:, :5], v[:, :5], la[:, :5], b[:, :5], w[:, :5], S0)
    o2, s2 = oracle.fwd(q[:, 5:], k[:, 5:], v[:, 5:], la[:, 5:], b[:, 5:], w[:, 5:], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, sf, rtol=1e-12, atol=1e-13)
    S = S0.copy()
    for t in range(13):
        ot, S = oracle.decode(q[:, t], k[:, t], v[:, t], la[:, t], b[:, t], w[:, t], S)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, sf, rtol=1e-12, atol=1e-13)


def test_decode_scalar_gate_broadcast():
    r = rng0(14)
    NH, dk, dv = 6, 4, 5
    q, k = r.standard_normal((NH, dk)), r.standard_normal((NH, dk))
    v, S = r.standard_normal((NH, dv)), r.standard_normal((NH, dk, dv))
    la, beta = -r.random(NH), r.random(NH)
    o, Sn = oracle.decode(q, k, v, la, beta, beta, S)
    o2, s2 = _gdn_form(q[:, None], k[:, None], v[:, None], np.exp(la)[:, None], beta[:, None], S)
    np.testing.assert_allclose(o, o2[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sn, s2, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- reverse mode


def _loss(args, dO, dSf):
    o, sf = oracle.fwd(*args)
    return float(np.sum(dO * o) + (0.0 if dSf is None else np.sum(dSf * sf)))


@pytest.mark.parametrize("with_dsf", [False, True])
def test_backward_finite_differences(with_dsf):
    """Central differences along random directions, T=32 (longer than the
    oracle's 64-token checkpoint segment is covered in the next test)."""
    T, dk, dv = 32, 5, 4
    q, k, v, la, b, w, S0 = _rand_case(T=T, dk=dk, dv=dv, seed=21, BH=1)
    r = rng0(22)
    dO = r.standard_normal(v.shape)
    dSf = r.standard_normal(S0.shape) if with_dsf else None
    g = oracle.bwd(q, k, v, la, b, w, S0, dO, dSf)
    names = ["q", "k", "v", "log_alpha", "b", "w", "S0"]
    gnames = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]
    base = [q, k, v, la, b, w, S0]
    eps = 1e-6
    for i, (n, gn) in enumerate(zip(names, gnames)):
        for trial in range(2):
            d = r.standard_normal(base[i].shape)
            plus = list(base); minus = list(base)
            plus[i] = base[i] + eps * d
            minus[i] = base[i] - eps * d
            fd = (_loss(plus, dO, dSf) - _loss(minus, dO, dSf)) / (2 * eps)
            an = float(np.sum(g[gn] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, fd, an)


def test_backward_across_checkpoint_segments():
    """T=150 spans three 64-token recompute segments; compare with T=150 finite
    differences on a few coordinates of every input."""
    T, dk, dv = 150, 3, 2
    q, k, v, la, b, w, S0 = _rand_case(T=T, dk=dk, dv=dv, seed=31, BH=1, decay=0.05)
    dO = rng0(32).standard_normal(v.shape)
    g = oracle.bwd(q, k, v, la, b, w, S0, dO)
    eps = 1e-6
    base = [q, k, v, la, b, w, S0]
    gnames = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]
    for i, gn in enumerate(gnames):
        for idx in [(0, 3, 0), (0, 70, 1), (0, 149, 0)] if i < 6 else [(0, 1, 1)]:
            plus = list(base); minus = list(base)
            plus[i] = base[i].copy(); minus[i] = base[i].copy()
            plus[i][idx] += eps
            minus[i][idx] -= eps
            fd = (_loss(plus, dO, None) - _loss(minus, dO, None)) / (2 * eps)
            assert abs(fd - g[gn][idx]) <= 1e-6 * max(1.0, abs(fd)), (gn, idx, fd, g[gn][idx])


def test_backward_tied_gate_reduction():
    """With tied scalar gates (Gated DeltaNet) the scalar gradients are the sums
    of the channel ones: d beta = sum_c db_c + sum_j dw_j, d log alpha = sum_c."""
    T, dk, dv = 20, 4, 3
    q, k, v, la, b, w, S0 = _rand_case(T=T, dk=dk, dv=dv, seed=41, BH=1)
    r = rng0(42)
    la_s = -r.random((1, T)) * 0.3
    beta = r.random((1, T))
    dO = r.standard_normal(v.shape)
    g = oracle.bwd(q, k, v, la_s, beta, beta, S0, dO)
    dbeta = g["db"].sum(-1) + g["dw"].sum(-1)
    dla = g["dlog_alpha"].sum(-1)
    eps = 1e-6

    def L(la_, beta_):
        o, _ = _gdn_form(q, k, v, np.exp(la_), beta_, S0)
        return float(np.sum(dO * o))
    for t in (0, 7, 19):
        e = np.zeros((1, T)); e[0, t] = eps
        fd_b = (L(la_s, beta + e) - L(la_s, beta - e)) / (2 * eps)
        fd_a = (L(la_s + e, beta) - L(la_s - e, beta)) / (2 * eps)
        assert abs(fd_b - dbeta[0, t]) < 1e-6 * max(1, abs(fd_b))
        assert abs(fd_a - dla[0, t]) < 1e-6 * max(1, abs(fd_a))

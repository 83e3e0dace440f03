"""Pins for the backward oracle (oracle/backward.py): fp64 autograd through the
serial recurrence is checked against things other than itself -- the C
oracle's forward, central finite differences of that forward, the exact
linearity of the output in v, and hand-derived closed forms for one token and
for the vanishing-decay limit.
"""
import math

import numpy as np
import pytest
import torch

from oracle import backward as ob


def rnd(seed, *shapes, scale=0.5):
    r = np.random.default_rng(seed)
    return [r.standard_normal(s) * scale for s in shapes]


def loss(oracle_mod, q, k, v, dout, g, lam, norm):
    out, _, _ = oracle_mod.forward(q, k, v, gamma=g, lam=lam, normalize=norm, want_state=False)
    return float((out * dout).sum())


CASES = [  # (gamma per head, ridge, normalize)
    (None, 0.0, False),
    ([0.9, 0.6], 0.0, False),
    ([0.95, 0.8], 0.25, False),
    ([0.97, 0.85], 0.25, True),
    (None, 0.0, True),
]


@pytest.mark.parametrize("g,lam,norm", CASES)
def test_forward_recurrence_matches_c_oracle(oracle_mod, g, lam, norm):
    q, k, v = rnd(11, (2, 2, 17, 5), (2, 2, 17, 5), (2, 2, 17, 3))
    out, den = ob.forward_recurrence(*(torch.tensor(x) for x in (q, k, v)), g, lam, norm)
    ro, rd, _ = oracle_mod.forward(q, k, v, gamma=g, lam=lam, normalize=norm, want_state=False)
    assert np.abs(out.numpy() - ro).max() <= 1e-12 * max(1.0, np.abs(ro).max())
    assert np.abs(den.numpy() - rd).max() <= 1e-12 * max(1.0, np.abs(rd).max())


@pytest.mark.parametrize("g,lam,norm", CASES)
@pytest.mark.parametrize("which", [0, 1, 2])
def test_gradients_match_finite_differences(oracle_mod, g, lam, norm, which):
    """Directional derivative of the C oracle's loss along a random direction of
    one input (central difference, O(eps^2) truncation) against <grad, u>."""
    B, H, n, d, dv = 1, 2, 11, 4, 3
    q, k, v, dout = rnd(21 + which, (B, H, n, d), (B, H, n, d), (B, H, n, dv), (B, H, n, dv))
    if norm:  # keep denominators away from zero: positive-leaning q, k
        q, k = np.abs(q) + 0.3, np.abs(k) + 0.3
    grads = ob.backward(q, k, v, dout, g, lam, norm)
    xs = [q, k, v]
    u = rnd(31 + which, xs[which].shape, scale=1.0)[0]
    eps = 1e-5
    plus = [x.copy() for x in xs]; minus = [x.copy() for x in xs]
    plus[which] += eps * u; minus[which] -= eps * u
    fd = (loss(oracle_mod, *plus, dout, g, lam, norm) - loss(oracle_mod, *minus, dout, g, lam, norm)) / (2 * eps)
    an = float((grads[which] * u).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("g,lam", [(None, 0.0), ([0.9, 0.7], 0.3)])
def test_dv_is_exact_for_the_linear_map(oracle_mod, g, lam):
    """Without the ratio, out is linear in v: L(v + u) - L(v) = <dv, u> exactly
    (no truncation error), for any u."""
    q, k, v, dout, u = rnd(41, (1, 2, 23, 4), (1, 2, 23, 4), (1, 2, 23, 3), (1, 2, 23, 3), (1, 2, 23, 3))
    _, _, dv = ob.backward(q, k, v, dout, g, lam, False)
    lhs = loss(oracle_mod, q, k, v + u, dout, g, lam, False) - loss(oracle_mod, q, k, v, dout, g, lam, False)
    assert abs(lhs - float((dv * u).sum())) <= 1e-11 * max(1.0, abs(lhs))


def test_single_token_closed_form():
    """One token: out = ((q.k)^2 + lam |q|^2) v, so with a = v . dout,
    dv = ((q.k)^2 + lam |q|^2) dout, dq = (2 (q.k) k + 2 lam q) a, dk = 2 (q.k) q a."""
    q, k, v, dout = rnd(51, (1, 1, 1, 6), (1, 1, 1, 6), (1, 1, 1, 4), (1, 1, 1, 4))
    lam = 0.7
    dq, dk, dv = ob.backward(q, k, v, dout, [0.8], lam, False)
    qk = float(q.ravel() @ k.ravel())
    a = float(v.ravel() @ dout.ravel())
    np.testing.assert_allclose(dv.ravel(), (qk * qk + lam * float(q.ravel() @ q.ravel())) * dout.ravel(), rtol=1e-13)
    np.testing.assert_allclose(dq.ravel(), (2 * qk * k.ravel() + 2 * lam * q.ravel()) * a, rtol=1e-13)
    np.testing.assert_allclose(dk.ravel(), 2 * qk * q.ravel() * a, rtol=1e-13)


def test_vanishing_decay_is_tokenwise():
    """With g -> 0 every token sees only itself, so each row follows the
    one-token closed form (g = 1e-30: cross-token terms are below 1e-30)."""
    n = 9
    q, k, v, dout = rnd(61, (1, 1, n, 3), (1, 1, n, 3), (1, 1, n, 2), (1, 1, n, 2))
    dq, dk, dv = ob.backward(q, k, v, dout, [1e-30], 0.0, False)
    for t in range(n):
        qt, kt, vt, gt = q[0, 0, t], k[0, 0, t], v[0, 0, t], dout[0, 0, t]
        qk, a = qt @ kt, vt @ gt
        np.testing.assert_allclose(dv[0, 0, t], qk * qk * gt, rtol=1e-12, atol=1e-25)
        np.testing.assert_allclose(dq[0, 0, t], 2 * qk * kt * a, rtol=1e-12, atol=1e-25)
        np.testing.assert_allclose(dk[0, 0, t], 2 * qk * qt * a, rtol=1e-12, atol=1e-25)


def test_empty_sequence():
    dq, dk, dv = ob.backward(np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 3)),
                             np.zeros((1, 2, 0, 3)))
    assert dq.shape == (1, 2, 0, 4) and dk.shape == (1, 2, 0, 4) and dv.shape == (1, 2, 0, 3)


def test_causality_of_gradients():
    """dout at token t only reaches inputs at tokens <= t."""
    n, t = 12, 6
    q, k, v = rnd(71, (1, 1, n, 4), (1, 1, n, 4), (1, 1, n, 3))
    dout = np.zeros((1, 1, n, 3)); dout[0, 0, t] = 1.0
    grads = ob.backward(q, k, v, dout, [0.9], 0.2, False)
    for gr in grads:
        assert np.all(gr[0, 0, t + 1:] == 0.0)
        assert np.any(gr[0, 0, :t + 1] != 0.0)


def test_forward_recurrence_from_a_state_matches_c_oracle(oracle_mod):
    """With an init state (a method-produced state of a prefix, from the C
    oracle), the torch recurrence continues exactly like the C oracle."""
    q, k, v = rnd(81, (1, 2, 30, 4), (1, 2, 30, 4), (1, 2, 30, 3))
    g = [0.9, 0.8]
    _, _, st = oracle_mod.forward(q[:, :, :12], k[:, :, :12], v[:, :, :12], gamma=g, lam=0.2)
    ro, rd, _ = oracle_mod.forward(q[:, :, 12:], k[:, :, 12:], v[:, :, 12:], gamma=g, lam=0.2, init=st,
                                   want_state=False)
    out, den = ob.forward_recurrence(*(torch.tensor(x[:, :, 12:]) for x in (q, k, v)), g, 0.2, False, st)
    assert np.abs(out.numpy() - ro).max() <= 1e-12 * max(1.0, np.abs(ro).max())
    assert np.abs(den.numpy() - rd).max() <= 1e-12 * max(1.0, np.abs(rd).max())


def test_gradients_from_a_state_are_those_of_the_whole_sequence(oracle_mod):
    """Splitting a sequence and continuing from the (detached) prefix state
    leaves the gradients of the suffix inputs that only suffix outputs reach
    unchanged: with dout zero on the prefix, the whole-sequence gradients of
    the suffix tokens equal the split ones."""
    q, k, v, dout = rnd(91, (1, 2, 26, 4), (1, 2, 26, 4), (1, 2, 26, 3), (1, 2, 26, 3))
    g, p = [0.95, 0.85], 10
    dout[:, :, :p] = 0.0
    whole = ob.backward(q, k, v, dout, g, 0.3, False)
    _, _, st = oracle_mod.forward(q[:, :, :p], k[:, :, :p], v[:, :, :p], gamma=g, lam=0.3)
    part = ob.backward(q[:, :, p:], k[:, :, p:], v[:, :, p:], dout[:, :, p:], g, 0.3, False, st)
    for a, b in zip(whole, part):
        np.testing.assert_allclose(a[:, :, p:], b, rtol=1e-11, atol=1e-13)


def _prefix_state(oracle_mod, seed, B, H, p, d, dv, g, lam):
    """A method-produced state (symmetric S) from a random prefix of p tokens,
    with C, m, G, h then moved off the method's manifold by random offsets so
    every part of the initial state is an independent variable."""
    q, k, v = rnd(seed, (B, H, p, d), (B, H, p, d), (B, H, p, dv))
    _, _, st = oracle_mod.forward(q, k, v, gamma=g, lam=lam)
    N = B * H
    oC, om, oG, oh = rnd(seed + 1, (N, d, dv), (N, d), (N, d, dv), (N, d), scale=0.3)
    st.C = st.C + oC; st.m = st.m + om; st.G = st.G + oG; st.h = st.h + oh
    return st


@pytest.mark.parametrize("g,lam,norm", CASES)
@pytest.mark.parametrize("part", ["S", "C", "m", "G", "h"])
def test_init_gradients_match_finite_differences(oracle_mod, g, lam, norm, part):
    """Directional derivative of the C oracle's loss along a random direction
    of one part of the initial state (symmetric for S, the form the method's
    states take) against <dinit, u>."""
    B, H, n, d, dv = 1, 2, 9, 4, 3
    q, k, v, dout = rnd(41, (B, H, n, d), (B, H, n, d), (B, H, n, dv), (B, H, n, dv))
    if norm:
        q, k = np.abs(q) + 0.3, np.abs(k) + 0.3
    st = _prefix_state(oracle_mod, 43, B, H, 5, d, dv, g, lam)
    if norm:  # positive-leaning prefix: denominators stay away from zero
        st.m = np.abs(st.m) + 0.5; st.h = 0.1 * st.h
    *_, dini = ob.backward(q, k, v, dout, g, lam, norm, st, init_grad=True)
    base = getattr(st, part)
    u = rnd(47, base.shape, scale=1.0)[0]
    if part == "S":
        u = u + np.swapaxes(u, -1, -2)
    eps = 1e-5

    def moved(sign):
        s2 = st.__class__(st.S.copy(), st.C.copy(), st.m.copy(), st.G.copy(), st.h.copy(), st.rho.copy())
        setattr(s2, part, base + sign * eps * u)
        out, _, _ = oracle_mod.forward(q, k, v, gamma=g, lam=lam, normalize=norm, init=s2, want_state=False)
        return float((out * dout).sum())

    fd = (moved(1) - moved(-1)) / (2 * eps)
    an = float((dini[part] * u).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def test_init_gradient_of_a_zero_state_is_the_prefix_chain_rule(oracle_mod):
    """Gradients with respect to a zero initial state, checked against the
    whole sequence: with the read-out of token t equal to q_t^T X_t where
    X_t = g^2 X_{t-1} + S_t q_t v_t^T (X = S C - G), the gradient of G_{-1}
    is -sum_t g^(2(t+1)) q_t dout_t^T, which a prepended token with k = 0
    cannot change.  Also: with no ridge and no ratio, dC_{-1} and dm_{-1}
    vanish at S_{-1} = 0, and dh_{-1} is zero without the ratio."""
    B, H, n, d, dv = 1, 2, 10, 4, 3
    q, k, v, dout = rnd(51, (B, H, n, d), (B, H, n, d), (B, H, n, dv), (B, H, n, dv))
    g = [0.9, 0.7]
    *_, dini = ob.backward(q, k, v, dout, g, 0.0, False, None, init_grad=True)
    gg = np.asarray(g)
    pw = gg[:, None] ** (2 * (np.arange(n)[None, :] + 1))          # [H, n]
    want_G = -np.einsum("hn,hna,hnj->haj", pw, q[0], dout[0])
    np.testing.assert_allclose(dini["G"], want_G, rtol=1e-12, atol=1e-14)
    # the S_t C_t and G_t paths cancel exactly in the algebra, to rounding here
    assert np.abs(dini["C"]).max() <= 1e-13 and np.abs(dini["m"]).max() <= 1e-13
    assert np.all(dini["h"] == 0.0)
    # dS at S_{-1} = 0, C_{-1} = 0: sum_j g^(j+1) q_j w_j^T with w_j = Gb_j v_j,
    # Gb_j = sum_{t>=j} g^(2(t-j)) q_t dout_t^T -- written out per token here
    want_S = np.zeros((H, d, d))
    for hh in range(H):
        for j in range(n):
            Gb = sum(gg[hh] ** (2 * (t - j)) * np.outer(q[0, hh, t], dout[0, hh, t]) for t in range(j, n))
            want_S[hh] += gg[hh] ** (j + 1) * np.outer(q[0, hh, j], Gb @ v[0, hh, j])
    np.testing.assert_allclose(dini["S"], want_S, rtol=1e-11, atol=1e-13)


def test_init_gradient_empty_sequence():
    *_, dini = ob.backward(np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 3)),
                           np.zeros((1, 2, 0, 3)), init_grad=True)
    assert dini["S"].shape == (2, 4, 4) and dini["C"].shape == (2, 4, 3)
    assert all(np.all(x == 0.0) for x in dini.values())


def _fin_loss(oracle_mod, q, k, v, dout, g, lam, norm, st, dfin):
    out, _, fin = oracle_mod.forward(q, k, v, gamma=g, lam=lam, normalize=norm, init=st)
    tot = float((out * dout).sum())
    for name in ("S", "C", "m", "G", "h"):
        tot += float((getattr(fin, name) * dfin[name]).sum())
    return tot


@pytest.mark.parametrize("g,lam,norm", CASES)
@pytest.mark.parametrize("which", ["q", "k", "v", "S", "C", "G"])
def test_final_state_gradients_match_finite_differences(oracle_mod, g, lam, norm, which):
    """With a gradient flowing into the final state, <grad, u> for a random
    direction of an input or of a part of the initial state against central
    differences of the C oracle's loss sum <out, dout> + sum <fin, dfin>."""
    B, H, n, d, dv = 1, 2, 9, 4, 3
    q, k, v, dout = rnd(61, (B, H, n, d), (B, H, n, d), (B, H, n, dv), (B, H, n, dv))
    if norm:
        q, k = np.abs(q) + 0.3, np.abs(k) + 0.3
    st = _prefix_state(oracle_mod, 63, B, H, 4, d, dv, g, lam)
    if norm:
        st.m = np.abs(st.m) + 0.5; st.h = 0.1 * st.h
    N = B * H
    dfin = dict(zip(("S", "C", "m", "G", "h"),
                    rnd(65, (N, d, d), (N, d, dv), (N, d), (N, d, dv), (N, d), scale=0.7)))
    import types
    dq, dk, dv_, dini = ob.backward(q, k, v, dout, g, lam, norm, st, init_grad=True,
                                    dfinal=types.SimpleNamespace(**dfin))
    eps = 1e-5
    xs = {"q": q, "k": k, "v": v}
    if which in xs:
        base, an_grad = xs[which], {"q": dq, "k": dk, "v": dv_}[which]
    else:
        base, an_grad = getattr(st, which), dini[which]
    u = rnd(67, base.shape, scale=1.0)[0]
    if which == "S":
        u = u + np.swapaxes(u, -1, -2)

    def moved(sign):
        s2 = st.__class__(st.S.copy(), st.C.copy(), st.m.copy(), st.G.copy(), st.h.copy(), st.rho.copy())
        x2 = {kk: vv.copy() for kk, vv in xs.items()}
        if which in x2:
            x2[which] = base + sign * eps * u
        else:
            setattr(s2, which, base + sign * eps * u)
        return _fin_loss(oracle_mod, x2["q"], x2["k"], x2["v"], dout, g, lam, norm, s2, dfin)

    fd = (moved(1) - moved(-1)) / (2 * eps)
    an = float((an_grad * u).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def test_final_state_gradient_of_an_empty_sequence_is_passed_through(oracle_mod):
    """n = 0: the final state is the initial one, so dinit = dfinal."""
    import types
    d, dv = 4, 3
    st = _prefix_state(oracle_mod, 69, 1, 2, 5, d, dv, [0.9, 0.8], 0.0)
    dfin = dict(zip(("S", "C", "m", "G", "h"), rnd(70, (2, d, d), (2, d, dv), (2, d), (2, d, dv), (2, d))))
    *_, dini = ob.backward(np.zeros((1, 2, 0, d)), np.zeros((1, 2, 0, d)), np.zeros((1, 2, 0, dv)),
                           np.zeros((1, 2, 0, dv)), [0.9, 0.8], 0.0, False, st, init_grad=True,
                           dfinal=types.SimpleNamespace(**dfin))
    for name in dfin:
        np.testing.assert_array_equal(dini[name], dfin[name])

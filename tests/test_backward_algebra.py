"""The chunked evaluation order of the backward kernels, written out in numpy
fp64 and checked against the autograd oracle (oracle/backward.py).  It pins
the algebra of the GPU design on the CPU and shares no code with the HIP path.

With the value rows widened by a constant 1 (V^ = [V | 1]) and the upstream
gradient of a token written as g^_t = [dnum_t | dden_t] (dnum = dout,
dden = 0 for the plain output; dnum = dout/den, dden = -(dout . out)/den for
the ratio), num and den are one linear map of V^, and the gradient is that
of a single masked second-order scan run in reverse time:

  u_j = S_j q_j                           (forward: S_j = sum_{i<=j} g^(j-i) k_i k_i^T)
  Gb_j = sum_{t>=j} g^(2(t-j)) q_t g^_t^T  Cb_j = sum_{t>=j} g^(t-j) q_t g^_t^T
  w_j = Gb_j v^_j                         T_i = sum_{j>=i} g^(j-i) (w_j q_j^T + q_j w_j^T)
  dq_t = X^_t g^_t + S_t w_t + lam (C^_t g^_t + Cb_t v^_t)
  dk_i = T_i k_i                          dv_j = Gb_j^T u_j + lam Cb_j^T q_j   (first dv columns)

where X^_t = [X_t | y_t] and C^_t = [C_t | m_t] are the forward's corrected
carries.  Per chunk (local tau; e = g^(tau+1), eh = g^(L-tau); carries from
the left (S0, X0, y0, C0, m0) and from the right (Gb', Cb', T')):

  Gam  = Gn V^T + gd 1^T,  Gam1 = Gam o D_g o L,  Gam2 = Gam o D_{g^2} o L
  W    = Gam2^T Q + diag(eh^2) (V Gbn'^T + 1 gbd'^T)
  dQ   = diag(e^2)(Gn X0^T + gd y0^T) + Gam2 U + diag(e) W S0 + ((W K^T) o D_g o L) K
         + lam [diag(e)(Gn C0^T + gd m0^T) + Gam1 Q + Gam1^T Q + diag(eh)(V Cbn'^T + 1 cbd'^T)]
  dK   = ((K Q^T) o Mu) W + ((K W^T) o Mu) Q + diag(eh) K T'       (Mu = (D_g o L)^T)
  dV   = P^T Gn + diag(eh^2) U Gbn' + lam diag(eh) Q Cbn'           (P: the forward's masked matrix)
  right-to-left carries: Gb <- Q^T diag(g^(2 tau)) G^ + g^(2L) Gb',  Cb likewise with g^tau, g^L,
                         T  <- W^T diag(g^tau) Q + Q^T diag(g^tau) W + g^L T'
"""
import numpy as np
import pytest

from oracle import backward as ob


def chunked_backward(Q, K, V, Gout, g, lam, norm, w):
    n, d = Q.shape
    dv = V.shape[1]
    chunks = [(s, min(w, n - s)) for s in range(0, n, w)]
    nc = len(chunks)
    # forward chunk algebra: carries before each chunk, U per chunk, num, den
    S0 = np.zeros((d, d)); C0 = np.zeros((d, dv)); m0 = np.zeros(d)
    X0 = np.zeros((d, dv)); y0 = np.zeros(d)
    carry, Us = [], []
    num = np.zeros((n, dv)); den = np.zeros(n)
    for s, L in chunks:
        Qc, Kc, Vc = Q[s:s + L], K[s:s + L], V[s:s + L]
        tau = np.arange(L)
        e, f = g ** (tau + 1.0), g ** (L - 1.0 - tau)
        diff = tau[:, None] - tau[None, :]
        Dg = np.where(diff >= 0, g ** np.maximum(diff, 0).astype(float), 0.0)
        A = (Qc @ Kc.T) * Dg
        U = e[:, None] * (Qc @ S0) + A @ Kc
        P = (Qc @ U.T) * Dg * Dg + lam * (Qc @ Qc.T) * Dg
        num[s:s + L] = P @ Vc + (e * e)[:, None] * (Qc @ X0) + lam * e[:, None] * (Qc @ C0)
        den[s:s + L] = P.sum(1) + e * e * (Qc @ y0) + lam * e * (Qc @ m0)
        carry.append((S0, C0, m0, X0, y0)); Us.append(U)
        rho = g ** float(L)
        S0 = rho * S0 + Kc.T @ (f[:, None] * Kc)
        C0 = rho * C0 + Qc.T @ (f[:, None] * Vc)
        m0 = rho * m0 + Qc.T @ f
        X0 = rho * rho * X0 + U.T @ ((f * f)[:, None] * Vc)
        y0 = rho * rho * y0 + U.T @ (f * f)
    if norm:
        o = num / den[:, None]
        Gn = Gout / den[:, None]
        gd = -(Gout * o).sum(1) / den
    else:
        Gn, gd = Gout, np.zeros(n)
    # right-to-left first-order carries
    RGn = np.zeros((nc + 1, d, dv)); rgd = np.zeros((nc + 1, d))
    RCn = np.zeros((nc + 1, d, dv)); rcd = np.zeros((nc + 1, d))
    for c in reversed(range(nc)):
        s, L = chunks[c]
        tau = np.arange(L)
        Qc = Q[s:s + L]
        w2, w1 = g ** (2.0 * tau), g ** tau
        RGn[c] = Qc.T @ (w2[:, None] * Gn[s:s + L]) + g ** (2.0 * L) * RGn[c + 1]
        rgd[c] = Qc.T @ (w2 * gd[s:s + L]) + g ** (2.0 * L) * rgd[c + 1]
        RCn[c] = Qc.T @ (w1[:, None] * Gn[s:s + L]) + g ** float(L) * RCn[c + 1]
        rcd[c] = Qc.T @ (w1 * gd[s:s + L]) + g ** float(L) * rcd[c + 1]
    # W per chunk, then the right-to-left T carry
    Ws = [None] * nc
    T = np.zeros((nc + 1, d, d))
    for c in reversed(range(nc)):
        s, L = chunks[c]
        tau = np.arange(L)
        Qc, Vc = Q[s:s + L], V[s:s + L]
        eh = g ** (L - tau.astype(float))
        diff = tau[:, None] - tau[None, :]
        Dg = np.where(diff >= 0, g ** np.maximum(diff, 0).astype(float), 0.0)
        Gam = Gn[s:s + L] @ Vc.T + gd[s:s + L][:, None]
        W = (Gam * Dg * Dg).T @ Qc + (eh * eh)[:, None] * (Vc @ RGn[c + 1].T + rgd[c + 1][None, :])
        Ws[c] = W
        w1 = g ** tau.astype(float)
        T[c] = W.T @ (w1[:, None] * Qc) + Qc.T @ (w1[:, None] * W) + g ** float(L) * T[c + 1]
    dQ = np.zeros_like(Q); dK = np.zeros_like(K); dV = np.zeros_like(V)
    for c, (s, L) in enumerate(chunks):
        S0, C0, m0, X0, y0 = carry[c]
        U, W = Us[c], Ws[c]
        Qc, Kc, Vc = Q[s:s + L], K[s:s + L], V[s:s + L]
        Gc, gdc = Gn[s:s + L], gd[s:s + L]
        tau = np.arange(L)
        e, eh = g ** (tau + 1.0), g ** (L - tau.astype(float))
        diff = tau[:, None] - tau[None, :]
        Dg = np.where(diff >= 0, g ** np.maximum(diff, 0).astype(float), 0.0)
        Gam = Gc @ Vc.T + gdc[:, None]
        G1, G2 = Gam * Dg, Gam * Dg * Dg
        dq = (e * e)[:, None] * (Gc @ X0.T + gdc[:, None] * y0[None, :]) + G2 @ U \
            + e[:, None] * (W @ S0) + ((W @ Kc.T) * Dg) @ Kc
        if lam:
            dq += lam * (e[:, None] * (Gc @ C0.T + gdc[:, None] * m0[None, :]) + G1 @ Qc + G1.T @ Qc
                         + eh[:, None] * (Vc @ RCn[c + 1].T + rcd[c + 1][None, :]))
        Mu = Dg.T
        dk = ((Kc @ Qc.T) * Mu) @ W + ((Kc @ W.T) * Mu) @ Qc + eh[:, None] * (Kc @ T[c + 1])
        P = (Qc @ U.T) * Dg * Dg + lam * (Qc @ Qc.T) * Dg
        dvv = P.T @ Gc + (eh * eh)[:, None] * (U @ RGn[c + 1]) + lam * eh[:, None] * (Qc @ RCn[c + 1])
        dQ[s:s + L], dK[s:s + L], dV[s:s + L] = dq, dk, dvv
    return dQ, dK, dV


@pytest.mark.parametrize("n,w", [(1, 4), (7, 4), (16, 4), (29, 8), (40, 16)])
@pytest.mark.parametrize("g,lam,norm", [(1.0, 0.0, False), (0.9, 0.0, False), (0.85, 0.3, False),
                                        (0.9, 0.3, True), (1.0, 0.0, True)])
def test_chunked_backward_matches_oracle(n, w, g, lam, norm):
    r = np.random.default_rng(100 + n + w)
    d, dv = 5, 3
    Q, K, V, Go = (r.standard_normal((n, x)) * 0.5 for x in (d, d, dv, dv))
    if norm:
        Q, K = np.abs(Q) + 0.3, np.abs(K) + 0.3
    ref = ob.backward(Q[None, None], K[None, None], V[None, None], Go[None, None], [g], lam, norm)
    got = chunked_backward(Q, K, V, Go, g, lam, norm, w)
    for x, y in zip(got, ref):
        y = y[0, 0]
        assert np.abs(x - y).max() <= 1e-11 * max(1.0, np.abs(y).max())


# ------------------------------------------------------------------------------
# The plain-numerator gradient as masked first-order maps, the form the
# one-launch backward runs: with LA(A, B, C; r)_t = sum_{s<=t} r^(t-s) (a_t.b_s) c_s
# and LA^rev the same over s >= t with r^(s-t),
#   U = LA(Q, K, K; g),  W = LA^rev(V, dO, Q; g^2)
#   dq = LA(dO, V, U; g^2) + LA(W, K, K; g)
#   dk = LA^rev(K, Q, W; g) + LA^rev(K, W, Q; g)
#   dv = LA^rev(U, Q, dO; g^2)
# (each a rearrangement of the sums above for lam = 0 and dnum = dout).

def _la(a, b, c, r):
    n = a.shape[0]
    t = np.arange(n)
    D = np.where(t[:, None] >= t[None, :], float(r) ** np.clip(t[:, None] - t[None, :], 0, None), 0.0)
    return ((a @ b.T) * D) @ c


def _la_rev(a, b, c, r):
    return _la(a[::-1], b[::-1], c[::-1], r)[::-1]


@pytest.mark.parametrize("n,d,dv,g", [(37, 5, 4, 1.0), (50, 6, 6, 0.9), (23, 3, 7, 0.75)])
def test_plain_gradient_is_first_order_maps(n, d, dv, g):
    r = np.random.default_rng(n + d)
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    dout = r.standard_normal((n, dv))
    dq, dk, dvv = (np.asarray(x)[0, 0] for x in
                   ob.backward(q[None, None], k[None, None], v[None, None], dout[None, None], gamma=[g])[:3])
    U = _la(q, k, k, g)
    Wm = _la_rev(v, dout, q, g * g)
    rel = lambda a, b: np.max(np.abs(a - b)) / np.max(np.abs(b))  # noqa: E731
    assert rel(_la(dout, v, U, g * g) + _la(Wm, k, k, g), dq) < 1e-12
    assert rel(_la_rev(k, q, Wm, g) + _la_rev(k, Wm, q, g), dk) < 1e-12
    assert rel(_la_rev(U, q, dout, g * g), dvv) < 1e-12


def _la_c(a, b, c, r, M):
    """LA with a carry M at position -1: y_t = M_t^T a_t, M_t = r M_{t-1} + b_t c_t^T.
    Returns y and the carry after the last token."""
    y = np.zeros((a.shape[0], c.shape[1]))
    for t in range(a.shape[0]):
        M = r * M + np.outer(b[t], c[t])
        y[t] = M.T @ a[t]
    return y, M


def _la_rev_c(a, b, c, r, M):
    y, M = _la_c(a[::-1], b[::-1], c[::-1], r, M)
    return y[::-1], M


class _St:
    def __init__(self, **kw):
        self.__dict__.update(kw)


@pytest.mark.parametrize("n,d,g", [(17, 4, 1.0), (23, 5, 0.9), (9, 3, 0.75), (1, 4, 0.8)])
def test_state_gradients_are_first_order_maps_with_carries(n, d, g):
    """With an initial state (S not symmetric) and a gradient flowing into the
    final state: the maps above from carries at position -1 (their own
    direction), two decayed terms, and the initial state's gradient from the
    final carries of W and of dk's map (the identity written out in
    bwd_la64.hip), against the oracle's autograd gradients."""
    r = np.random.default_rng(100 + n + d)
    q, k, v, dout = (0.5 * r.standard_normal((n, d)) for _ in range(4))
    S0, C0, G0 = (r.standard_normal((d, d)) for _ in range(3))
    m0, h0 = r.standard_normal(d), r.standard_normal(d)
    dS, dC, dG = (r.standard_normal((d, d)) for _ in range(3))
    dm, dh = r.standard_normal(d), r.standard_normal(d)
    init = _St(S=S0[None], C=C0[None], m=m0[None], G=G0[None], h=h0[None])
    dfin = _St(S=dS[None], C=dC[None], m=dm[None], G=dG[None], h=dh[None])
    dq_r, dk_r, dv_r, di = ob.backward(q[None, None], k[None, None], v[None, None], dout[None, None], gamma=[g],
                                       init=init, init_grad=True, dfinal=dfin)
    g2, p = g * g, np.arange(n)[::-1].astype(float)  # p = n - 1 - t
    U, Sn = _la_c(q, k, k, g, S0)
    Cn = g ** n * C0 + sum(g ** (n - 1 - s) * np.outer(q[s], v[s]) for s in range(n))
    mn = g ** n * m0 + sum(g ** (n - 1 - s) * q[s] for s in range(n))
    DS, DC, Dm = dS + Cn @ dG.T + np.outer(mn, dh), dC + Sn @ dG, dm + Sn @ dh
    dX, dY, X0 = -dG, -dh, S0.T @ C0 - G0
    W, MW = _la_rev_c(v, dout, q, g2, dX.T / g2)
    W = W + (g2 ** p)[:, None] * dY[None]
    dq = (_la_c(W, k, k, g, S0.T)[0] + _la_c(dout, v, U, g2, X0.T)[0]
          + (g ** p)[:, None] * (v @ DC.T + Dm[None]))
    y1, MK = _la_rev_c(k, q, W, g, DS / g)
    y2, MK2 = _la_rev_c(k, W, q, g, DS.T / g)
    assert np.allclose(MK2, MK.T)  # one symmetric carry serves both maps of dk
    dvv = _la_rev_c(U, q, dout, g2, dX / g2)[0] + (g ** p)[:, None] * (q @ DC)
    dX0, dY0 = g2 * MW.T, g2 ** n * dY
    parts = {"S": g * MK + C0 @ dX0.T + np.outer(m0, dY0), "C": g ** n * DC + S0 @ dX0,
             "m": g ** n * Dm + S0 @ dY0, "G": -dX0, "h": -dY0}
    rel = lambda a, b: np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)  # noqa: E731
    assert rel(dq, dq_r[0, 0]) < 1e-12
    assert rel(y1 + y2, dk_r[0, 0]) < 1e-12
    assert rel(dvv, dv_r[0, 0]) < 1e-12
    for name, x in parts.items():
        assert rel(x, np.asarray(di[name])[0]) < 1e-12, name

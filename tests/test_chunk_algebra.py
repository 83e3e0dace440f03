"""The chunked evaluation order used by the HIP kernels, written out in numpy
fp64 and checked against the serial-recurrence oracle.  This pins the
algebra of the GPU design on the CPU (it shares no code with the HIP path).

Per chunk of L <= w tokens (local indices tau, sigma), carry-in at the chunk
start (S0, C0, m0) and the "corrected" carries X0 = S0 C0 - G0, y0 = S0 m0 - h0:

  e_tau = g^(tau+1), f_sigma = g^(L-1-sigma), rho = g^L
  A   = (Q K^T) o D_g o L            (D_g[t,s] = g^(t-s), L = lower incl. diag)
  U   = diag(e) Q S0 + A K           (row sigma = S_{s+sigma} q_sigma)
  P   = (Q U^T) o D_{g^2} o L
  R   = (Q Q^T) o D_g o L            (ridge only)
  num = P V + diag(e^2) Q X0 + lam (diag(e) Q C0 + R V)
  den = P 1 + diag(e^2) Q y0 + lam (diag(e) Q m0 + R 1)
  S0 <- rho S0 + K^T diag(f) K,  C0 <- rho C0 + Q^T diag(f) V,  m0 <- rho m0 + Q^T f
  X0 <- rho^2 X0 + U^T diag(f^2) V,  y0 <- rho^2 y0 + U^T f^2
and at the end G = S C - X, h = S m - y.  The X recurrence follows from the
streaming identities: S_t C_t - G_t = g^2 (S_{t-1} C_{t-1} - G_{t-1}) + S_t q_t v_t^T.
"""
import math

import numpy as np
import pytest


def chunked(Q, K, V, g, lam, w, init=None):
    n, d = Q.shape
    dv = V.shape[1]
    if init is None:
        S0 = np.zeros((d, d)); C0 = np.zeros((d, dv)); m0 = np.zeros(d)
        X0 = np.zeros((d, dv)); y0 = np.zeros(d)
    else:
        S0, C0, m0, G0, h0 = (np.array(x, dtype=np.float64) for x in init)
        X0 = S0 @ C0 - G0
        y0 = S0 @ m0 - h0
    num = np.zeros((n, dv)); den = np.zeros(n)
    for s in range(0, n, w):
        Qc, Kc, Vc = Q[s:s + w], K[s:s + w], V[s:s + w]
        L = Qc.shape[0]
        tau = np.arange(L)
        e = g ** (tau + 1.0)
        f = g ** (L - 1.0 - tau)
        rho = g ** float(L)
        diff = tau[:, None] - tau[None, :]
        low = diff >= 0
        Dg = np.where(low, g ** np.maximum(diff, 0).astype(float), 0.0)
        Dg2 = Dg * Dg
        A = (Qc @ Kc.T) * Dg
        U = e[:, None] * (Qc @ S0) + A @ Kc
        P = (Qc @ U.T) * Dg2
        R = (Qc @ Qc.T) * Dg
        num[s:s + L] = P @ Vc + (e * e)[:, None] * (Qc @ X0) + lam * (e[:, None] * (Qc @ C0) + R @ Vc)
        den[s:s + L] = P.sum(1) + e * e * (Qc @ y0) + lam * (e * (Qc @ m0) + R.sum(1))
        S0 = rho * S0 + Kc.T @ (f[:, None] * Kc)
        C0 = rho * C0 + Qc.T @ (f[:, None] * Vc)
        m0 = rho * m0 + Qc.T @ f
        X0 = rho * rho * X0 + U.T @ ((f * f)[:, None] * Vc)
        y0 = rho * rho * y0 + U.T @ (f * f)
    return num, den, (S0, C0, m0, S0 @ C0 - X0, S0 @ m0 - y0)


@pytest.mark.parametrize("n,d,dv,w,g,lam", [
    (64, 8, 8, 16, 1.0, 0.0),
    (77, 8, 4, 16, 0.97, 0.1),     # ragged tail
    (50, 4, 6, 64, 0.9, 0.0),      # single partial chunk
    (96, 16, 16, 32, 0.999, 1.0),
])
def test_chunked_equals_serial(oracle_mod, n, d, dv, w, g, lam):
    r = np.random.default_rng(n + d + w)
    s = 1 / math.sqrt(d)
    q = r.standard_normal((1, 1, n, d)) * s
    k = r.standard_normal((1, 1, n, d)) * s
    v = r.standard_normal((1, 1, n, dv)) * s
    out, den, st = oracle_mod.forward(q, k, v, gamma=[g], lam=lam)
    num_c, den_c, fin = chunked(q[0, 0], k[0, 0], v[0, 0], g, lam, w)
    assert np.max(np.abs(num_c - out[0, 0])) <= 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(den_c - den[0, 0])) <= 1e-12 * np.max(np.abs(den))
    for a, b in zip(fin, (st.S[0], st.C[0], st.m[0], st.G[0], st.h[0])):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(np.max(np.abs(b)), 1e-300)


def test_chunked_from_init_state(oracle_mod):
    r = np.random.default_rng(3)
    n, d, dv, w, g, lam = 70, 8, 5, 16, 0.95, 0.2
    q = r.standard_normal((1, 1, n, d)) * 0.3
    k = r.standard_normal((1, 1, n, d)) * 0.3
    v = r.standard_normal((1, 1, n, dv)) * 0.3
    _, _, st = oracle_mod.forward(q[:, :, :30], k[:, :, :30], v[:, :, :30], gamma=[g], lam=lam)
    out, den, fin = oracle_mod.forward(q[:, :, 30:], k[:, :, 30:], v[:, :, 30:], gamma=[g], lam=lam,
                                       init=st)
    init = (st.S[0], st.C[0], st.m[0], st.G[0], st.h[0])
    num_c, den_c, f = chunked(q[0, 0, 30:], k[0, 0, 30:], v[0, 0, 30:], g, lam, w, init)
    assert np.max(np.abs(num_c - out[0, 0])) <= 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(den_c - den[0, 0])) <= 1e-12 * np.max(np.abs(den))
    assert np.max(np.abs(f[3] - fin.G[0])) <= 1e-12 * np.max(np.abs(fin.G))

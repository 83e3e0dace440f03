"""Brute-force evaluation of the masked second-order HLA definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here uses
prefix summaries or recurrences: every quantity is the explicit sum over
token indices that the pages' identities stand for, so it pins the serial
recurrence in ``hla_oracle.c`` from outside.

Definition (Higher-order Linear Attention; symmetric second-order operator
A A^T V with A = Q K^T, gist.science page "Asymmetrische ..." and "Dritte
Ordnung" items; causal mask keeping positions on and before the current
token, paperlayer.ai page sec. 2.1 and 3.1, applied to both the inner index i
and the outer index j; decay as an attenuation factor per token of distance,
paperlayer.ai page sec. 4.3; ridge lambda*I added to S at read-out,
paperlayer.ai page sec. 5.1):

  num_t = sum_{j<=t} sum_{i<=j} g^(2t-i-j) (q_t.k_i)(k_i.q_j) v_j
          + lambda * sum_{j<=t} g^(t-j) (q_t.q_j) v_j
  den_t = the same with every v_j replaced by 1

Cost O(n^3 d); use only on tiny inputs.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Sequence

import numpy as np


def _pow(g, e):
    # 0**0 == 1 for the g = 0 limit, in both Fraction and float
    return g ** e if e != 0 else (Fraction(1) if isinstance(g, Fraction) else 1.0)


def masked_exact(q: Sequence[Sequence], k: Sequence[Sequence], v: Sequence[Sequence],
                 gamma=Fraction(1), lam=Fraction(0)):
    """Exact-rational definition for one head.  q, k: n x d; v: n x dv lists of
    Fractions (or ints).  Returns (num: n x dv, den: n) as Fractions."""
    n = len(q)
    d, dv = len(q[0]), len(v[0])
    g, lam = Fraction(gamma), Fraction(lam)

    def dot(a, b):
        return sum((Fraction(x) * Fraction(y) for x, y in zip(a, b)), Fraction(0))

    num, den = [], []
    for t in range(n):
        row = [Fraction(0)] * dv
        dn = Fraction(0)
        for j in range(t + 1):
            w = Fraction(0)
            for i in range(j + 1):
                w += _pow(g, 2 * t - i - j) * dot(q[t], k[i]) * dot(k[i], q[j])
            w += lam * _pow(g, t - j) * dot(q[t], q[j])
            for c in range(dv):
                row[c] += w * Fraction(v[j][c])
            dn += w
        num.append(row)
        den.append(dn)
    return num, den


def masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, gamma: float = 1.0, lam: float = 0.0):
    """fp64 definition for one head: explicit loops over t and j, the inner
    sum over i <= j vectorised.  q, k: [n,d]; v: [n,dv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    num = np.zeros((n, v.shape[1]))
    den = np.zeros(n)
    for t in range(n):
        qk_t = k[: t + 1] @ q[t]                     # (q_t . k_i), i <= t
        for j in range(t + 1):
            i = np.arange(j + 1)
            kq_j = k[: j + 1] @ q[j]                 # (k_i . q_j), i <= j
            wts = np.array([_pow(gamma, 2 * t - ii - j) for ii in i])
            w = float(np.sum(wts * qk_t[: j + 1] * kq_j))
            w += lam * _pow(gamma, t - j) * float(q[t] @ q[j])
            num[t] += w * v[j]
            den[t] += w
    return num, den


def prefix_moments(q, k, v, t: int, gamma: float = 1.0):
    """Direct decayed sums S_t, C_t, m_t (paperlayer.ai page sec. 3; gist.science
    page "Zustandserhaltung"), no recurrence."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    w = np.array([_pow(gamma, t - i) for i in range(t + 1)])
    S = (k[: t + 1] * w[:, None]).T @ k[: t + 1]
    C = (q[: t + 1] * w[:, None]).T @ v[: t + 1]
    m = (q[: t + 1] * w[:, None]).sum(axis=0)
    return S, C, m


def future_pairs(q, k, v, t: int, gamma: float = 1.0):
    """Direct sums of the pairs with the key index after the query index,
    G_t = sum_{j < i <= t} g^(2t-i-j) k_i (k_i.q_j) v_j^T and
    h_t = sum_{j < i <= t} g^(2t-i-j) k_i (k_i.q_j): the "future terms" that the
    cross summaries remove from the naive product S_t C_t (gist.science page,
    "Strenge Kausalitaet")."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d, dv = q.shape[1], v.shape[1]
    G = np.zeros((d, dv))
    h = np.zeros(d)
    for i in range(t + 1):
        for j in range(i):
            c = _pow(gamma, 2 * t - i - j) * float(k[i] @ q[j])
            G += c * np.outer(k[i], v[j])
            h += c * k[i]
    return G, h


# ---------------------------------------------------------------------------
# the asymmetric variant (AHLA) and third order, by their definitions
#
# AHLA (paperlayer.ai page sec. 6 and 6.1; gist.science page "Methodik" item
# 2): the left-cascaded product Q (K^T Q)(K^T V) with the causal mask on
# both factors, decay g per token of distance:
#   num_t = sum_{j<=t} sum_{i<=j} g^(t-i) (q_t.k_j)(q_j.k_i) v_i
# Third order (paperlayer.ai page sec. 7 and 7.1; gist.science page
# "Methodik" item 3): A A^T A V with A = Q K^T, masked at every factor, no
# decay:
#   num_t = sum_{j<=t} sum_{i<=j} sum_{l<=j} (q_t.k_i)(k_i.q_j)(q_j.k_l) v_l
# den_t: the same with every value equal to one.

def ahla_exact(q, k, v, gamma=Fraction(1)):
    """Exact-rational AHLA definition for one head (lists of Fractions/ints)."""
    n, dv = len(q), len(v[0])
    g = Fraction(gamma)

    def dot(a, b):
        return sum((Fraction(x) * Fraction(y) for x, y in zip(a, b)), Fraction(0))

    num, den = [], []
    for t in range(n):
        row = [Fraction(0)] * dv
        dn = Fraction(0)
        for j in range(t + 1):
            for i in range(j + 1):
                w = _pow(g, t - i) * dot(q[t], k[j]) * dot(q[j], k[i])
                for c in range(dv):
                    row[c] += w * Fraction(v[i][c])
                dn += w
        num.append(row)
        den.append(dn)
    return num, den


def ahla(q, k, v, gamma: float = 1.0):
    """fp64 AHLA definition for one head: explicit loops over t, j, i."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    num = np.zeros((n, v.shape[1]))
    den = np.zeros(n)
    for t in range(n):
        for j in range(t + 1):
            a = float(q[t] @ k[j])
            for i in range(j + 1):
                w = _pow(gamma, t - i) * a * float(q[j] @ k[i])
                num[t] += w * v[i]
                den[t] += w
    return num, den


def third_exact(q, k, v):
    """Exact-rational third-order definition for one head."""
    n, dv = len(q), len(v[0])

    def dot(a, b):
        return sum((Fraction(x) * Fraction(y) for x, y in zip(a, b)), Fraction(0))

    num, den = [], []
    for t in range(n):
        row = [Fraction(0)] * dv
        dn = Fraction(0)
        for j in range(t + 1):
            for i in range(j + 1):
                a = dot(q[t], k[i]) * dot(k[i], q[j])
                for l in range(j + 1):
                    w = a * dot(q[j], k[l])
                    for c in range(dv):
                        row[c] += w * Fraction(v[l][c])
                    dn += w
        num.append(row)
        den.append(dn)
    return num, den


def third(q, k, v):
    """fp64 third-order definition for one head: explicit loops over t, j, i, l."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    num = np.zeros((n, v.shape[1]))
    den = np.zeros(n)
    for t in range(n):
        for j in range(t + 1):
            for i in range(j + 1):
                a = float(q[t] @ k[i]) * float(k[i] @ q[j])
                for l in range(j + 1):
                    w = a * float(q[j] @ k[l])
                    num[t] += w * v[l]
                    den[t] += w
    return num, den

"""Pins of the AHLA and third-order oracles (oracle/higher.py,
oracle/higher_oracle.c) against what the definitions and the mathematics
fix, none of which shares the oracle's recurrence:

* the brute-force definitions (explicit sums over token indices, exact
  rationals and fp64; oracle/brute.py);
* the matrix forms: AHLA num = (A o D_g o L)((A o D_g o L) V) and third order
  num = ((A_L A_L^T) o L)(A_L V), A = Q K^T, A_L = A o L (numpy products);
* hand-derived worked examples (d = 1, dyadic values, exact in fp64);
* closed forms: all-ones inputs, one token, the g -> 0 limit;
* third order equal to the second-order oracle run on the first-order causal
  linear-attention values v'_j = sum_{l<=j} (q_j . k_l) v_l;
* composition: scan-composed segment summaries equal the serial state,
  associativity and identity; split-point continuation; decode = next row;
  strict causality.
"""
import numpy as np
import pytest
from fractions import Fraction

from oracle import brute, higher


def rng_qkv(seed, n, d, dv, B=1, H=1):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, n, d)) / np.sqrt(d), r.standard_normal((B, H, n, d)) / np.sqrt(d),
            r.standard_normal((B, H, n, dv)) / np.sqrt(d))


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def masks(n, g):
    t = np.arange(n)
    L = (t[:, None] >= t[None, :]).astype(np.float64)
    D = np.where(L > 0, float(g) ** np.clip(t[:, None] - t[None, :], 0, None), 0.0)
    return L, D


# --------------------------------------------------------------------- AHLA

@pytest.mark.parametrize("g", [1.0, 0.9, 0.5])
def test_ahla_matches_brute_force(g):
    q, k, v = rng_qkv(1, 13, 3, 4)
    out, den, _ = higher.ahla_forward(q, k, v, gamma=[g])
    nr, dr = brute.ahla(q[0, 0], k[0, 0], v[0, 0], g)
    assert rel(out[0, 0], nr) < 1e-12 and rel(den[0, 0], dr) < 1e-12


@pytest.mark.parametrize("g", [1.0, 0.95])
def test_ahla_matrix_form(g):
    q, k, v = rng_qkv(2, 40, 8, 5)
    Q, K, V = q[0, 0], k[0, 0], v[0, 0]
    _, D = masks(40, g)
    A = (Q @ K.T) * D
    out, den, _ = higher.ahla_forward(q, k, v, gamma=[g])
    assert rel(out[0, 0], A @ (A @ V)) < 1e-12
    assert rel(den[0, 0], A @ (A @ np.ones(40))) < 1e-12


def test_ahla_worked_example_by_hand():
    """d = dv = 1, q = (1, 2, -1), k = (1, 1, 2), v = (1, -1, 3), g = 1.
    num_t = sum_{j<=t} (q_t k_j) sum_{i<=j} (q_j k_i) v_i:
      t=0: (1)(1)(1) = 1
      t=1: (2)(1*1*1) + (2)(2*1*1 + 2*1*(-1)) = 2 + 0 = 2
      t=2: (-1)(1) + (-1)(0) + (-2)(-1 + 1 - 6) = -1 + 0 + 12 = 11
    den_t (every v = 1): 1; 2 + 2*(2 + 2) = 10; -1 - 4 + (-2)(-1 - 1 - 2) = 3."""
    q = np.array([1.0, 2.0, -1.0]).reshape(1, 1, 3, 1)
    k = np.array([1.0, 1.0, 2.0]).reshape(1, 1, 3, 1)
    v = np.array([1.0, -1.0, 3.0]).reshape(1, 1, 3, 1)
    out, den, st = higher.ahla_forward(q, k, v)
    assert out[0, 0, :, 0].tolist() == [1.0, 2.0, 11.0]
    assert den[0, 0].tolist() == [1.0, 10.0, 3.0]
    # and the exact-rational definition agrees, also with decay 1/2
    for g in (Fraction(1), Fraction(1, 2)):
        ne, de = brute.ahla_exact([[1], [2], [-1]], [[1], [1], [2]], [[1], [-1], [3]], g)
        o, dn, _ = higher.ahla_forward(q, k, v, gamma=[float(g)])
        assert [float(x[0]) for x in ne] == o[0, 0, :, 0].tolist()
        assert [float(x) for x in de] == dn[0, 0].tolist()
    # final summaries: P = sum k v = 1 - 1 + 6, m = 4, R = sum k q = 1 + 2 - 2
    assert st.P[0, 0, 0] == 6.0 and st.m[0, 0] == 4.0 and st.R[0, 0, 0] == 1.0


@pytest.mark.parametrize("g", [1.0, 0.8])
def test_ahla_all_ones(g):
    d, dv, n = 3, 2, 7
    ones = np.ones((1, 1, n, d))
    out, den, _ = higher.ahla_forward(ones, ones, np.ones((1, 1, n, dv)), gamma=[g])
    # num_t = d^2 sum_{j<=t} sum_{i<=j} g^(t-i) = d^2 sum_{i<=t} (t-i+1) g^(t-i)
    want = [d * d * sum((t - i + 1) * g ** (t - i) for i in range(t + 1)) for t in range(n)]
    assert np.allclose(out[0, 0, :, 0], want, rtol=1e-13) and np.allclose(den[0, 0], want, rtol=1e-13)
    if g == 1.0:
        assert out[0, 0, :, 0].tolist() == [d * d * (t + 1) * (t + 2) / 2 for t in range(n)]


def test_ahla_one_token_and_zero_decay():
    q, k, v = rng_qkv(3, 9, 4, 3)
    out, _, _ = higher.ahla_forward(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    qk = float(q[0, 0, 0] @ k[0, 0, 0])
    assert rel(out[0, 0, 0], qk * qk * v[0, 0, 0]) < 1e-14
    out0, _, _ = higher.ahla_forward(q, k, v, gamma=[0.0])  # only i = j = t survives
    qkt = np.einsum("td,td->t", q[0, 0], k[0, 0])
    assert rel(out0[0, 0], (qkt ** 2)[:, None] * v[0, 0]) < 1e-14


def test_ahla_is_not_the_symmetric_operator():
    import oracle
    q, k, v = rng_qkv(4, 20, 4, 4)
    a, _, _ = higher.ahla_forward(q, k, v)
    s, _, _ = oracle.forward(q, k, v)
    assert rel(a, s) > 0.1


@pytest.mark.parametrize("g", [1.0, 0.93])
def test_ahla_scan_composition_equals_serial(g):
    q, k, v = rng_qkv(5, 50, 4, 3, H=2)
    cuts = [0, 11, 30, 50]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        _, _, s = higher.ahla_forward(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], gamma=[g, g])
        parts.append(s)
    _, _, whole = higher.ahla_forward(q, k, v, gamma=[g, g])
    left = higher.ahla_compose(higher.ahla_compose(parts[0], parts[1]), parts[2])
    right = higher.ahla_compose(parts[0], higher.ahla_compose(parts[1], parts[2]))
    for name in ("P", "m", "E", "n", "R", "rho"):
        assert rel(getattr(left, name), getattr(whole, name)) < 1e-12, name
        assert rel(getattr(right, name), getattr(whole, name)) < 1e-12, name
    ident = higher.AhlaState.zeros(2, 4, 3)
    c = higher.ahla_compose(ident, parts[1])
    for name in ("P", "m", "E", "n", "R", "rho"):
        assert np.array_equal(getattr(c, name), getattr(parts[1], name))


def test_ahla_continuation_decode_and_causality():
    q, k, v = rng_qkv(6, 31, 4, 3, B=2, H=2)
    g = [0.9, 1.0]
    out, den, _ = higher.ahla_forward(q, k, v, gamma=g)
    o1, _, s1 = higher.ahla_forward(q[:, :, :17], k[:, :, :17], v[:, :, :17], gamma=g)
    o2, _, _ = higher.ahla_forward(q[:, :, 17:], k[:, :, 17:], v[:, :, 17:], gamma=g, init=s1)
    assert rel(np.concatenate([o1, o2], axis=2), out) < 1e-12
    _, _, s30 = higher.ahla_forward(q[:, :, :30], k[:, :, :30], v[:, :, :30], gamma=g)
    od, dd, _ = higher.ahla_decode(s30, q[:, :, 30], k[:, :, 30], v[:, :, 30], gamma=g)
    assert rel(od, out[:, :, 30]) < 1e-12 and rel(dd, den[:, :, 30]) < 1e-12
    q2 = q.copy()
    q2[:, :, 20:] += 1.0
    o3, _, _ = higher.ahla_forward(q2, k, v, gamma=g)
    assert np.array_equal(o3[:, :, :20], out[:, :, :20])


# -------------------------------------------------------------- third order

def test_third_matches_brute_force():
    q, k, v = rng_qkv(11, 9, 3, 2)
    out, den, _ = higher.third_forward(q, k, v)
    nr, dr = brute.third(q[0, 0], k[0, 0], v[0, 0])
    assert rel(out[0, 0], nr) < 1e-12 and rel(den[0, 0], dr) < 1e-12


def test_third_matrix_form():
    q, k, v = rng_qkv(12, 40, 8, 5)
    Q, K, V = q[0, 0], k[0, 0], v[0, 0]
    L, _ = masks(40, 1.0)
    AL = (Q @ K.T) * L
    out, den, _ = higher.third_forward(q, k, v)
    assert rel(out[0, 0], ((AL @ AL.T) * L) @ (AL @ V)) < 1e-12
    assert rel(den[0, 0], ((AL @ AL.T) * L) @ (AL @ np.ones(40))) < 1e-12


def test_third_is_second_order_on_linear_attention_values():
    """num3(Q, K, V) = num2(Q, K, V') with v'_j = sum_{l<=j} (q_j . k_l) v_l,
    by the second-order oracle (pinned on its own); den3 likewise with
    v'_j = q_j . sum_{l<=j} k_l."""
    import oracle
    q, k, v = rng_qkv(13, 33, 5, 4, H=2)
    vp = np.zeros_like(v)
    for h in range(2):
        Q, K, V = q[0, h], k[0, h], v[0, h]
        L, _ = masks(33, 1.0)
        vp[0, h] = ((Q @ K.T) * L) @ V
    vd = np.einsum("bhjd,bhjd->bhj", q, np.cumsum(k, axis=2))[..., None]
    out, den, _ = higher.third_forward(q, k, v)
    n2, _, _ = oracle.forward(q, k, vp)
    d2, _, _ = oracle.forward(q, k, vd)
    assert rel(out, n2) < 1e-12 and rel(den, d2[..., 0]) < 1e-12


def test_third_worked_example_by_hand():
    """d = dv = 1, q = (1, 2, -1), k = (1, 1, 2), v = (1, -1, 3).  First-order
    values v'_j = q_j sum_{l<=j} k_l v_l = (1, 2*0, -1*6) = (1, 0, -6), then
    num_t = sum_{j<=t} sum_{i<=j} (q_t k_i)(k_i q_j) v'_j:
      t=0: 1;  t=1: (2)(1)(1) + 0 = 2;  t=2: (-1)(1)(1) + 0 + (1 + 1 + 4)(-6) = -37.
    den: v'_j = q_j sum_{l<=j} k_l = (1, 4, -4):
      t=0: 1;  t=1: 2 + (4 + 4) 4 = 34;  t=2: -1 + (-2 - 2) 4 + 6 (-4) = -41."""
    q = np.array([1.0, 2.0, -1.0]).reshape(1, 1, 3, 1)
    k = np.array([1.0, 1.0, 2.0]).reshape(1, 1, 3, 1)
    v = np.array([1.0, -1.0, 3.0]).reshape(1, 1, 3, 1)
    out, den, _ = higher.third_forward(q, k, v)
    assert out[0, 0, :, 0].tolist() == [1.0, 2.0, -37.0]
    assert den[0, 0].tolist() == [1.0, 34.0, -41.0]
    ne, de = brute.third_exact([[1], [2], [-1]], [[1], [1], [2]], [[1], [-1], [3]])
    assert [float(x[0]) for x in ne] == [1.0, 2.0, -37.0] and [float(x) for x in de] == [1.0, 34.0, -41.0]


def test_third_all_ones_and_one_token():
    d, dv, n = 2, 3, 6
    ones = np.ones((1, 1, n, d))
    out, den, _ = higher.third_forward(ones, ones, np.ones((1, 1, n, dv)))
    want = [d ** 3 * (t + 1) * (t + 2) * (2 * t + 3) / 6 for t in range(n)]  # d^3 sum_{j<=t} (j+1)^2
    assert out[0, 0, :, 0].tolist() == want and den[0, 0].tolist() == want
    q, k, v = rng_qkv(14, 1, 4, 3)
    o1, _, _ = higher.third_forward(q, k, v)
    qk = float(q[0, 0, 0] @ k[0, 0, 0])
    assert rel(o1[0, 0, 0], qk ** 3 * v[0, 0, 0]) < 1e-14


def test_third_scan_composition_equals_serial():
    q, k, v = rng_qkv(15, 41, 4, 3, H=2)
    cuts = [0, 9, 25, 41]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        _, _, s = higher.third_forward(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b])
        parts.append(s)
    _, _, whole = higher.third_forward(q, k, v)
    left = higher.third_compose(higher.third_compose(parts[0], parts[1]), parts[2])
    right = higher.third_compose(parts[0], higher.third_compose(parts[1], parts[2]))
    names = ("S", "P", "m", "F", "Fd", "SQ", "M", "Nq", "Nd")
    for name in names:
        assert rel(getattr(left, name), getattr(whole, name)) < 1e-12, name
        assert rel(getattr(right, name), getattr(whole, name)) < 1e-12, name
    ident = higher.ThirdState.zeros(2, 4, 3)
    c = higher.third_compose(ident, parts[1])
    for name in names:
        assert np.array_equal(getattr(c, name), getattr(parts[1], name))


def test_third_continuation_decode_and_causality():
    q, k, v = rng_qkv(16, 27, 4, 3, B=2, H=2)
    out, den, _ = higher.third_forward(q, k, v)
    o1, _, s1 = higher.third_forward(q[:, :, :13], k[:, :, :13], v[:, :, :13])
    o2, _, _ = higher.third_forward(q[:, :, 13:], k[:, :, 13:], v[:, :, 13:], init=s1)
    assert rel(np.concatenate([o1, o2], axis=2), out) < 1e-12
    _, _, s26 = higher.third_forward(q[:, :, :26], k[:, :, :26], v[:, :, :26])
    od, dd, _ = higher.third_decode(s26, q[:, :, 26], k[:, :, 26], v[:, :, 26])
    assert rel(od, out[:, :, 26]) < 1e-12 and rel(dd, den[:, :, 26]) < 1e-12
    k2 = k.copy()
    k2[:, :, 15:] *= -2.0
    o3, _, _ = higher.third_forward(q, k2, v)
    assert np.array_equal(o3[:, :, :15], out[:, :, :15])

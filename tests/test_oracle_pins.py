"""Pins for the CPU oracle: the serial recurrence in oracle/hla_oracle.c is
checked against things other than itself -- exact worked examples, the
brute-force masked definition, closed forms, special cases that reduce to
textbook formulas, and the invariants the pages state (exact scan/serial
equivalence, associativity, strict causality, constant-size streaming state).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_d1.json")


def rng_qkv(seed, B, H, n, d, dv, scale=None):
    r = np.random.default_rng(seed)
    s = scale if scale is not None else 1.0 / math.sqrt(d)
    return (r.standard_normal((B, H, n, d)) * s, r.standard_normal((B, H, n, d)) * s,
            r.standard_normal((B, H, n, dv)) * s)


def rel_row(x, ref):
    x = np.asarray(x).reshape(-1, np.asarray(x).shape[-1])
    ref = np.asarray(ref).reshape(x.shape)
    return float(np.max(np.max(np.abs(x - ref), axis=1) / np.maximum(np.max(np.abs(ref), axis=1), 1e-300)))


def rel_all(x, ref):
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300))


# --------------------------------------------------------------------------
# exact worked examples (d = dv = 1)

def test_worked_example_by_hand():
    # gamma = 1, lambda = 0, q = (1,2,-1), k = (1,1,2), v = (1,-1,3):
    # num_t = q_t * sum_{j<=t} (sum_{i<=j} k_i^2) q_j v_j
    #   t=0: 1*(1*1*1) = 1
    #   t=1: 2*(1 + (1+1)*2*(-1)) = 2*(1-4) = -6
    #   t=2: -1*(1 - 4 + (1+1+4)*(-1)*3) = -1*(-21) = 21
    # den_t: the same with v = 1: 1, 2*(1+4) = 10, -1*(1+4-6) = 1
    with open(GOLDEN) as f:
        doc = json.load(f)
    c0 = doc["cases"][0]
    assert c0["gamma"] == "1/1" and c0["lambda"] == "0/1"
    assert [Fraction(r[0]) for r in c0["num"]] == [1, -6, 21]
    assert [Fraction(x) for x in c0["den"]] == [1, 10, 1]


def test_golden_matches_exact_brute_force():
    with open(GOLDEN) as f:
        doc = json.load(f)
    for case in doc["cases"]:
        num, den = brute.masked_exact(doc["q"], doc["k"], doc["v"],
                                      Fraction(case["gamma"]), Fraction(case["lambda"]))
        assert [[str(x) if x.denominator != 1 else f"{x.numerator}/1" for x in r] for r in num] == \
            [[str(Fraction(x)) if Fraction(x).denominator != 1 else f"{Fraction(x).numerator}/1"
              for x in r] for r in case["num"]]
        assert den == [Fraction(x) for x in case["den"]]


def test_oracle_worked_example_exact(oracle_mod):
    with open(GOLDEN) as f:
        doc = json.load(f)
    q = np.array(doc["q"], dtype=np.float64)[None, None]
    k = np.array(doc["k"], dtype=np.float64)[None, None]
    v = np.array(doc["v"], dtype=np.float64)[None, None]
    for case in doc["cases"]:
        g, lam = float(Fraction(case["gamma"])), float(Fraction(case["lambda"]))
        out, den, st = oracle_mod.forward(q, k, v, gamma=[g], lam=lam)
        assert out[0, 0, :, 0].tolist() == [float(Fraction(r[0])) for r in case["num"]]
        assert den[0, 0].tolist() == [float(Fraction(x)) for x in case["den"]]
        outn, _, _ = oracle_mod.forward(q, k, v, gamma=[g], lam=lam, normalize=True)
        assert outn[0, 0, :, 0].tolist() == [float(Fraction(r[0]) / Fraction(x))
                                            for r, x in zip(case["num"], case["den"])]
    # final state for gamma = 1: S = sum k^2 = 6, C = sum q v = -4, m = sum q = 2,
    # G = sum_{j<i} k_i^2 q_j v_j = 1*(1*1) + 4*(1*1 + 2*(-1)) = -3,
    # h = sum_{j<i} k_i^2 q_j = 1*1 + 4*(1+2) = 13
    _, _, st = oracle_mod.forward(q, k, v)
    assert (st.S.item(), st.C.item(), st.m.item(), st.G.item(), st.h.item(), st.rho.item()) == \
        (6.0, -4.0, 2.0, -3.0, 13.0, 1.0)


# --------------------------------------------------------------------------
# brute-force definition on small random inputs

@pytest.mark.parametrize("d,dv,n,g,lam", [
    (3, 5, 23, 1.0, 0.0),
    (4, 2, 37, 0.93, 0.3),
    (5, 5, 17, 0.5, 1.0),
    (2, 7, 29, 0.999, 0.0),
    (6, 3, 11, 0.0, 0.2),
])
def test_oracle_matches_brute_force(oracle_mod, d, dv, n, g, lam):
    q, k, v = rng_qkv(100 + d * 7 + dv, 1, 2, n, d, dv, scale=1.0)
    gam = [g, 0.75 * g + 0.25 if g > 0 else 0.0]
    out, den, _ = oracle_mod.forward(q, k, v, gamma=gam, lam=lam)
    for h in range(2):
        num_ref, den_ref = brute.masked(q[0, h], k[0, h], v[0, h], gam[h], lam)
        assert rel_all(out[0, h], num_ref) < 1e-12
        assert rel_all(den[0, h], den_ref) < 1e-12
    outn, _, _ = oracle_mod.forward(q, k, v, gamma=gam, lam=lam, normalize=True)
    np.testing.assert_allclose(outn, out / den[..., None], rtol=1e-14, atol=0)


# --------------------------------------------------------------------------
# closed forms and special cases

@pytest.mark.parametrize("d,dv", [(3, 3), (4, 2)])
def test_all_ones_closed_form(oracle_mod, d, dv):
    n = 40
    q = np.ones((1, 1, n, d)); k = np.ones((1, 1, n, d)); v = np.ones((1, 1, n, dv))
    out, den, _ = oracle_mod.forward(q, k, v)
    t = np.arange(n)
    expect = d * d * (t + 1) * (t + 2) / 2.0
    assert np.array_equal(out[0, 0], np.repeat(expect[:, None], dv, axis=1))
    assert np.array_equal(den[0, 0], expect)
    # with decay: num_t = d^2 * sum_{j<=t} sum_{i<=j} g^(2t-i-j)
    #           = d^2 * sum_{j<=t} g^(2(t-j)) * (1 - g^(j+1)) / (1 - g)
    g = 0.8
    out, _, _ = oracle_mod.forward(q, k, v, gamma=[g])
    ex = np.array([d * d * sum(g ** (2 * (tt - j)) * (1 - g ** (j + 1)) / (1 - g)
                               for j in range(tt + 1)) for tt in range(n)])
    assert rel_all(out[0, 0, :, 0], ex) < 1e-13


def test_single_token(oracle_mod):
    q, k, v = rng_qkv(5, 2, 3, 1, 6, 4)
    lam = 0.37
    out, den, _ = oracle_mod.forward(q, k, v, lam=lam)
    qk = np.einsum("bhnd,bhnd->bhn", q, k)[..., 0]
    qq = np.einsum("bhnd,bhnd->bhn", q, q)[..., 0]
    expect = (qk ** 2 + lam * qq)[..., None] * v[:, :, 0]
    assert rel_all(out[:, :, 0], expect) < 1e-14
    assert rel_all(den[:, :, 0], qk ** 2 + lam * qq) < 1e-14


def test_zero_decay_limit(oracle_mod):
    # g = 0: only j = i = t survives: num_t = ((q_t.k_t)^2 + lam |q_t|^2) v_t
    q, k, v = rng_qkv(6, 1, 2, 9, 5, 3)
    lam = 0.25
    out, den, _ = oracle_mod.forward(q, k, v, gamma=[0.0, 0.0], lam=lam)
    qk = np.einsum("bhnd,bhnd->bhn", q, k)
    qq = np.einsum("bhnd,bhnd->bhn", q, q)
    expect = (qk ** 2 + lam * qq)[..., None] * v
    assert rel_all(out, expect) < 1e-14


def test_ridge_term_is_first_order_linear_attention(oracle_mod):
    # num(lam) - num(0) = lam * sum_{j<=t} g^(t-j) (q_t.q_j) v_j :
    # causal first-order linear attention with keys = queries, written directly
    q, k, v = rng_qkv(7, 1, 1, 31, 4, 6, scale=1.0)
    g, lam = 0.9, 0.7
    o1, d1, _ = oracle_mod.forward(q, k, v, gamma=[g], lam=lam)
    o0, d0, _ = oracle_mod.forward(q, k, v, gamma=[g], lam=0.0)
    Q, V = q[0, 0], v[0, 0]
    n = Q.shape[0]
    lin = np.zeros_like(V); lind = np.zeros(n)
    for t in range(n):
        for j in range(t + 1):
            w = g ** (t - j) * float(Q[t] @ Q[j])
            lin[t] += w * V[j]; lind[t] += w
    assert rel_all(o1[0, 0] - o0[0, 0], lam * lin) < 1e-11
    assert rel_all(d1[0, 0] - d0[0, 0], lam * lind) < 1e-11


def test_den_is_num_with_unit_values(oracle_mod):
    q, k, v = rng_qkv(8, 2, 2, 20, 5, 3)
    ones = np.ones(v.shape[:-1] + (1,))
    out, den, _ = oracle_mod.forward(q, k, v, gamma=[0.95, 0.8], lam=0.1)
    out1, _, _ = oracle_mod.forward(q, k, ones, gamma=[0.95, 0.8], lam=0.1)
    assert rel_all(out1[..., 0], den) < 1e-14


# --------------------------------------------------------------------------
# cross summaries: the unmasked closed form and the "future pairs"

@pytest.mark.parametrize("g", [1.0, 0.85])
def test_cross_summaries_are_future_pairs(oracle_mod, g):
    d, dv, n = 4, 3, 14
    q, k, v = rng_qkv(9, 1, 1, n, d, dv, scale=1.0)
    Q, K, V = q[0, 0], k[0, 0], v[0, 0]
    lam = 0.3
    out, den, _ = oracle_mod.forward(q, k, v, gamma=[g], lam=lam)
    for t in range(n):
        _, _, st = oracle_mod.forward(q[:, :, : t + 1], k[:, :, : t + 1], v[:, :, : t + 1],
                                      gamma=[g], lam=lam)
        S, C, m = brute.prefix_moments(Q, K, V, t, g)
        G, h = brute.future_pairs(Q, K, V, t, g)
        assert rel_all(st.S[0], S) < 1e-13 and rel_all(st.C[0], C) < 1e-13
        assert rel_all(st.m[0], m) < 1e-13
        assert rel_all(st.G[0], G) < 1e-12 and rel_all(st.h[0], h) < 1e-12
        assert abs(st.rho[0] - g ** (t + 1)) < 1e-15
        # unmasked closed form: num_t + q_t^T G_t - lam q_t^T C_t = q_t^T S_t C_t
        unmasked = Q[t] @ S @ C
        lhs = out[0, 0, t] + Q[t] @ G - lam * (Q[t] @ C)
        assert rel_all(lhs, unmasked) < 1e-11
        lhs_d = den[0, 0, t] + Q[t] @ h - lam * (Q[t] @ m)
        assert abs(lhs_d - Q[t] @ S @ m) <= 1e-11 * max(1.0, abs(Q[t] @ S @ m))


# --------------------------------------------------------------------------
# state algebra: exact scan == serial, associativity, identity

def _seg_state(oracle_mod, q, k, v, a, b, gam):
    _, _, st = oracle_mod.forward(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], gamma=gam)
    return st


def _close_state(x, y, tol):
    for name in ("S", "C", "m", "G", "h", "rho"):
        A, Bm = getattr(x, name), getattr(y, name)
        assert rel_all(A, Bm) <= tol, name


@pytest.mark.parametrize("gam", [[1.0, 1.0], [0.9, 0.97]])
def test_compose_of_segments_equals_serial(oracle_mod, gam):
    d, dv, n = 5, 4, 45
    q, k, v = rng_qkv(10, 1, 2, n, d, dv)
    full = _seg_state(oracle_mod, q, k, v, 0, n, gam)
    # chunked scan with a ragged tail: chunks of 8 over 45 tokens
    bounds = list(range(0, n, 8)) + [n]
    acc = None
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg = _seg_state(oracle_mod, q, k, v, a, b, gam)
        acc = seg if acc is None else oracle_mod.compose(acc, seg)
        pre = _seg_state(oracle_mod, q, k, v, 0, b, gam)
        _close_state(acc, pre, 1e-12)
    _close_state(acc, full, 1e-12)


def test_compose_associative_and_identity(oracle_mod):
    from hla_inputs import random_state_fp32
    N, d, dv = 3, 6, 4
    a, b, c = [oracle_mod.State(*(x.double().numpy() for x in random_state_fp32(N, d, dv, s)))
               for s in (1, 2, 3)]
    ab_c = oracle_mod.compose(oracle_mod.compose(a, b), c)
    a_bc = oracle_mod.compose(a, oracle_mod.compose(b, c))
    _close_state(ab_c, a_bc, 1e-13)
    e = oracle_mod.State.zeros(N, d, dv)
    _close_state(oracle_mod.compose(e, a), a, 0)
    _close_state(oracle_mod.compose(a, e), a, 0)
    # not commutative: the cross term is ordered (keys of the later segment)
    ba = oracle_mod.compose(b, a)
    assert rel_all(ba.G, oracle_mod.compose(a, b).G) > 1e-3


# --------------------------------------------------------------------------
# streaming: split-point continuation, decode == next row, causality

@pytest.mark.parametrize("p", [1, 13, 30])
def test_split_point_continuation(oracle_mod, p):
    d, dv, n = 4, 6, 31
    q, k, v = rng_qkv(11, 2, 2, n, d, dv)
    gam, lam = [0.97, 1.0], 0.05
    out, den, fin = oracle_mod.forward(q, k, v, gamma=gam, lam=lam)
    o1, d1, s1 = oracle_mod.forward(q[:, :, :p], k[:, :, :p], v[:, :, :p], gamma=gam, lam=lam)
    o2, d2, s2 = oracle_mod.forward(q[:, :, p:], k[:, :, p:], v[:, :, p:], gamma=gam, lam=lam,
                                    init=s1)
    assert rel_row(np.concatenate([o1, o2], axis=2), out) < 1e-12
    assert rel_all(np.concatenate([d1, d2], axis=2), den) < 1e-12
    _close_state(s2, fin, 1e-12)


def test_decode_equals_next_row(oracle_mod):
    d, dv, n = 5, 3, 19
    q, k, v = rng_qkv(12, 2, 3, n + 1, d, dv)
    gam, lam = [1.0, 0.9, 0.99], 0.2
    out, den, fin = oracle_mod.forward(q, k, v, gamma=gam, lam=lam)
    _, _, st = oracle_mod.forward(q[:, :, :n], k[:, :, :n], v[:, :, :n], gamma=gam, lam=lam)
    o, dn, st2 = oracle_mod.decode(st, q[:, :, n], k[:, :, n], v[:, :, n], gamma=gam, lam=lam)
    assert rel_row(o, out[:, :, n]) < 1e-13
    assert rel_all(dn, den[:, :, n]) < 1e-13
    _close_state(st2, fin, 1e-13)
    on, _, _ = oracle_mod.decode(st, q[:, :, n], k[:, :, n], v[:, :, n], gamma=gam, lam=lam,
                                 normalize=True)
    assert rel_row(on, o / dn[..., None]) < 1e-14


def test_strict_causality(oracle_mod):
    d, dv, n = 4, 4, 25
    q, k, v = rng_qkv(13, 1, 1, n, d, dv)
    out, den, _ = oracle_mod.forward(q, k, v, gamma=[0.9], lam=0.1)
    t = 11
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    r = np.random.default_rng(0)
    q2[:, :, t + 1:] += r.standard_normal(q2[:, :, t + 1:].shape)
    k2[:, :, t + 1:] += r.standard_normal(k2[:, :, t + 1:].shape)
    v2[:, :, t + 1:] += r.standard_normal(v2[:, :, t + 1:].shape)
    o2, d2, _ = oracle_mod.forward(q2, k2, v2, gamma=[0.9], lam=0.1)
    assert np.array_equal(o2[:, :, : t + 1], out[:, :, : t + 1])
    assert np.array_equal(d2[:, :, : t + 1], den[:, :, : t + 1])
    assert not np.allclose(o2[:, :, t + 1:], out[:, :, t + 1:])


def test_heads_independent_and_batch_layout(oracle_mod):
    d, dv, n = 3, 2, 10
    q, k, v = rng_qkv(14, 2, 3, n, d, dv)
    gam = [1.0, 0.8, 0.6]
    out, den, fin = oracle_mod.forward(q, k, v, gamma=gam, lam=0.1)
    for b in range(2):
        for h in range(3):
            o1, d1, s1 = oracle_mod.forward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                            v[b:b + 1, h:h + 1], gamma=[gam[h]], lam=0.1)
            assert np.array_equal(o1[0, 0], out[b, h])
            assert np.array_equal(s1.G[0], fin.G[b * 3 + h])


def test_threads_do_not_change_results(oracle_mod):
    q, k, v = rng_qkv(15, 3, 4, 33, 8, 8)
    o1, d1, s1 = oracle_mod.forward(q, k, v, gamma=[0.9] * 4, threads=1)
    o8, d8, s8 = oracle_mod.forward(q, k, v, gamma=[0.9] * 4, threads=8)
    assert np.array_equal(o1, o8) and np.array_equal(d1, d8) and np.array_equal(s1.G, s8.G)

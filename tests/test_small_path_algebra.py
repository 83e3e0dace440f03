"""The short-sequence forward computes the masked second-order numerator as
two causal first-order maps (Higher-order Linear Attention, paperlayer.ai
summary sec. 3.1, the mask, and sec. 4.3, the decay: the masked output keeps
the pairs of the key moment and the query-value moment whose key comes no
later than its query).  With
LA(A, B, C; r)_t = sum over s <= t of r^(t-s) (a_t . b_s) c_s:

    U = LA(Q, K, K; g),   out = LA(Q, U, V; g^2).

These CPU tests check that identity in fp64 against the serial oracle,
which runs the state recurrence token by token, and check that plausible
slips in it (the decay of the second map taken as g, or the maps' mask taken
as strict) are caught.
"""
import numpy as np
import pytest

import oracle



def la(a, b, c, r, strict=False):
    """LA(A, B, C; r) over one head: a, b [n, da], c [n, dc], in fp64."""
    n = a.shape[0]
    t = np.arange(n)
    e = t[:, None] - t[None, :]
    mask = e > 0 if strict else e >= 0
    w = np.where(mask, np.power(r, np.where(mask, e, 0)), 0.0)
    return ((a @ b.T) * w) @ c


def two_maps(q, k, v, g, second_decay_square=True, strict=False):
    B, H, n, _ = q.shape
    out = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            gh = 1.0 if g is None else g[h]
            u = la(q[b, h], k[b, h], k[b, h], gh, strict)
            out[b, h] = la(q[b, h], u, v[b, h], gh * gh if second_decay_square else gh, strict)
    return out


def inputs(B, H, n, d, dv, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, n, d)) / np.sqrt(d), rng.standard_normal((B, H, n, d)) / np.sqrt(d),
            rng.standard_normal((B, H, n, dv)) / np.sqrt(d))


def rel(x, ref):
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("B,H,n,d,dv,g", [
    (1, 1, 256, 16, 16, None),          # the small fp32 workload's shape
    (2, 3, 37, 16, 32, [0.9, 0.5, 1.0]),
    (1, 2, 1, 32, 16, [0.3, 1.0]),
    (1, 2, 70, 32, 32, [0.97, 0.75]),
])
def test_two_maps_equal_the_serial_recurrence(B, H, n, d, dv, g):
    q, k, v = inputs(B, H, n, d, dv, seed=B * 1000 + n)
    ref = oracle.forward(q, k, v, gamma=g, want_state=False)[0]
    assert rel(two_maps(q, k, v, g), ref) < 1e-12


def test_slips_in_the_identity_are_caught():
    q, k, v = inputs(1, 1, 48, 16, 16, seed=7)
    ref = oracle.forward(q, k, v, gamma=[0.9], want_state=False)[0]
    assert rel(two_maps(q, k, v, [0.9]), ref) < 1e-12
    assert rel(two_maps(q, k, v, [0.9], second_decay_square=False), ref) > 1e-3
    assert rel(two_maps(q, k, v, [0.9], strict=True), ref) > 1e-3


def test_the_last_token_is_a_closed_form():
    # o_{n-1} = sum over i <= j of (q . k_i)(k_i . q_j) v_j with no decay,
    # written as q^T S_j q_j summed against v_j
    q, k, v = inputs(1, 1, 9, 4, 3, seed=11)
    Q, K, V = q[0, 0], k[0, 0], v[0, 0]
    o = np.zeros(3)
    for j in range(9):
        S = sum(np.outer(K[i], K[i]) for i in range(j + 1))
        o += (Q[8] @ S @ Q[j]) * V[j]
    assert rel(two_maps(q, k, v, None)[0, 0, 8], o) < 1e-13

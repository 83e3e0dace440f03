"""CPU checks of the packed key-moment layout (tests/packed.py) and of the
oracle's grouped decode step (oracle.decode_mq)."""
import numpy as np
import pytest
import torch

import hla_inputs as inputs
import packed


@pytest.mark.parametrize("d", [32, 64, 128])
def test_packed_order_is_the_upper_triangle_once(d):
    ix = packed.order(d)
    assert len(ix) == d * (d + 1) // 2
    assert np.all(ix[:, 0] <= ix[:, 1])
    assert len({(int(a), int(b)) for a, b in ix}) == len(ix)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_pack_unpack_round_trip(d):
    rng = np.random.default_rng(d)
    a = rng.standard_normal((3, d, d))
    S = a + a.transpose(0, 2, 1)
    P = packed.pack(S)
    assert P.shape == (3, d * (d + 1) // 2)
    assert np.array_equal(packed.unpack(P, d), S)
    # the first stored elements are row 0 of the first diagonal tile
    assert np.array_equal(P[:, :32], S[:, 0, :32])


@pytest.mark.parametrize("G,H", [(1, 4), (2, 4), (4, 4)])
def test_decode_mq_is_the_per_head_step_with_the_group_keys(oracle_mod, G, H):
    """decode_mq equals one ordinary decode per query head with its group's
    k and v, and keeps S equal within a group (checked against a loop over
    heads that calls the single-head decode on each)."""
    B, d, dv, R = 2, 16, 8, H // G
    (pq, pk, pv), (q1, k1, v1) = inputs.decode_inputs(B, G, 20, d, dv, torch.float32, seed=170 + G)
    pq = inputs.qkv(B, H, 20, d, dv, torch.float32, seed=171)[0]
    q1 = inputs.decode_inputs(B, H, 0, d, dv, torch.float32, seed=172)[1][0]
    g = [0.9] * R + [0.95] * R if G == 2 else [0.97] * H
    # the prefix with the group's keys and values on every head of the group
    rep = lambda x: x.repeat_interleave(R, dim=1)
    _, _, st = oracle_mod.forward(pq, rep(pk), rep(pv), gamma=g, lam=0.1)
    out, den, new = oracle_mod.decode_mq(st, q1, k1, v1, gamma=g, lam=0.1)
    for b in range(B):
        for h in range(H):
            i = b * H + h
            one = oracle_mod.State(*(np.ascontiguousarray(x[i:i + 1]) for x in st.flat()))
            o1, d1, s1 = oracle_mod.decode(one, q1[b:b + 1, h:h + 1], k1[b:b + 1, h // R:h // R + 1],
                                           v1[b:b + 1, h // R:h // R + 1], gamma=[g[h]], lam=0.1)
            assert np.array_equal(o1[0, 0], out[b, h]) and np.array_equal(d1[0, 0], den[b, h])
            assert np.array_equal(s1.S[0], new.S[i]) and np.array_equal(s1.G[0], new.G[i])

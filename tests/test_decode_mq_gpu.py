"""GPU parity of the decode step with a packed key moment shared by groups of
query heads (hla_decode_step_mq) and of the key-moment pack / unpack calls,
against the fp64 oracle (oracle.decode_mq: the ordinary per-head step with
the group's keys and values) and the packed layout written out index by index
(tests/packed.py)."""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
import packed
from parity import TOL, naive_scales, row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("d", [32, 64, 128])
def test_pack_and_unpack_match_the_layout(d):
    rng = np.random.default_rng(200 + d)
    a = rng.standard_normal((37, d, d)).astype(np.float32)
    S = a + a.transpose(0, 2, 1)
    Sg = torch.from_numpy(S).to(DEV)
    P = hla.key_moment_pack(Sg)
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), packed.pack(S))
    P_nan = torch.full_like(Sg, float("nan"))
    U = hla.key_moment_unpack(P, d, out=P_nan)
    torch.cuda.synchronize()
    assert torch.equal(U.cpu(), torch.from_numpy(S))


def grouped_setup(B, H, G, prefix, d, dv, seed, gamma=None, ridge=0.0):
    """A prefix folded by the oracle with each group's k, v on all of its
    query heads; the fp32-rounded states go to both sides (the GPU side with S
    packed, one per group)."""
    import oracle
    R = H // G
    q = inputs.qkv(B, H, prefix, d, dv, torch.bfloat16, seed)[0]
    _, k, v = inputs.qkv(B, G, prefix, d, dv, torch.bfloat16, seed + 1)
    rep = lambda x: x.repeat_interleave(R, dim=1)
    _, _, st = oracle.forward(q, rep(k), rep(v), gamma=gamma, lam=ridge)
    st32 = {n: torch.from_numpy(getattr(st, n)).float() for n in ("S", "C", "m", "G", "h", "rho")}
    ref = oracle.State(*(st32[n].double().numpy() for n in ("S", "C", "m", "G", "h", "rho")))
    S_groups = st32["S"].reshape(B, G, R, d, d)[:, :, 0].reshape(B * G, d, d)
    rho_groups = st32["rho"].reshape(B, G, R)[:, :, 0].reshape(B * G)
    gpu = hla.MqState(torch.from_numpy(packed.pack(S_groups.numpy())).to(DEV),
                      *(st32[n].to(DEV) for n in ("C", "m", "G", "h")), rho_groups.to(DEV).contiguous())
    return gpu, ref


def check_mq_state(gpu: hla.MqState, ref, B, H, G, d, tol):
    R = H // G
    S_full = packed.unpack(gpu.S.cpu().double().numpy(), d)             # [B*G, d, d]
    S_heads = np.repeat(S_full.reshape(B, G, d, d), R, axis=1).reshape(B * H, d, d)
    sc, sm = naive_scales(ref.S, ref.C, ref.m)
    got = {"S": S_heads, "C": gpu.C.cpu(), "m": gpu.m.cpu(), "G": gpu.G.cpu(), "h": gpu.h.cpu()}
    for k in ("S", "C", "m", "G", "h"):
        scale = sc if k == "G" else sm if k == "h" else None
        e = slab_err(got[k], getattr(ref, k), scale=scale)
        assert e <= tol, f"state {k}: slab error {e:.3e}"
    rho = gpu.rho.cpu().double().numpy()
    ref_rho = np.asarray(ref.rho, np.float32).astype(np.float64).reshape(B, G, R)[:, :, 0].reshape(-1)
    assert np.allclose(rho, ref_rho, rtol=1e-5, atol=1.2e-38)


CASES = [  # B, H, G, d, dv, gamma, ridge, normalize
    (4, 8, 8, 128, 128, None, 0.0, False),       # unshared, packed
    (4, 8, 1, 128, 128, None, 0.0, False),       # multi-query: one group
    (2, 8, 2, 64, 32, "per_group", 1e-3, True),  # grouped, decay per group, ridge, ratio
    (3, 4, 4, 32, 64, "decay", 0.5, False),
    (2, 16, 4, 128, 16, "per_group", 0.0, True),
    (16, 4, 1, 64, 64, None, 0.0, False),        # 16 groups: the XCD-grouped head order
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}G{c[2]}d{c[3]}dv{c[4]}-{c[5]}-l{c[6]}-n{int(c[7])}")
def test_decode_mq_three_steps(case):
    import oracle
    B, H, G, d, dv, gk, ridge, norm = case
    R = H // G
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.97] * H)
    elif gk == "per_group":
        g = inputs.gamma_list_fp32([1 - 2.0 ** -(3 + h // R) for h in range(H)])
    ridge = inputs.ridge_fp32(ridge)
    gpu, ref = grouped_setup(B, H, G, 48, d, dv, 210 + d + G, gamma=g, ridge=ridge)
    tol = TOL[torch.bfloat16]
    for step in range(3):
        q1 = inputs.qkv(B, H, 1, d, dv, torch.bfloat16, 300 + step)[0][:, :, 0].contiguous()
        _, k1, v1 = (x[:, :, 0].contiguous() for x in inputs.qkv(B, G, 1, d, dv, torch.bfloat16, 310 + step))
        out, den = hla.decode_step_mq(q1.to(DEV), k1.to(DEV), v1.to(DEV), gpu, gamma=g, ridge=ridge,
                                      normalize=norm, return_den=True)
        torch.cuda.synchronize()
        r_out, r_den, ref = oracle.decode_mq(ref, q1, k1, v1, gamma=g, lam=ridge, normalize=norm)
        if norm:
            keep = np.abs(r_den) >= 1e-2 * np.median(np.abs(r_den))
            e = row_err(out.cpu().numpy()[keep], r_out[keep])
        else:
            e = row_err(out.cpu(), r_out)
        print(f"step {step}: row error {e:.3e}")
        assert e <= tol
        assert slab_err(den.cpu().reshape(-1, 1), r_den.reshape(-1, 1)) <= tol
        check_mq_state(gpu, ref, B, H, G, d, 1e-5)


def test_decode_mq_unshared_matches_decode_step():
    """With one query head per group the packed step is the ordinary step on
    packed storage: out and every state part agree with hla_decode_step
    (to fp32 rounding order) and S stays the packed form of its S."""
    B, H, d, dv = 8, 16, 128, 128
    st = inputs.random_state_fp32(B * H, d, dv, 220, scale=0.1)
    full = hla.State(*(t.to(DEV) for t in st))
    mq = hla.MqState(hla.key_moment_pack(full.S), full.C.clone(), full.m.clone(), full.G.clone(), full.h.clone(),
                     full.rho.clone())
    q, k, v = (x.to(DEV) for x in inputs.decode_inputs(B, H, 0, d, dv, torch.bfloat16, seed=221)[1])
    o1, d1 = hla.decode_step(q, k, v, full, return_den=True)
    o2, d2 = hla.decode_step_mq(q, k, v, mq, return_den=True)
    torch.cuda.synchronize()
    assert row_err(o2.cpu(), o1.cpu()) <= 1e-5
    assert slab_err(d2.cpu().reshape(-1, 1), d1.cpu().reshape(-1, 1)) <= 1e-5
    assert torch.equal(hla.key_moment_unpack(mq.S, d).cpu(), full.S.cpu())  # same elementwise update
    for a, b in ((mq.C, full.C), (mq.m, full.m), (mq.G, full.G), (mq.h, full.h), (mq.rho, full.rho)):
        assert torch.equal(a, b)


def test_decode_mq_writes_every_output_and_rejects_bad_groups():
    B, H, G, d, dv = 4, 8, 2, 64, 64
    gpu, _ = grouped_setup(B, H, G, 16, d, dv, 230)
    q1 = inputs.qkv(B, H, 1, d, dv, torch.bfloat16, 231)[0][:, :, 0].contiguous().to(DEV)
    _, k1, v1 = (x[:, :, 0].contiguous().to(DEV) for x in inputs.qkv(B, G, 1, d, dv, torch.bfloat16, 232))
    out = torch.full((B, H, dv), float("nan"), device=DEV)
    den = torch.full((B, H), float("nan"), device=DEV)
    hla.decode_step_mq(q1, k1, v1, gpu, out=out, den=den)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(den).all()
    with pytest.raises(hla.HlaError, match="gamma"):
        hla.decode_step_mq(q1, k1, v1, gpu, gamma=[0.9, 0.9, 0.9, 0.8, 0.9, 0.9, 0.9, 0.9])
    k3 = torch.zeros(B, 3, d, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(hla.HlaError, match="kv_heads"):
        hla.decode_step_mq(q1, k3, torch.zeros(B, 3, dv, dtype=torch.bfloat16, device=DEV), gpu)

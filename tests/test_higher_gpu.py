"""GPU parity of the asymmetric variant (hla_ahla_forward, hla_ahla_decode_step)
and of masked third order (hla_third_forward, hla_third_decode_step) against
the fp64 oracle (oracle/higher.py) on identical seeded inputs.  Tolerances as
for the second-order path: 2e-3 for bf16 inputs and 1e-5 for fp32 inputs, on
the row error of outputs and the slab error of denominators and states."""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from oracle import higher
from parity import TOL, ratio_err, row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def on_gpu(*ts):
    return [t.to(DEV).contiguous() for t in ts]


def gammas(gk, H):
    if gk == "decay":
        return inputs.gamma_list_fp32([0.97] * H)
    if gk == "per_head":
        return inputs.gamma_list_fp32([1 - 2.0 ** -(3 + h % 6) for h in range(H)])
    return None


def check_out(o, d, ro, rd, normalize, tol):
    if normalize:
        e, _ = ratio_err(o, ro, rd)
    else:
        e = row_err(o, ro)
    print(f"output error {e:.3e}")
    assert e <= tol
    ed = slab_err(d, rd, lead=2)
    print(f"den slab error {ed:.3e}")
    assert ed <= tol


AHLA_CASES = [  # B, H, n, d, dv, w, dtype, gamma, normalize
    (1, 2, 100, 16, 16, 16, torch.float32, None, False),
    (2, 2, 77, 32, 64, 32, torch.float32, "decay", False),
    (1, 3, 130, 64, 16, 64, torch.float32, "per_head", True),
    (1, 1, 300, 128, 128, 128, torch.float32, "decay", False),
    (2, 2, 129, 64, 64, 64, torch.bfloat16, None, False),
    (1, 2, 200, 64, 64, 16, torch.bfloat16, "per_head", True),
    (1, 2, 257, 128, 64, 128, torch.bfloat16, "decay", False),
    (2, 1, 1, 64, 64, 64, torch.bfloat16, None, False),
]


def _ids(cases):
    return [f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}dv{c[4]}w{c[5]}{'bf16' if c[6] == torch.bfloat16 else 'f32'}-{c[7]}"
            f"{'-norm' if c[8] else ''}" for c in cases]


@pytest.mark.parametrize("case", AHLA_CASES, ids=_ids(AHLA_CASES))
def test_ahla_sweep(case):
    B, H, n, d, dv, w, dtype, gk, norm = case
    q, k, v = inputs.qkv(B, H, n, d, dv, dtype, seed=600 + n + d + dv + w)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = gammas(gk, H)
    out, den, fin = hla.ahla_forward(*on_gpu(q, k, v), gamma=g, normalize=norm, chunk=w, return_den=True,
                                     return_state=True)
    torch.cuda.synchronize()
    ro, rd, rf = higher.ahla_forward(q, k, v, gamma=g, normalize=norm)
    tol = TOL[dtype]
    check_out(out.cpu(), den.cpu(), ro, rd, norm, tol)
    for name in ("P", "m", "E", "n"):
        e = slab_err(getattr(fin, name).cpu(), getattr(rf, name))
        assert e <= max(tol, 1e-5), f"state {name}: {e:.3e}"
    ref_rho = np.asarray(rf.rho, np.float32).astype(np.float64)
    assert np.allclose(fin.rho.cpu().double().numpy(), ref_rho, rtol=1e-5, atol=1.2e-38)


THIRD_CASES = [
    (1, 2, 100, 16, 16, 16, torch.float32, None, False),
    (2, 2, 77, 32, 64, 32, torch.float32, None, True),
    (1, 1, 300, 128, 128, 128, torch.float32, None, False),
    (2, 2, 129, 64, 64, 64, torch.bfloat16, None, False),
    (1, 2, 200, 64, 32, 16, torch.bfloat16, None, True),
    (1, 2, 257, 128, 64, 128, torch.bfloat16, None, False),
    (2, 1, 1, 64, 64, 64, torch.bfloat16, None, False),
]


@pytest.mark.parametrize("case", THIRD_CASES, ids=_ids(THIRD_CASES))
def test_third_sweep(case):
    B, H, n, d, dv, w, dtype, _, norm = case
    q, k, v = inputs.qkv(B, H, n, d, dv, dtype, seed=700 + n + d + dv + w)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    out, den, fin = hla.third_forward(*on_gpu(q, k, v), normalize=norm, chunk=w, return_den=True,
                                      return_state=True)
    torch.cuda.synchronize()
    ro, rd, rf = higher.third_forward(q, k, v, normalize=norm)
    tol = TOL[dtype]
    check_out(out.cpu(), den.cpu(), ro, rd, norm, tol)
    for name in ("S", "P", "m", "F", "Fd"):
        e = slab_err(getattr(fin, name).cpu(), getattr(rf, name))
        assert e <= max(tol, 1e-5), f"state {name}: {e:.3e}"


@pytest.mark.parametrize("third", [False, True])
def test_bench_shape(third):
    """B4 H8 n2048 d = dv = 64 bf16, chunk 64 (AHLA with decay per head)."""
    w = inputs.FWD_D64
    q, k, v = inputs.workload_qkv(w, 1011 + int(third))
    g = None if third else inputs.gamma_list_fp32([1 - 2.0 ** -(5 + h) for h in range(w.H)])
    if third:
        out, _, _ = hla.third_forward(*on_gpu(q, k, v), chunk=64)
        ro, _, _ = higher.third_forward(q, k, v, want_state=False)
    else:
        out, _, _ = hla.ahla_forward(*on_gpu(q, k, v), gamma=g, chunk=64)
        ro, _, _ = higher.ahla_forward(q, k, v, gamma=g, want_state=False)
    torch.cuda.synchronize()
    e = row_err(out.cpu(), ro)
    print(f"row error {e:.3e}")
    assert e <= TOL[torch.bfloat16]


@pytest.mark.parametrize("third", [False, True])
def test_continuation_and_decode(third):
    """forward(t < p) -> final state -> forward(t >= p, init) equals the whole
    sequence, and a decode step from the GPU state equals the next row."""
    B, H, n, d, dv, p = 2, 3, 301, 64, 32, 133
    q, k, v = on_gpu(*inputs.qkv(B, H, n + 1, d, dv, torch.float32, seed=800 + int(third)))
    g = None if third else inputs.gamma_list_fp32([0.99, 0.97, 1.0])
    fwd = (lambda *a, **kw: hla.third_forward(*a, **kw)) if third else \
        (lambda *a, **kw: hla.ahla_forward(*a, gamma=g, **kw))
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    whole, wden, _ = fwd(sl(q, 0, n), sl(k, 0, n), sl(v, 0, n), return_den=True)
    o1, _, s1 = fwd(sl(q, 0, p), sl(k, 0, p), sl(v, 0, p), return_state=True)
    o2, _, s2 = fwd(sl(q, p, n), sl(k, p, n), sl(v, p, n), init=s1, return_state=True)
    torch.cuda.synchronize()
    assert row_err(torch.cat([o1, o2], dim=2).cpu(), whole.cpu()) <= 1e-5
    nxt, _, _ = fwd(q, k, v)
    if third:
        o, dn = hla.third_decode_step(q[:, :, n].contiguous(), k[:, :, n].contiguous(), v[:, :, n].contiguous(), s2,
                                      return_den=True)
    else:
        o, dn = hla.ahla_decode_step(q[:, :, n].contiguous(), k[:, :, n].contiguous(), v[:, :, n].contiguous(), s2,
                                     gamma=g, return_den=True)
    torch.cuda.synchronize()
    assert row_err(o.cpu(), nxt[:, :, n].cpu()) <= 1e-5


@pytest.mark.parametrize("third,dtype,d,dv,norm", [(False, torch.bfloat16, 128, 128, False),
                                                   (False, torch.float32, 32, 64, True),
                                                   (True, torch.bfloat16, 128, 64, False),
                                                   (True, torch.float32, 64, 16, True)])
def test_decode_against_oracle(third, dtype, d, dv, norm):
    """Three decode steps from an oracle state (fp32-rounded, given to both)."""
    B, H = 4, 4
    (pq, pk, pv), _ = inputs.decode_inputs(B, H, 40, d, dv, dtype, seed=820 + d)
    if norm:
        pq, pk = (x.float().abs().add(0.1).to(dtype) for x in (pq, pk))
    g = None if third else inputs.gamma_list_fp32([0.95, 0.99, 1.0, 0.9])
    if third:
        _, _, rs = higher.third_forward(pq, pk, pv)
        parts = {n: torch.from_numpy(getattr(rs, n)).float() for n in ("S", "P", "m", "F", "Fd")}
        ref = higher.ThirdState(*(parts[n].double().numpy() for n in ("S", "P", "m", "F", "Fd")))
        st = hla.ThirdState(*(parts[n].to(DEV) for n in ("S", "P", "m", "F", "Fd")))
    else:
        _, _, rs = higher.ahla_forward(pq, pk, pv, gamma=g)
        parts = {n: torch.from_numpy(getattr(rs, n)).float() for n in ("P", "m", "E", "n", "rho")}
        ref = higher.AhlaState(*(parts[n].double().numpy() for n in ("P", "m", "E", "n")), None,
                               parts["rho"].double().numpy())
        st = hla.AhlaState(*(parts[n].to(DEV) for n in ("P", "m", "E", "n", "rho")))
    tol = TOL[dtype]
    for step in range(3):
        _, (q1, k1, v1) = inputs.decode_inputs(B, H, 0, d, dv, dtype, seed=830 + step)
        if norm:
            q1, k1 = (x.float().abs().add(0.1).to(dtype) for x in (q1, k1))
        if third:
            o, dn = hla.third_decode_step(*on_gpu(q1, k1, v1), st, normalize=norm, return_den=True)
            ro, rd, ref = higher.third_decode(ref, q1, k1, v1, normalize=norm)
        else:
            o, dn = hla.ahla_decode_step(*on_gpu(q1, k1, v1), st, gamma=g, normalize=norm, return_den=True)
            ro, rd, ref = higher.ahla_decode(ref, q1, k1, v1, gamma=g, normalize=norm)
        torch.cuda.synchronize()
        assert row_err(o.cpu(), ro) <= tol
        assert slab_err(dn.cpu().reshape(-1, 1), rd.reshape(-1, 1)) <= tol
    for name in (("S", "P", "m", "F", "Fd") if third else ("P", "m", "E", "n")):
        assert slab_err(getattr(st, name).cpu(), getattr(ref, name)) <= 1e-5, name


@pytest.mark.parametrize("third", [False, True])
def test_causality_nan_poison_and_errors(third):
    B, H, n, d, dv = 1, 2, 256, 64, 64
    q, k, v = on_gpu(*inputs.qkv(B, H, n, d, dv, torch.bfloat16, seed=840))
    fwd = hla.third_forward if third else hla.ahla_forward
    # every output and denominator is written (the chunked fp32 kernels: a
    # denominator is asked for)
    out = torch.full((B, H, n, dv), float("nan"), device=DEV)
    den = torch.full((B, H, n), float("nan"), device=DEV)
    fwd(q, k, v, out=out, den=den)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(den).all()
    # causality, bitwise, on the numerator-only one-launch path
    out = torch.full((B, H, n, dv), float("nan"), device=DEV)
    fwd(q, k, v, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    for t in (0, 63, 64, 200):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        for x in (q2, k2, v2):
            x[:, :, t + 1:] = -x[:, :, t + 1:]
        o2, _, _ = fwd(q2, k2, v2)
        assert torch.equal(o2[:, :, : t + 1], out[:, :, : t + 1]), t
    p_ridge = dict(gamma=[0.9, 0.9])
    if third:
        with pytest.raises(hla.HlaError, match="no decay"):
            hla._binding._higher_forward(True, q, k, v, [0.9, 0.9], False, 0, None, False, False, None, None,
                                         None, None)
    else:
        out2, _, _ = hla.ahla_forward(q, k, v, **p_ridge)  # decay is fine for AHLA
        torch.cuda.synchronize()
        assert torch.isfinite(out2).all()


ONE_LAUNCH = [  # B, H, n: the bench shape (one segment of four chunks per workgroup), ragged
    (4, 8, 2048), (2, 3, 64 * 13 + 37),  # (14 one-chunk segments per head), a looped grid (288 segments),
    (4, 8, 64 * 32 + 37), (1, 2, 50), (2, 1, 1)]  # one segment, one token


@pytest.mark.parametrize("third", [False, True])
@pytest.mark.parametrize("B,H,n", ONE_LAUNCH)
def test_one_launch_path(third, B, H, n):
    """bf16, d = dv = 64, chunk 64, numerator only.  The first-order map
    gives the intermediate values as a bf16 pair, and the second map (first
    order for AHLA, second order for third order) takes that pair as its
    values: for AHLA both maps in one launch, the pair kept in LDS (two
    hand-offs); for third order two launches, the pair through HBM.  The
    control block counts the launches and shows that no wait gave up.  AHLA
    with a decay per head down to 0.75."""
    q, k, v = inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=1700 + n + H + int(third))
    g = None if third else inputs.gamma_list_fp32([(0.75, 0.9, 0.97, 1.0, 0.999, 0.8, 0.95, 0.99)[h % 8]
                                                   for h in range(H)])
    size_fn = hla._binding.load().hla_third_workspace_size if third else hla._binding.load().hla_ahla_workspace_size
    p, _keep = hla._binding._params(B, H, n, 64, 64, 64, torch.bfloat16, g, 0.0, False)
    ws = torch.zeros(int(size_fn(hla._binding.ctypes.byref(p))), dtype=torch.uint8, device=DEV)
    fwd = hla.third_forward if third else hla.ahla_forward
    kw = {} if third else {"gamma": g}
    out, _, _ = fwd(*on_gpu(q, k, v), chunk=64, workspace=ws, **kw)
    torch.cuda.synchronize()
    words = ws[:16].view(torch.int32).cpu().tolist()
    assert words[2] == (2 if third else 1) and words[3] == 0, words
    ro, _, _ = (higher.third_forward(q, k, v, want_state=False) if third
                else higher.ahla_forward(q, k, v, gamma=g, want_state=False))
    e = row_err(out.cpu(), ro)
    print(f"row error {e:.3e}")
    assert e <= TOL[torch.bfloat16]
    out2, _, _ = fwd(*on_gpu(q, k, v), chunk=64, workspace=ws, **kw)  # the same workspace again
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    assert ws[:16].view(torch.int32).cpu().tolist()[2] == (4 if third else 2)


def test_one_launch_ahla_give_up_poisons_and_recovers():
    """With control word 4 = -1 the chained AHLA launch's waits give up after
    one unsuccessful poll (both hand-offs).  Every output row is then the
    normal bits or holds a NaN, the first chunk of each head (its segment
    waits on nothing) is exact, and NaN rows appear exactly when a wait gave
    up.  With word 4 back to 0 the next call on the same workspace gives the
    normal bits again."""
    B, H, n = 4, 8, 2048
    q, k, v = inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=1750)
    g = inputs.gamma_list_fp32([(0.75, 0.9, 0.97, 1.0, 0.999, 0.8, 0.95, 0.99)[h % 8] for h in range(H)])
    p, _keep = hla._binding._params(B, H, n, 64, 64, 64, torch.bfloat16, g, 0.0, False)
    ws = torch.zeros(int(hla._binding.load().hla_ahla_workspace_size(hla._binding.ctypes.byref(p))),
                     dtype=torch.uint8, device=DEV)
    qg, kg, vg = on_gpu(q, k, v)
    ref, _, _ = hla.ahla_forward(qg, kg, vg, gamma=g, chunk=64, workspace=ws)
    words = ws[:64].view(torch.int32)
    words[4] = -1
    out, _, _ = hla.ahla_forward(qg, kg, vg, gamma=g, chunk=64, workspace=ws)
    torch.cuda.synchronize()
    w = words.cpu().tolist()
    assert w[2] == 2, w
    rows_nan = torch.isnan(out).any(dim=-1)
    rows_same = (out == ref).all(dim=-1)
    assert bool((rows_nan | rows_same).all()), "a row is neither NaN nor the normal result"
    assert bool(rows_same[:, :, :64].all()), "the first chunk of a head waits on nothing"
    assert bool(rows_nan.any()) == (w[3] > 0)
    words[4] = 0
    again, _, _ = hla.ahla_forward(qg, kg, vg, gamma=g, chunk=64, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)

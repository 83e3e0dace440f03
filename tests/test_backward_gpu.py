"""GPU parity of the backward (hla_backward_chunked through the C ABI) against
the fp64 autograd oracle (oracle/backward.py) on identical seeded inputs.

The chunked backward computes in fp32 from exactly widened inputs, so bf16
and fp32 inputs share one gate: slab error (per (b, h), max |x - ref| /
max |ref|) of each gradient at most 1e-5 (fp32 accumulation over a few
hundred terms of mixed sign; see the tolerance reading in the design notes).
bf16 calls with d = dv = 64, chunk 64, no ridge, ratio or states and every
decay >= 0.75 take the one-launch backward instead (first-order maps on bf16
MFMA, fp32 intermediates carried as bf16 pairs); its gate is FTOL
(tests/test_backward_fast_gpu.py).  With the
ratio, q and k are drawn positive (|x| + 0.1 of the seeded draws) so that
every denominator is bounded away from zero.
"""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GTOL = 1e-5
FTOL = 1e-4  # the one-launch backward (bf16 pairs: products to about 2^-16)


def fast_path(dtype, d, dv, chunk, gk, lam, norm):
    return (dtype == torch.bfloat16 and d == dv == 64 and chunk == 64 and lam == 0.0 and not norm
            and gk in (None, "decay", "per_head"))


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def make(B, H, n, d, dv, dtype, gk, norm, seed):
    q, k, v = inputs.qkv(B, H, n, d, dv, dtype, seed=seed)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.97] * H)
    elif gk == "per_head":
        g = inputs.gamma_list_fp32([1 - 2.0 ** -(3 + h % 6) for h in range(H)])
    elif gk == "strong":  # g^k underflows fp32 inside a 128-token chunk (0.3^80 < 1e-38)
        g = inputs.gamma_list_fp32([0.3, 0.6][:H])
    dout = inputs.upstream(B, H, n, dv, seed=seed + 7)
    return q, k, v, dout, g


def run_gpu(q, k, v, dout, g, lam, norm, chunk):
    qg, kg, vg, dg = (x.to(DEV).contiguous() for x in (q, k, v, dout))
    out = hla.backward_chunked(qg, kg, vg, dg, gamma=g, ridge=lam, normalize=norm, chunk=chunk)
    torch.cuda.synchronize()
    return [x.cpu() for x in out]


def check(got, ref, names=("dq", "dk", "dv"), tol=GTOL):
    errs = {}
    for name, x, r in zip(names, got, ref):
        e = slab_err(x, r, lead=2)
        errs[name] = e
        print(f"{name}: slab {e:.3e} row {row_err(x, r):.3e}")
    for name, e in errs.items():
        assert e <= tol, f"{name}: slab error {e:.3e} > {tol:.0e}"


CASES = [
    # B, H, n, d, dv, chunk, dtype, gamma, ridge, normalize
    (1, 2, 150, 32, 32, 64, torch.float32, "per_head", 0.0, False),
    (1, 2, 150, 32, 32, 64, torch.float32, "per_head", 0.3, False),
    (1, 2, 150, 32, 32, 64, torch.float32, "per_head", 0.3, True),
    (2, 3, 257, 64, 64, 64, torch.bfloat16, "decay", 0.0, False),
    (1, 2, 300, 128, 128, 128, torch.bfloat16, "decay", 1e-3, True),
    (1, 1, 33, 16, 128, 16, torch.float32, None, 0.0, False),
    (1, 2, 70, 128, 32, 32, torch.float32, None, 0.2, False),
    (2, 2, 1, 64, 64, 64, torch.bfloat16, None, 0.0, False),
    (1, 1, 64, 16, 16, 16, torch.float32, "decay", 0.0, True),
    (1, 3, 200, 64, 16, 128, torch.bfloat16, "per_head", 0.5, False),
    (1, 2, 300, 32, 32, 128, torch.float32, "strong", 0.2, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}dv{c[4]}w{c[5]}"
                         f"{'bf16' if c[6] == torch.bfloat16 else 'f32'}-{c[7]}-l{c[8]}-r{int(c[9])}")
def test_backward_matches_oracle(case):
    B, H, n, d, dv, chunk, dtype, gk, lam, norm = case
    q, k, v, dout, g = make(B, H, n, d, dv, dtype, gk, norm, seed=500 + n + d)
    lam = inputs.ridge_fp32(lam)
    got = run_gpu(q, k, v, dout, g, lam, norm, chunk)
    from oracle import backward as ob
    ref = ob.backward(q, k, v, dout, g, lam, norm)
    check(got, ref, tol=FTOL if fast_path(dtype, d, dv, chunk, gk, lam, norm) else GTOL)


def test_backward_headline_shape_sampled_heads():
    """The B4 H8 n2048 d64 bf16 workload at full size; the oracle checks two
    (b, h) slabs (heads are independent)."""
    w = inputs.FWD_D64
    q, k, v = inputs.workload_qkv(w, seed=1001)
    dout = inputs.upstream(w.B, w.H, w.n, w.dv, seed=1008)
    got = run_gpu(q, k, v, dout, None, 0.0, False, w.chunk)
    from oracle import backward as ob
    for b, h in ((0, 0), (3, 7)):
        sl = lambda x: x[b:b + 1, h:h + 1]  # noqa: E731
        ref = ob.backward(sl(q), sl(k), sl(v), sl(dout))
        check([sl(x) for x in got], ref, tol=FTOL)  # the one-launch backward


def test_backward_deterministic_and_causal():
    B, H, n, d, dv = 1, 2, 200, 64, 64
    q, k, v, dout, g = make(B, H, n, d, dv, torch.bfloat16, "decay", False, seed=77)
    a = run_gpu(q, k, v, dout, g, 0.1, False, 64)
    b = run_gpu(q, k, v, dout, g, 0.1, False, 64)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    t = 90  # upstream gradient only up to token t: nothing after t receives any
    d2 = dout.clone()
    d2[:, :, t + 1:] = 0
    c = run_gpu(q, k, v, d2, g, 0.1, False, 64)
    for x in c:
        assert torch.count_nonzero(x[:, :, t + 1:]) == 0
        assert torch.count_nonzero(x[:, :, :t + 1]) > 0


def test_backward_agrees_with_forward_difference():
    """<grad, u> against differences of the GPU forward itself along a random
    direction (consistency of the two entry points, independent of the
    oracle).  Without the ratio, out is of degree 5 in (q, k, v) (q_t, k_i,
    k_i, q_j, v_j), so L(x + h u) is a quintic in h, the central difference is
    D(h) = a1 + a3 h^2 + a5 h^4, and two Richardson steps give the derivative
    a1 exactly; only the forward's fp32 rounding remains."""
    B, H, n, d, dv = 1, 2, 96, 32, 32
    q, k, v, dout, g = make(B, H, n, d, dv, torch.float32, "per_head", False, seed=88)
    grads = run_gpu(q, k, v, dout, g, 0.2, False, 32)
    gen = torch.Generator().manual_seed(5)
    u = [torch.randn(x.shape, generator=gen) * 0.1 for x in (q, k, v)]

    def L(h):
        xs = [(x + h * du).to(DEV) for x, du in zip((q, k, v), u)]
        out, _, _ = hla.forward_chunked(*xs, gamma=g, ridge=0.2, chunk=32)
        return float((out.double().cpu() * dout.double()).sum())

    def D(h):
        return (L(h) - L(-h)) / (2 * h)

    def R1(h):
        return (4 * D(h / 2) - D(h)) / 3
    h = 1.0
    fd = (16 * R1(h / 2) - R1(h)) / 15
    an = sum(float((gr.double() * du.double()).sum()) for gr, du in zip(grads, u))
    assert abs(fd - an) <= 2e-4 * abs(an), (fd, an)


@pytest.mark.parametrize("dtype,d,chunk,norm", [(torch.bfloat16, 64, 64, False), (torch.float32, 32, 16, True)])
def test_backward_from_a_state(dtype, d, chunk, norm):
    """Continuing from the state of a prefix (its fp64 oracle state rounded to
    fp32, given to both sides), held constant."""
    import types

    import oracle
    from oracle import backward as ob
    B, H, n0, n = 1, 2, 100, 150
    q, k, v = inputs.qkv(B, H, n0 + n, d, d, dtype, seed=61 + d)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = inputs.gamma_list_fp32([0.97, 0.995])
    lam = inputs.ridge_fp32(0.1)
    _, _, st = oracle.forward(q[:, :, :n0], k[:, :, :n0], v[:, :, :n0], gamma=g, lam=lam)
    f32 = {name: torch.tensor(getattr(st, name), dtype=torch.float32) for name in ("S", "C", "m", "G", "h")}
    init = hla.State(*(f32[x].to(DEV) for x in ("S", "C", "m", "G", "h")))
    qs, ks, vs = (x[:, :, n0:].contiguous() for x in (q, k, v))
    dout = inputs.upstream(B, H, n, d, seed=71)
    qg, kg, vg, dg = (x.to(DEV) for x in (qs, ks, vs, dout))
    got = hla.backward_chunked(qg, kg, vg, dg, gamma=g, ridge=lam, normalize=norm, chunk=chunk, init=init)
    torch.cuda.synchronize()
    ref = ob.backward(qs, ks, vs, dout, g, lam, norm, types.SimpleNamespace(**f32))
    check([x.cpu() for x in got], ref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_autograd_op(dtype):
    """hla.attention as a torch autograd op: loss.backward() through the C ABI
    gives the oracle's gradients (returned in the inputs' dtype)."""
    from oracle import backward as ob
    B, H, n, d, dv = 1, 2, 130, 64, 32
    q, k, v, dout, g = make(B, H, n, d, dv, dtype, "per_head", False, seed=99)
    qg, kg, vg = (x.to(DEV).requires_grad_(True) for x in (q, k, v))
    out = hla.attention(qg, kg, vg, gamma=g, ridge=0.1, chunk=64)
    (out * dout.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    ref = ob.backward(q, k, v, dout, g, inputs.ridge_fp32(0.1), False)
    got = [x.grad.float().cpu() for x in (qg, kg, vg)]
    assert all(x.grad.dtype == dtype for x in (qg, kg, vg))
    if dtype == torch.float32:
        check(got, ref)
    else:  # gradients rounded to bf16 on return: within bf16's half-ulp of the fp32 result
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            e = slab_err(x, r, lead=2)
            assert e <= 2 ** -8, f"{name}: {e:.3e}"


def _dinit_check(got, ref, tol=GTOL):
    """Each part's max abs error over the heads' largest gradient entry in
    that part, floored at 1e-3 of the largest entry over all parts (parts
    that vanish in the algebra are only zero to rounding in the oracle)."""
    top = max(float(np.abs(ref[p]).max()) for p in ref)
    for part in ("S", "C", "m", "G", "h"):
        x = getattr(got, part).double().cpu().numpy()
        r = np.asarray(ref[part]).reshape(x.shape)
        scale = max(float(np.abs(r).max()), 1e-3 * top, 1e-30)
        e = float(np.abs(x - r).max()) / scale
        print(f"dinit.{part}: {e:.3e}")
        assert e <= tol, f"dinit.{part}: error {e:.3e} > {tol:.0e}"


DINIT_CASES = [
    # dtype, d, dv, chunk, n, gamma, ridge, normalize, with init
    (torch.float32, 32, 32, 16, 150, "per_head", 0.1, False, True),
    (torch.bfloat16, 64, 64, 64, 150, "decay", 0.0, False, True),
    (torch.float32, 32, 16, 32, 97, "per_head", 0.2, True, True),
    (torch.bfloat16, 128, 128, 128, 300, "decay", 1e-3, True, True),
    (torch.float32, 16, 64, 16, 70, None, 0.0, False, False),
    (torch.float32, 64, 32, 64, 130, "per_head", 0.3, False, False),
]


@pytest.mark.parametrize("case", DINIT_CASES, ids=lambda c: f"{'bf16' if c[0] == torch.bfloat16 else 'f32'}"
                         f"-d{c[1]}dv{c[2]}w{c[3]}n{c[4]}-{c[5]}-l{c[6]}-r{int(c[7])}-init{int(c[8])}")
def test_backward_initial_state_gradient(case):
    """dL/d(init) through hla_backward_chunked against the fp64 autograd
    oracle, from a prefix state (rounded to fp32 and given to both sides) or
    from the zero state; dq, dk, dv are the same bits with and without it."""
    import types

    import oracle
    from oracle import backward as ob
    dtype, d, dv, chunk, n, gk, lam, norm, with_init = case
    B, H, n0 = 1, 2, 60
    q, k, v = inputs.qkv(B, H, n0 + n, d, dv, dtype, seed=91 + d + n)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.97] * H)
    elif gk == "per_head":
        g = inputs.gamma_list_fp32([0.95, 0.99])
    lam = inputs.ridge_fp32(lam)
    init = ref_init = None
    if with_init:
        _, _, st = oracle.forward(q[:, :, :n0], k[:, :, :n0], v[:, :, :n0], gamma=g, lam=lam)
        f32 = {name: torch.tensor(getattr(st, name), dtype=torch.float32) for name in ("S", "C", "m", "G", "h")}
        if not norm:  # off the method's states: C, G moved independently of S
            f32["C"] = f32["C"] + 0.3 * inputs.upstream(1, 1, B * H * d, dv, seed=93).reshape(B * H, d, dv)
            f32["G"] = f32["G"] - 0.2 * inputs.upstream(1, 1, B * H * d, dv, seed=94).reshape(B * H, d, dv)
        init = hla.State(*(f32[x].to(DEV) for x in ("S", "C", "m", "G", "h")))
        ref_init = types.SimpleNamespace(**f32)
    qs, ks, vs = (x[:, :, n0:].contiguous() for x in (q, k, v))
    dout = inputs.upstream(B, H, n, dv, seed=97)
    qg, kg, vg, dg = (x.to(DEV) for x in (qs, ks, vs, dout))
    dini = hla.State.empty(B * H, d, dv, DEV)
    for t in dini.tensors():
        t.fill_(float("nan"))
    got = hla.backward_chunked(qg, kg, vg, dg, gamma=g, ridge=lam, normalize=norm, chunk=chunk, init=init,
                               dinit=dini)
    plain = hla.backward_chunked(qg, kg, vg, dg, gamma=g, ridge=lam, normalize=norm, chunk=chunk, init=init)
    torch.cuda.synchronize()
    for a, b in zip(got, plain):
        assert torch.equal(a, b)
    assert torch.all(dini.rho == 0.0)
    *ref, rdini = ob.backward(qs, ks, vs, dout, g, lam, norm, ref_init, init_grad=True)
    tol = FTOL if fast_path(dtype, d, dv, chunk, gk, lam, norm) else GTOL
    check([x.cpu() for x in got], ref, tol=tol)
    _dinit_check(dini, rdini, tol)


def test_backward_initial_state_gradient_empty_sequence():
    """n = 0: the gradient of an empty sum is zero in every part set."""
    q = torch.zeros(1, 2, 0, 32, dtype=torch.float32, device=DEV)
    v = torch.zeros(1, 2, 0, 16, dtype=torch.float32, device=DEV)
    dini = hla.State.empty(2, 32, 16, DEV)
    for t in dini.tensors():
        t.fill_(float("nan"))
    hla.backward_chunked(q, q, v, v.clone(), dinit=dini)
    torch.cuda.synchronize()
    for t in dini.tensors():
        assert torch.all(t == 0.0)


DFIN_CASES = [
    # dtype, d, dv, chunk, n, gamma, ridge, normalize, with init
    (torch.float32, 32, 32, 16, 150, "per_head", 0.0, False, True),
    (torch.float32, 32, 16, 32, 97, "per_head", 0.2, False, True),
    (torch.bfloat16, 64, 64, 64, 150, "decay", 0.0, False, False),
    (torch.float32, 32, 32, 32, 120, "decay", 0.1, True, True),
    (torch.bfloat16, 128, 128, 128, 300, "decay", 1e-3, True, True),
    (torch.float32, 16, 64, 16, 70, None, 0.0, False, True),
    (torch.float32, 64, 32, 64, 45, "strong", 0.0, False, False),
]


@pytest.mark.parametrize("case", DFIN_CASES, ids=lambda c: f"{'bf16' if c[0] == torch.bfloat16 else 'f32'}"
                         f"-d{c[1]}dv{c[2]}w{c[3]}n{c[4]}-{c[5]}-l{c[6]}-r{int(c[7])}-init{int(c[8])}")
def test_backward_final_state_gradient(case):
    """A gradient flowing into the final state (dfinal): dq, dk, dv and dinit
    through hla_backward_chunked against the fp64 autograd oracle of
    sum <out, dout> + sum <final part, dfinal part>."""
    import types

    import oracle
    from oracle import backward as ob
    dtype, d, dv, chunk, n, gk, lam, norm, with_init = case
    B, H, n0 = 1, 2, 40
    q, k, v = inputs.qkv(B, H, n0 + n, d, dv, dtype, seed=101 + d + n)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.97] * H)
    elif gk == "per_head":
        g = inputs.gamma_list_fp32([0.95, 0.99])
    elif gk == "strong":
        g = inputs.gamma_list_fp32([0.3, 0.6])
    lam = inputs.ridge_fp32(lam)
    init = ref_init = None
    if with_init:
        _, _, st = oracle.forward(q[:, :, :n0], k[:, :, :n0], v[:, :, :n0], gamma=g, lam=lam)
        f32 = {name: torch.tensor(getattr(st, name), dtype=torch.float32) for name in ("S", "C", "m", "G", "h")}
        init = hla.State(*(f32[x].to(DEV) for x in ("S", "C", "m", "G", "h")))
        ref_init = types.SimpleNamespace(**f32)
    N = B * H
    shapes = {"S": (N, d, d), "C": (N, d, dv), "m": (N, d), "G": (N, d, dv), "h": (N, d)}
    dfin = {name: 0.1 * inputs.upstream(1, 1, 1, int(np.prod(shp)), seed=103 + i).reshape(shp)
            for i, (name, shp) in enumerate(shapes.items())}
    qs, ks, vs = (x[:, :, n0:].contiguous() for x in (q, k, v))
    dout = inputs.upstream(B, H, n, dv, seed=107)
    qg, kg, vg, dg = (x.to(DEV) for x in (qs, ks, vs, dout))
    dini = hla.State.empty(N, d, dv, DEV)
    dfin_dev = hla.State(*(dfin[x].to(DEV) for x in ("S", "C", "m", "G", "h")))
    got = hla.backward_chunked(qg, kg, vg, dg, gamma=g, ridge=lam, normalize=norm, chunk=chunk, init=init,
                               dinit=dini, dfinal=dfin_dev)
    torch.cuda.synchronize()
    *ref, rdini = ob.backward(qs, ks, vs, dout, g, lam, norm, ref_init, init_grad=True,
                              dfinal=types.SimpleNamespace(**dfin))
    tol = FTOL if fast_path(dtype, d, dv, chunk, gk, lam, norm) else GTOL
    check([x.cpu() for x in got], ref, tol=tol)
    _dinit_check(dini, rdini, tol)


@pytest.mark.parametrize("dtype,norm,lam", [(torch.float32, False, 0.0), (torch.bfloat16, True, 0.05)])
def test_backward_segments_chain_to_the_whole_sequence(dtype, norm, lam):
    """Sequence-sharded training on one GPU: segment A's final state (GPU
    forward) starts segment B; B's backward returns dinit, which A's backward
    takes as dfinal.  Together they give the whole sequence's gradients (fp64
    oracle over all tokens)."""
    from oracle import backward as ob
    B, H, na, nb, d, dv = 1, 2, 130, 90, 32, 32
    q, k, v = inputs.qkv(B, H, na + nb, d, dv, dtype, seed=111)
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = inputs.gamma_list_fp32([0.98, 0.995])
    lam = inputs.ridge_fp32(lam)
    dout = inputs.upstream(B, H, na + nb, dv, seed=113)
    qg, kg, vg, dg = (x.to(DEV) for x in (q, k, v, dout))
    sa = lambda x: x[:, :, :na].contiguous()
    sb = lambda x: x[:, :, na:].contiguous()
    _, _, stA = hla.forward_chunked(sa(qg), sa(kg), sa(vg), gamma=g, ridge=lam, normalize=norm, chunk=32,
                                    return_state=True)
    dB = hla.State.empty(B * H, d, dv, DEV)
    gB = hla.backward_chunked(sb(qg), sb(kg), sb(vg), sb(dg), gamma=g, ridge=lam, normalize=norm, chunk=32,
                              init=stA, dinit=dB)
    gA = hla.backward_chunked(sa(qg), sa(kg), sa(vg), sa(dg), gamma=g, ridge=lam, normalize=norm, chunk=32,
                              dfinal=dB)
    torch.cuda.synchronize()
    got = [torch.cat([a.cpu(), b.cpu()], dim=2) for a, b in zip(gA, gB)]
    ref = ob.backward(q, k, v, dout, g, lam, norm)
    check(got, ref)


@pytest.mark.parametrize("norm,lam", [(False, 0.0), (True, 0.05)])
def test_autograd_op_chains_segments(norm, lam):
    """hla.attention with a state: three segments chained through their
    states under one loss.backward() give the whole sequence's gradients
    (fp64 oracle), and a leaf initial state receives the oracle's dinit."""
    import types

    from oracle import backward as ob
    B, H, d, dv, cuts = 1, 2, 32, 32, (0, 70, 160, 230)
    n = cuts[-1]
    q, k, v = inputs.qkv(B, H, n, d, dv, torch.float32, seed=121)
    if norm:
        q, k = (x.abs().add(0.1) for x in (q, k))
    g = inputs.gamma_list_fp32([0.97, 0.99])
    lam = inputs.ridge_fp32(lam)
    dout = inputs.upstream(B, H, n, dv, seed=123)
    N = B * H
    ini = {"S": 0.05 * torch.eye(d).repeat(N, 1, 1), "C": 0.1 * inputs.upstream(1, 1, N * d, dv, seed=125).reshape(N, d, dv),
           "m": torch.full((N, d), 0.5), "G": torch.zeros(N, d, dv), "h": torch.zeros(N, d)}
    qg, kg, vg = (x.to(DEV).requires_grad_(True) for x in (q, k, v))
    st = hla.State(*(ini[x].to(DEV).requires_grad_(True) for x in ("S", "C", "m", "G", "h")))
    leaf = st
    loss = 0.0
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = lambda x: x[:, :, a:b].contiguous()
        out, st = hla.attention(sl(qg), sl(kg), sl(vg), gamma=g, ridge=lam, normalize=norm, chunk=32, init=st)
        loss = loss + (out * sl(dout.to(DEV))).sum()
    loss.backward()
    torch.cuda.synchronize()
    *ref, rdini = ob.backward(q, k, v, dout, g, lam, norm, types.SimpleNamespace(**ini), init_grad=True)
    check([x.grad.cpu() for x in (qg, kg, vg)], ref)
    # the op reads S through its symmetric part, so the leaf S receives the
    # symmetric part of the oracle's gradient (which counts every entry of S
    # as its own variable)
    rS = np.asarray(rdini["S"])
    rdini = dict(rdini, S=0.5 * (rS + rS.transpose(0, 2, 1)))
    _dinit_check(types.SimpleNamespace(**{x: getattr(leaf, x).grad for x in ("S", "C", "m", "G", "h")}), rdini)


def test_autograd_op_symmetrises_the_initial_key_moment():
    """A leaf initial S that is not symmetric (as after an optimizer step)
    enters through its symmetric part: the op's output equals the forward
    from (S + S^T)/2, the gradient S receives has no antisymmetric part, it
    equals the oracle's dinit symmetrised, and one SGD step from a symmetric
    S keeps S symmetric."""
    import types

    from oracle import backward as ob
    B, H, n, d, dv = 1, 2, 90, 32, 32
    q, k, v = inputs.qkv(B, H, n, d, dv, torch.float32, seed=131)
    g = inputs.gamma_list_fp32([0.97, 0.99])
    dout = inputs.upstream(B, H, n, dv, seed=133)
    N = B * H
    gen = torch.Generator().manual_seed(135)
    a = 0.05 * torch.randn(N, d, d, generator=gen)
    ini = {"S": a + 0.01 * torch.eye(d),  # not symmetric
           "C": 0.1 * torch.randn(N, d, dv, generator=gen), "m": 0.1 * torch.randn(N, d, generator=gen),
           "G": torch.zeros(N, d, dv), "h": torch.zeros(N, d)}
    Ssym = 0.5 * (ini["S"] + ini["S"].transpose(1, 2))  # the same fp32 operations as the op's
    qg, kg, vg = (x.to(DEV) for x in (q, k, v))
    st = hla.State(*(ini[x].to(DEV).requires_grad_(True) for x in ("S", "C", "m", "G", "h")))
    out, _ = hla.attention(qg, kg, vg, gamma=g, chunk=32, init=st)
    (out * dout.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    ref_out, _, _ = hla.forward_chunked(qg, kg, vg, gamma=g, chunk=32,
                                        init=hla.State(Ssym.to(DEV), *(ini[x].to(DEV) for x in ("C", "m", "G", "h"))))
    assert torch.equal(out.detach(), ref_out)
    dS = st.S.grad.cpu().double()
    assert float((dS - dS.transpose(1, 2)).abs().max()) == 0.0
    sym = dict(ini, S=Ssym)
    *_, rdini = ob.backward(q, k, v, dout, g, 0.0, False, types.SimpleNamespace(**sym), init_grad=True)
    rS = np.asarray(rdini["S"], dtype=np.float64)
    rS = 0.5 * (rS + rS.transpose(0, 2, 1))
    e = slab_err(dS, rS)
    print(f"symmetrised dS slab error {e:.3e}")
    assert e <= GTOL
    # one SGD step from the symmetric S: S stays exactly symmetric
    S1 = (Ssym.to(DEV) - 0.1 * st.S.grad).cpu()
    assert torch.equal(S1, S1.transpose(1, 2))

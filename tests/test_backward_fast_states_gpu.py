"""GPU parity of the one-launch backward with states against the fp64
autograd oracle: an initial state, a gradient flowing into the final state,
and the gradient of the initial state, each present or not.

bf16 calls with d = dv = 64, chunk 64, no ridge or ratio and every decay >=
0.75 take the first-order maps with carries in and out (the identity is
pinned on the CPU in tests/test_backward_algebra.py; Higher-order Linear
Attention, paperlayer.ai summary sec. 4: the reverse-mode scan, whose state
is what a sequence split hands across).  As for the plain one-launch
backward, products with bf16 pairs put the gate at the slab error FTOL =
1e-4; each part of the initial state's gradient is gated at the same level
against its largest entry.  The control block shows the expected launch
count and that no wait gave up.
"""
import sys
import types

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FTOL = 1e-4
BF = torch.bfloat16
PARTS = ("S", "C", "m", "G", "h")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def gammas(kind, H):
    if kind == "decay":
        return inputs.gamma_list_fp32([0.97] * H)
    if kind == "per_head":
        return inputs.gamma_list_fp32([(0.75, 0.9, 0.99, 1.0, 0.999, 0.8, 0.95, 0.97)[h % 8] for h in range(H)])
    return None


def make_state(N, seed, symmetric):
    """A state off the method's own: every part i.i.d. (S made symmetric or left as is)."""
    shapes = {"S": (N, 64, 64), "C": (N, 64, 64), "m": (N, 64), "G": (N, 64, 64), "h": (N, 64)}
    st = {name: inputs.upstream(1, 1, 1, int(np.prod(shp)), seed=seed + i).reshape(shp)
          for i, (name, shp) in enumerate(shapes.items())}
    if symmetric:
        st["S"] = 0.5 * (st["S"] + st["S"].transpose(-1, -2))
    return st


def one_pass(B, H, n):
    # segments of up to four 64-token chunks, about 256 per map
    BH, nc = B * H, -(-n // 64)
    target = -(-256 // BH)
    L = min(max(-(-nc // target), 1), 4)
    P = -(-nc // L)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return BH * P <= cus and 2 * BH <= 240


def expected_launches(B, H, n, with_dfin):
    # U (with the C_n map), W, then two pairs of maps; one after the other when looped
    return 4 if one_pass(B, H, n) else (2 if with_dfin else 1) + 1 + 2 + 2


def dev_state(st):
    return hla.State(*(st[x].to(DEV).contiguous() for x in PARTS))


def run(q, k, v, dout, g, init, dfin, with_dinit, ws=None):
    B, H, n, _ = q.shape
    N = B * H
    need = hla.backward_workspace_size(B, H, n, 64, 64, chunk=64, gamma=g)
    if ws is None:  # arbitrary contents: the call clears what it needs
        ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    dini = None
    if with_dinit:
        dini = hla.State.empty(N, 64, 64, DEV)
        for t in dini.tensors():
            t.fill_(float("nan"))
    got = hla.backward_chunked(*(x.to(DEV).contiguous() for x in (q, k, v, dout)), gamma=g, chunk=64, workspace=ws,
                               init=None if init is None else dev_state(init), dinit=dini,
                               dfinal=None if dfin is None else dev_state(dfin))
    torch.cuda.synchronize()
    words = ws[:16].view(torch.int32).cpu().tolist()
    want = expected_launches(B, H, n, dfin is not None)
    assert words[2] == want and words[3] == 0, f"the one-launch backward did not run cleanly ({want} launches): {words}"
    if dini is not None:
        assert torch.all(dini.rho == 0.0)
    return [x.cpu() for x in got], dini


def check(got, ref):
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        e = slab_err(x, r, lead=2)
        print(f"{name}: slab {e:.3e} row {row_err(x, r):.3e}")
        assert e <= FTOL, f"{name}: slab error {e:.3e} > {FTOL:.0e}"


def check_dinit(got, ref):
    """Each part's max abs error over that part's largest entry, floored at
    1e-3 of the largest entry over all parts."""
    top = max(float(np.abs(np.asarray(ref[p])).max()) for p in PARTS)
    for part in PARTS:
        x = got[part].double().numpy()
        r = np.asarray(ref[part]).reshape(x.shape)
        scale = max(float(np.abs(r).max()), 1e-3 * top, 1e-30)
        e = float(np.abs(x - r).max()) / scale
        print(f"dinit.{part}: {e:.3e}")
        assert e <= FTOL, f"dinit.{part}: error {e:.3e} > {FTOL:.0e}"


def oracle_check(q, k, v, dout, g, init, dfin, got, dini):
    from oracle import backward as ob
    B, H = q.shape[:2]
    heads = ((0, 0), (B // 2, H // 2), (B - 1, H - 1)) if B * H > 8 else None
    ns = lambda st, i: None if st is None else types.SimpleNamespace(  # noqa: E731
        **{x: st[x][i] for x in PARTS})
    groups = [(slice(0, B), slice(0, H), slice(0, B * H), g)] if heads is None else \
        [(slice(b, b + 1), slice(h, h + 1), slice(b * H + h, b * H + h + 1), None if g is None else [g[h]])
         for b, h in heads]
    for bs, hs, ns_, gg in groups:
        sl = lambda x: x[bs, hs]  # noqa: E731
        res = ob.backward(sl(q), sl(k), sl(v), sl(dout), gg, 0.0, False, ns(init, ns_), init_grad=dini is not None,
                          dfinal=ns(dfin, ns_))
        check([sl(x) for x in got], res[:3])
        if dini is not None:
            check_dinit({x: getattr(dini, x).cpu()[ns_] for x in PARTS}, res[3])


CASES = [  # B, H, n, gamma, init, dfinal, dinit, S symmetric
    (4, 8, 2048, "per_head", True, True, True, True),      # the bench shape (three sampled heads)
    (2, 3, 64 * 13 + 37, "per_head", True, True, True, False),  # ragged one-chunk segments, S not symmetric
    (4, 8, 64 * 32 + 37, "decay", True, True, True, True),  # a looped grid: the maps one after the other
    (1, 2, 50, "per_head", True, True, True, False),        # one segment
    (2, 1, 1, None, True, True, True, True),                # one token
    (1, 2, 150, "decay", False, True, True, True),          # no initial state
    (1, 2, 150, "per_head", True, False, True, True),       # no final-state gradient
    (1, 2, 150, None, True, False, False, True),            # an initial state only
    (1, 2, 150, "decay", False, True, False, True),         # a final-state gradient only
    (1, 2, 150, "per_head", False, False, True, True),      # the zero state's gradient only
    (2, 64, 100, "decay", True, True, True, False),         # more heads than two maps' ticket counters
]


@pytest.mark.parametrize("B,H,n,gk,with_init,with_dfin,with_dinit,sym", CASES)
def test_fast_backward_with_states(B, H, n, gk, with_init, with_dfin, with_dinit, sym):
    N = B * H
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=2100 + n + H)
    dout = inputs.upstream(B, H, n, 64, seed=2101 + n)
    g = gammas(gk, H)
    init = make_state(N, 2200 + n, sym) if with_init else None
    dfin = {x: 0.1 * t for x, t in make_state(N, 2300 + n, False).items()} if with_dfin else None
    got, dini = run(q, k, v, dout, g, init, dfin, with_dinit)
    oracle_check(q, k, v, dout, g, init, dfin, got, dini)


def test_fast_backward_with_states_deterministic_and_reusable():
    """Bit-identical gradients and initial-state gradient on a reused workspace."""
    B, H, n = 2, 4, 700
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=2400)
    dout = inputs.upstream(B, H, n, 64, seed=2401)
    g = gammas("per_head", H)
    init, dfin = make_state(B * H, 2402, True), make_state(B * H, 2410, False)
    need = hla.backward_workspace_size(B, H, n, 64, 64, chunk=64, gamma=g)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    a, da = run(q, k, v, dout, g, init, dfin, True, ws)
    b, db = run(q, k, v, dout, g, init, dfin, True, ws)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip(da.tensors(), db.tensors()):
        assert torch.equal(x, y)


def test_fast_backward_segments_chain_to_the_whole_sequence():
    """Sequence-sharded training: segment A's final state (GPU forward) starts
    segment B; B's backward returns dinit, which A's backward takes as
    dfinal.  Together they give the whole sequence's gradients (fp64 oracle),
    every call on the one-launch paths."""
    from oracle import backward as ob
    B, H, nA, nB = 2, 4, 700, 555
    n = nA + nB
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=2500)
    dout = inputs.upstream(B, H, n, 64, seed=2501)
    g = gammas("per_head", H)
    qg, kg, vg, dg = (x.to(DEV).contiguous() for x in (q, k, v, dout))
    A, Bs = slice(0, nA), slice(nA, n)
    sl = lambda x, s: x[:, :, s].contiguous()  # noqa: E731
    _, _, stA = hla.forward_chunked(sl(qg, A), sl(kg, A), sl(vg, A), gamma=g, chunk=64, return_state=True)
    dB = hla.State.empty(B * H, 64, 64, DEV)
    gB = hla.backward_chunked(sl(qg, Bs), sl(kg, Bs), sl(vg, Bs), sl(dg, Bs), gamma=g, chunk=64, init=stA, dinit=dB)
    gA = hla.backward_chunked(sl(qg, A), sl(kg, A), sl(vg, A), sl(dg, A), gamma=g, chunk=64, dfinal=dB)
    torch.cuda.synchronize()
    got = [torch.cat([a.cpu(), b.cpu()], dim=2) for a, b in zip(gA, gB)]
    check(got, ob.backward(q, k, v, dout, g))


def test_fast_backward_with_states_soak_bitwise():
    """50 calls of the shard backward at the bench shape (initial state,
    dfinal in, dinit out) on one workspace, each compared bitwise with the
    first; the loop stops at the first mismatch."""
    B, H, n = 4, 8, 2048
    N = B * H
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, 64, 64, BF, seed=2600))
    dout = inputs.upstream(B, H, n, 64, seed=2601).to(DEV)
    g = gammas("per_head", H)
    init, dfin = dev_state(make_state(N, 2602, True)), dev_state(make_state(N, 2610, False))
    ws = torch.empty(hla.backward_workspace_size(B, H, n, 64, 64, chunk=64, gamma=g), dtype=torch.uint8, device=DEV)

    def call():
        dini = hla.State.empty(N, 64, 64, DEV)
        got = hla.backward_chunked(q, k, v, dout, gamma=g, chunk=64, workspace=ws, init=init, dfinal=dfin, dinit=dini)
        return list(got) + [t for t in dini.tensors() if t is not None]

    ref = [x.clone() for x in call()]
    for i in range(50):
        for j, (x, r) in enumerate(zip(call(), ref)):
            assert torch.equal(x, r), f"call {i}: output {j} differs"
    words = ws[:16].view(torch.int32).cpu().tolist()
    assert words[3] == 0, words

"""GPU robustness of the library: every output written, results that do not
depend on what else runs on the device, and failures that are never silent.

* NaN-poisoned outputs and states: every path (both one-launch forwards, the
  generic forward with a final state, decode, compose) overwrites every
  element it owns.
* Two forward calls on two streams whose grids cannot be resident together
  (each one-launch grid holds a workgroup per CU) give the same bits as the
  same calls made one after the other.
* Bounded soaks of repeated calls (the bench shape, the d = 128 kernel, the
  d = 64 kernel with states, AHLA's chained map), compared bitwise, stop at
  their first mismatch.
* A wait that gives up (forced from the host through control word 4) turns
  the outputs that depend on it into NaN, never into wrong numbers.
* Compose at its full size (4096 pairs, d = dv = 128) against the oracle, and
  the GPU forward's final state on the 512-token decode prefix (sampled heads)
  against the oracle, followed by a decode step from that GPU state.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
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


def ctrl_words(ws):
    return ws[:16].view(torch.int32).cpu().tolist()


def nan_state(N, d, dv):
    st = hla.State.empty(N, d, dv, DEV)
    for t in st.tensors():
        t.fill_(float("nan"))
    return st


def check_state(got: hla.State, ref, tol, names=("S", "C", "m", "G", "h")):
    sc, sm = naive_scales(ref.S, ref.C, ref.m)
    for k in names:
        scale = sc if k == "G" else sm if k == "h" else None
        e = slab_err(getattr(got, k).cpu(), getattr(ref, k), scale=scale)
        print(f"state {k}: slab error {e:.3e}")
        assert e <= tol, f"state {k}: slab error {e:.3e} > {tol:.0e}"


# ---------------------------------------------------------------------------
# every output element is written

def test_fused128_writes_every_output():
    B, H, n = 1, 16, 4096 + 37
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, 128, 128, torch.bfloat16, seed=61))
    g = inputs.gamma_list_fp32([0.999] * H)
    out = torch.full((B, H, n, 128), float("nan"), device=DEV)
    ws = torch.zeros(hla.workspace_size(B, H, n, 128, 128), dtype=torch.uint8, device=DEV)
    hla.forward_chunked(q, k, v, gamma=g, out=out, workspace=ws)
    ref, _, _ = hla.forward_chunked(q, k, v, gamma=g)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[2] == 1, "the one-launch d=128 path did not run"
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("d,dtype,norm", [(64, torch.bfloat16, True), (64, torch.float32, True),
                                          (32, torch.float32, False), (128, torch.bfloat16, False)])
def test_forward_with_state_writes_every_output(d, dtype, norm):
    """bf16 d = 64: the one-launch kernel's state variant; otherwise the generic kernels."""
    B, H, n = 2, 3, 301
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, d, dtype, seed=62 + d))
    if norm:
        q, k = (x.float().abs().add(0.1).to(dtype) for x in (q, k))
    g = inputs.gamma_list_fp32([0.97, 0.999, 1.0])
    out = torch.full((B, H, n, d), float("nan"), device=DEV)
    den = torch.full((B, H, n), float("nan"), device=DEV)
    fin = nan_state(B * H, d, d)
    hla.forward_chunked(q, k, v, gamma=g, ridge=1e-3, normalize=norm, out=out, den=den, final_state=fin)
    o2, d2, f2 = hla.forward_chunked(q, k, v, gamma=g, ridge=1e-3, normalize=norm, return_den=True,
                                     return_state=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(den).all()
    assert torch.equal(out, o2) and torch.equal(den, d2)
    for a, b in zip(fin.tensors(), f2.tensors()):
        assert torch.isfinite(a).all()
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,dv", [(128, 128), (64, 32)])
def test_decode_writes_every_output(d, dv):
    B, H = 16, 16
    st = inputs.random_state_fp32(B * H, d, dv, 63, scale=0.1)
    state = hla.State(*(t.to(DEV) for t in st))
    q, k, v = (x.to(DEV) for x in inputs.decode_inputs(B, H, 0, d, dv, torch.bfloat16, seed=64)[1])
    out = torch.full((B, H, dv), float("nan"), device=DEV)
    den = torch.full((B, H), float("nan"), device=DEV)
    hla.decode_step(q, k, v, state, out=out, den=den)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(den).all()
    for t in state.tensors():
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("d,dv", [(128, 128), (16, 64)])
def test_compose_writes_every_output(d, dv):
    N = 300
    a = hla.State(*(t.to(DEV) for t in inputs.random_state_fp32(N, d, dv, 65)))
    b = hla.State(*(t.to(DEV) for t in inputs.random_state_fp32(N, d, dv, 66)))
    r = nan_state(N, d, dv)
    hla.state_compose(a, b, r)
    r2 = hla.state_compose(a, b)
    torch.cuda.synchronize()
    for x, y in zip(r.tensors(), r2.tensors()):
        assert torch.isfinite(x).all()
        assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# results independent of what else runs

def _headline_inputs(seed):
    w = inputs.FWD_D64
    return [x.to(DEV) for x in inputs.workload_qkv(w, seed)]


def test_two_streams_whose_grids_cannot_both_be_resident():
    """Each one-launch grid takes a workgroup per CU (its LDS fills the CU),
    so two of them launched on two streams cannot all be resident at once.
    Pairs: the bench shape with itself, with the looped ratio shape (64
    heads, more segments than CUs) and with the d = 128 kernel.  Both
    kernels take segments by ticket, so a wait only ever targets a running
    workgroup."""
    qa, ka, va = _headline_inputs(71)
    r = inputs.RATIO_DECAY_D64
    qb, kb, vb = (x.to(DEV) for x in inputs.qkv(r.B, r.H, 2048, 64, 64, torch.bfloat16, seed=72))
    qc, kc, vc = (x.to(DEV) for x in inputs.qkv(1, 16, 8192, 128, 128, torch.bfloat16, seed=73))
    gc = inputs.gamma_list_fp32([0.999] * 16)
    calls = {
        "a": lambda ws, out: hla.forward_chunked(qa, ka, va, chunk=64, workspace=ws, out=out),
        "b": lambda ws, out: hla.forward_chunked(qb, kb, vb, gamma=r.gamma, ridge=r.ridge, normalize=True,
                                                 chunk=64, workspace=ws, out=out),
        "c": lambda ws, out: hla.forward_chunked(qc, kc, vc, gamma=gc, workspace=ws, out=out),
    }
    shapes = {"a": (4, 8, 2048, 64), "b": (8, 8, 2048, 64), "c": (1, 16, 8192, 128)}
    refs = {}
    for key, f in calls.items():
        B, H, n, d = shapes[key]
        ws = torch.zeros(hla.workspace_size(B, H, n, d, d, chunk=64 if d == 64 else 0), dtype=torch.uint8,
                         device=DEV)
        refs[key] = f(ws, torch.empty(B, H, n, d, device=DEV))[0].clone()
        torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for first, second in (("a", "a"), ("a", "b"), ("b", "a"), ("c", "a"), ("a", "c")):
        for rep in range(5):
            wss, outs = [], []
            for key in (first, second):
                B, H, n, d = shapes[key]
                wss.append(torch.zeros(hla.workspace_size(B, H, n, d, d, chunk=64 if d == 64 else 0),
                                       dtype=torch.uint8, device=DEV))
                outs.append(torch.empty(B, H, n, d, device=DEV))
            torch.cuda.synchronize()
            with torch.cuda.stream(s1):
                calls[first](wss[0], outs[0])
            with torch.cuda.stream(s2):
                calls[second](wss[1], outs[1])
            torch.cuda.synchronize()
            for key, ws, out in zip((first, second), wss, outs):
                assert ctrl_words(ws)[3] == 0, (first, second, rep)
                assert torch.equal(out, refs[key]), (first, second, rep, key)


def test_soak_bench_shape_bitwise():
    """300 calls of the bench shape on one workspace, each compared bitwise
    with the first; the loop stops at the first mismatch."""
    q, k, v = _headline_inputs(74)
    w = inputs.FWD_D64
    ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, 64, 64, chunk=64), dtype=torch.uint8, device=DEV)
    ref, _, _ = hla.forward_chunked(q, k, v, chunk=64, workspace=ws)
    ref = ref.clone()
    out = torch.empty_like(ref)
    for i in range(300):
        hla.forward_chunked(q, k, v, chunk=64, workspace=ws, out=out)
        assert torch.equal(out, ref), f"call {i} differs"
    assert ctrl_words(ws)[3] == 0


def _soak(call, reps):
    ref = [x.clone() for x in call()]
    for i in range(reps):
        for j, (x, r) in enumerate(zip(call(), ref)):
            assert torch.equal(x, r), f"call {i}: output {j} differs"


def test_soak_other_one_launch_kernels_bitwise():
    """Bounded soaks, compared bitwise with the first call and stopping at the
    first mismatch, of the other kernels that hand sums between workgroups:
    the d = 128 forward (16 segments per head), the d = 64 forward with
    initial and final states, and AHLA's chained map (two hand-offs per
    segment)."""
    g16 = inputs.gamma_list_fp32([0.999] * 16)
    q, k, v = (x.to(DEV) for x in inputs.qkv(1, 16, 16384, 128, 128, torch.bfloat16, seed=75))
    ws = torch.zeros(hla.workspace_size(1, 16, 16384, 128, 128, gamma=g16), dtype=torch.uint8, device=DEV)
    _soak(lambda: [hla.forward_chunked(q, k, v, gamma=g16, workspace=ws)[0]], 30)
    assert ctrl_words(ws)[3] == 0

    g8 = inputs.gamma_list_fp32([0.97, 0.9, 1.0, 0.99, 0.75, 0.8, 0.95, 0.999])
    q, k, v = (x.to(DEV) for x in inputs.qkv(4, 8, 2048, 64, 64, torch.bfloat16, seed=76))
    init = hla.State(*(t.to(DEV).contiguous() for t in inputs.random_state_fp32(32, 64, 64, seed=77, scale=0.1)))
    ws = torch.zeros(hla.workspace_size(4, 8, 2048, 64, 64, chunk=64, gamma=g8), dtype=torch.uint8, device=DEV)

    def with_states():
        out, _, fin = hla.forward_chunked(q, k, v, gamma=g8, chunk=64, init=init, return_state=True, workspace=ws)
        return [out] + [t for t in fin.tensors() if t is not None]

    _soak(with_states, 30)
    assert ctrl_words(ws)[3] == 0
    _soak(lambda: [hla.ahla_forward(q, k, v, gamma=g8, chunk=64)[0]], 30)


@pytest.mark.parametrize("d,B,H,n", [(64, 4, 8, 2048), (128, 1, 16, 4096)])
def test_give_up_makes_dependent_outputs_nan(d, B, H, n):
    """With control word 4 = -1 the waits give up (the d = 128 kernel without
    polling, the d = 64 kernel after one unsuccessful poll).  Every output row
    is then either the same bits as a normal call or holds a NaN, the first
    segment of each head (it waits on nothing) is exact, and a launch whose
    waits gave up has NaN rows."""
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, d, torch.bfloat16, seed=76))
    ref, _, _ = hla.forward_chunked(q, k, v)
    ws = torch.zeros(hla.workspace_size(B, H, n, d, d), dtype=torch.uint8, device=DEV)
    ws[:64].view(torch.int32)[4] = -1
    out, _, _ = hla.forward_chunked(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    w = ctrl_words(ws)
    assert w[2] == 1, w
    rows_nan = torch.isnan(out).any(dim=-1)
    rows_same = (out == ref).all(dim=-1)
    assert bool((rows_nan | rows_same).all()), "a row is neither NaN nor the normal result"
    assert bool(rows_same[:, :, :64].all()), "the first chunk of a head waits on nothing"
    if w[3] > 0:
        assert bool(rows_nan.any())
    if d == 128:
        assert w[3] > 0 and bool(rows_nan.any())
    else:
        assert bool(rows_nan.any()) == (w[3] > 0)


# ---------------------------------------------------------------------------
# compose at full size; the prefix's final state and decode from it

def _compose_oracle_threaded(a, b, threads=16):
    import oracle
    N = a.S.shape[0]
    bounds = np.linspace(0, N, threads + 1).astype(int)

    def part(i):
        lo, hi = bounds[i], bounds[i + 1]
        sl = lambda s: oracle.State(*(np.ascontiguousarray(x[lo:hi]) for x in s.flat()))
        return oracle.compose(sl(a), sl(b))

    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(part, range(threads)))
    return oracle.State(*(np.concatenate([getattr(p, f) for p in parts]) for f in ("S", "C", "m", "G", "h", "rho")))


def test_compose_full_size_4096_pairs_d128():
    import oracle
    N, d, dv = 4096, 128, 128
    a = inputs.random_state_fp32(N, d, dv, 81, scale=0.1)
    b = inputs.random_state_fp32(N, d, dv, 82, scale=0.1)
    r = hla.state_compose(hla.State(*(t.to(DEV) for t in a)), hla.State(*(t.to(DEV) for t in b)))
    torch.cuda.synchronize()
    ref = _compose_oracle_threaded(oracle.State(*(t.double().numpy() for t in a)),
                                   oracle.State(*(t.double().numpy() for t in b)))
    check_state(r, ref, 1e-5)
    assert np.allclose(r.rho.cpu().double().numpy(), np.asarray(ref.rho, np.float32), rtol=1e-6)


def test_prefix_final_state_then_decode_sampled_heads():
    """The decode workload's 512-token prefix (B256 x H16 states, d = dv =
    128, bf16) folded by the GPU forward into final states; sampled batch
    rows are checked against the oracle's fold, then one decode step runs
    from the GPU states and its outputs are checked against the oracle's
    decode from its own states."""
    import oracle
    w = inputs.DECODE_D128
    (q, k, v), (q1, k1, v1) = inputs.decode_inputs(w.B, w.H, w.n, w.d, w.dv, torch.bfloat16, 1004)
    _, _, st = hla.forward_chunked(q.to(DEV), k.to(DEV), v.to(DEV), return_state=True)
    rows = [0, 97, 255]
    idx = torch.tensor([b * w.H + h for b in rows for h in range(w.H)])
    got = hla.State(*(t.cpu()[idx] for t in st.tensors()))  # before the decode step updates st in place
    out, _ = hla.decode_step(q1.to(DEV), k1.to(DEV), v1.to(DEV), st)
    torch.cuda.synchronize()
    sl = lambda x: x[rows].contiguous()
    _, _, rst = oracle.forward(sl(q), sl(k), sl(v))
    tol = TOL[torch.bfloat16]
    check_state(got, rst, tol)
    r_out, _, _ = oracle.decode(rst, sl(q1), sl(k1), sl(v1))
    e = row_err(out.cpu()[rows], r_out)
    print(f"decode-from-GPU-prefix row error {e:.3e}")
    assert e <= tol

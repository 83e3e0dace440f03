"""GPU parity of the one-launch backward against the fp64 autograd oracle.

bf16 calls with d = dv = 64, chunk 64, no ridge, ratio or states and every
decay >= 0.75 compute the gradient of the plain second-order numerator as
seven masked first-order maps, forward and reverse in time (the identity is
pinned on the CPU in tests/test_backward_algebra.py; Higher-order Linear
Attention, paperlayer.ai summary sec. 4: the reverse-mode scan).  dout, and
the intermediates U = S q and W, are carried as bf16 pairs (hi = bf16(x),
lo = bf16(x - hi)), and each product with a pair drops lo * lo, about 2^-16
of the product; so the gate is the slab error FTOL = 1e-4 rather than the
chunked fp32 backward's 1e-5.  The control block at the start of the
workspace counts the launches (the call clears it itself: the backward
workspace needs no initialisation) and shows that no wait gave up: W's map,
then two grids of two independent maps each, or, where a map's segments do
not fit one pass of the device, those four maps one after the other.
"""
import sys

import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FTOL = 1e-4
BF = torch.bfloat16


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


def expected_launches(B, H, n):
    # segments of up to four 64-token chunks, about 256 per map
    BH, nc = B * H, -(-n // 64)
    target = -(-256 // BH)
    L = min(max(-(-nc // target), 1), 4)
    P = -(-nc // L)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 3 if BH * P <= cus and 2 * BH <= 240 else 5


def fast_backward(q, k, v, dout, g, ws=None):
    B, H, n, d = q.shape
    qg, kg, vg, dg = (x.to(DEV).contiguous() for x in (q, k, v, dout))
    need = hla.backward_workspace_size(B, H, n, d, d, chunk=64, gamma=g)
    if ws is None:  # arbitrary contents: the call clears what it needs
        ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    out = hla.backward_chunked(qg, kg, vg, dg, gamma=g, chunk=64, workspace=ws)
    torch.cuda.synchronize()
    words = ws[:16].view(torch.int32).cpu().tolist()
    want = expected_launches(B, H, n)
    assert words[2] == want and words[3] == 0, f"the one-launch backward did not run cleanly ({want} launches): {words}"
    return [x.cpu() for x in out]


def check(got, ref):
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        e = slab_err(x, r, lead=2)
        print(f"{name}: slab {e:.3e} row {row_err(x, r):.3e}")
        assert e <= FTOL, f"{name}: slab error {e:.3e} > {FTOL:.0e}"


CASES = [  # B, H, n, gamma: one segment of four chunks per workgroup at the headline
    (4, 8, 2048, None), (2, 3, 64 * 13 + 37, "per_head"),  # shape; ragged one-chunk segments;
    (4, 8, 64 * 32 + 37, "decay"), (1, 2, 50, "per_head"), (2, 1, 1, None),  # a looped grid; one segment; one token
    (2, 64, 100, "per_head")]  # more heads than two maps' ticket counters: the pairs launch one after the other


@pytest.mark.parametrize("B,H,n,gk", CASES)
def test_fast_backward_matches_oracle(B, H, n, gk):
    from oracle import backward as ob
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=1800 + n + H)
    dout = inputs.upstream(B, H, n, 64, seed=1801 + n)
    g = gammas(gk, H)
    got = fast_backward(q, k, v, dout, g)
    if B * H > 8:  # the oracle on three sampled heads (heads are independent)
        for b, h in ((0, 0), (B // 2, H // 2), (B - 1, H - 1)):
            sl = lambda x: x[b:b + 1, h:h + 1]  # noqa: E731
            gh = None if g is None else [g[h]]
            check([sl(x) for x in got], ob.backward(sl(q), sl(k), sl(v), sl(dout), gh))
    else:
        check(got, ob.backward(q, k, v, dout, g))


def test_fast_backward_matches_the_chunked_backward():
    """The same inputs widened exactly to fp32 take the chunked fp32 backward."""
    B, H, n = 2, 4, 700
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=1900)
    dout = inputs.upstream(B, H, n, 64, seed=1901)
    g = gammas("per_head", H)
    fast = fast_backward(q, k, v, dout, g)
    ref = hla.backward_chunked(*(x.float().to(DEV) for x in (q, k, v)), dout.to(DEV), gamma=g, chunk=64)
    torch.cuda.synchronize()
    for x, r in zip(fast, ref):
        assert slab_err(x, r.cpu(), lead=2) <= FTOL


def test_fast_backward_deterministic_causal_and_reusable():
    """Bit-identical on a reused workspace; an upstream gradient zero after
    token t gives exactly zero gradients after t (every map there sums only
    zero terms) and nonzero ones before."""
    B, H, n = 1, 2, 300
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=1950)
    dout = inputs.upstream(B, H, n, 64, seed=1951)
    g = gammas("decay", H)
    need = hla.backward_workspace_size(B, H, n, 64, 64, chunk=64, gamma=g)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    a = fast_backward(q, k, v, dout, g, ws)
    b = fast_backward(q, k, v, dout, g, ws)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    t = 130
    d2 = dout.clone()
    d2[:, :, t + 1:] = 0
    c = fast_backward(q, k, v, d2, g, ws)
    for x in c:
        assert torch.count_nonzero(x[:, :, t + 1:]) == 0
        assert torch.count_nonzero(x[:, :, :t + 1]) > 0


def test_fast_backward_soak_bitwise():
    """100 calls of the bench shape (B4 H8 n2048, decay per head) on one
    workspace, each compared bitwise with the first; the loop stops at the
    first mismatch.  Every call hands segment sums between workgroups in each
    of its maps, so a lost or early hand-off would show as a difference."""
    B, H, n = 4, 8, 2048
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, 64, 64, BF, seed=1990))
    dout = inputs.upstream(B, H, n, 64, seed=1991).to(DEV)
    g = gammas("per_head", H)
    ws = torch.empty(hla.backward_workspace_size(B, H, n, 64, 64, chunk=64, gamma=g), dtype=torch.uint8, device=DEV)
    ref = [x.clone() for x in hla.backward_chunked(q, k, v, dout, gamma=g, chunk=64, workspace=ws)]
    for i in range(100):
        got = hla.backward_chunked(q, k, v, dout, gamma=g, chunk=64, workspace=ws)
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(x, r), f"call {i}: {name} differs"
    words = ws[:16].view(torch.int32).cpu().tolist()
    assert words[3] == 0, words

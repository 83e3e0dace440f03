"""GPU parity of the one-launch d = 128 forward when it takes an initial
state and/or returns a final state, against the fp64 oracle.

bf16, d = dv = 128, plain numerator, every decay >= 0.75: the kernel's
state variant.  The initial state enters the carries of every segment; for
a final state every segment also sums its value moment, query sum and y
increment in its first walk and publishes them with its X increment, and
the last segment of each head forms (S, C, m, G, h, rho).  Cases: several
segments per head (one-pass grid), ragged tails, one segment per head
(which then walks twice), decay per head, continuation across a split, an
initial state that no prefix produces, composition of segment states, and
the failure path forced from the host.  Control word 2 (launch count)
shows that the one-launch kernel ran, word 3 that no wait gave up.
Masked second-order HLA: Higher-order Linear Attention (paperlayer.ai
summary), sec. 4 (carry-in prefixes of the chunk scan) and sec. 4.2.
"""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import TOL, naive_scales, row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF = torch.bfloat16
D = 128


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def ctrl_words(ws):
    return ws[:16].view(torch.int32).cpu().tolist()


def gammas(kind, H):
    if kind == "decay":
        return inputs.gamma_list_fp32([0.999] * H)
    if kind == "per_head":
        return inputs.gamma_list_fp32([(0.75, 0.9, 0.99, 1.0, 0.999, 0.8, 0.95, 0.97)[h % 8] for h in range(H)])
    return None


def fast(q, k, v, *, gamma=None, init=None, state=True, ws=None):
    B, H, n, d = q.shape
    qg, kg, vg = (x.to(DEV).contiguous() for x in (q, k, v))
    if ws is None:
        ws = torch.zeros(hla.workspace_size(B, H, n, d, d), dtype=torch.uint8, device=DEV)
    before = ctrl_words(ws)[2]
    out, _, fin = hla.forward_chunked(qg, kg, vg, gamma=gamma, init=init, return_state=state, workspace=ws)
    torch.cuda.synchronize()
    w = ctrl_words(ws)
    assert w[2] == before + 1, f"the one-launch path did not run: {w}"
    assert w[3] == 0, f"a wait gave up: {w}"
    return out, fin


def check_state(gpu, ref, tol):
    g = {k: getattr(gpu, k).cpu().double().numpy() for k in ("S", "C", "m", "G", "h", "rho")}
    sc, sm = naive_scales(ref.S, ref.C, ref.m)
    for k in ("S", "C", "m", "G", "h"):
        scale = sc if k == "G" else sm if k == "h" else None
        e = slab_err(g[k], getattr(ref, k), scale=scale)
        print(f"state {k}: slab error {e:.3e}")
        assert e <= tol, f"state {k}: slab error {e:.3e} > {tol:.0e}"
    ref_rho = np.asarray(ref.rho, dtype=np.float32).astype(np.float64)
    assert np.allclose(g["rho"], ref_rho, rtol=2e-5, atol=1.2e-38), "rho"
    S = gpu.S.cpu()
    assert torch.equal(S, S.transpose(1, 2)), "the final key moment is not exactly symmetric"


GRIDS = [  # B, H, n: 16 segments of 4 chunks per head; 38 one-chunk segments per head with a
    (1, 16, 4096), (1, 4, 64 * 37 + 11),  # ragged tail; one segment per head (B*H = 256)
    (2, 128, 150), (1, 1, 1)]


@pytest.mark.parametrize("B,H,n", GRIDS)
@pytest.mark.parametrize("gk", [None, "per_head"])
def test_final_state(B, H, n, gk):
    import oracle
    q, k, v = inputs.qkv(B, H, n, D, D, BF, seed=1100 + n + H)
    g = gammas(gk, H)
    out, fin = fast(q, k, v, gamma=g)
    ro, _, rf = oracle.forward(q, k, v, gamma=g)
    e = row_err(out.cpu(), ro)
    print(f"row error {e:.3e}")
    assert e <= TOL[BF]
    check_state(fin, rf, TOL[BF])


@pytest.mark.parametrize("B,H,n,split", [(1, 16, 4096, 2085), (1, 4, 1000, 133)])
def test_continuation_across_a_split(B, H, n, split):
    import oracle
    q, k, v = inputs.qkv(B, H, n, D, D, BF, seed=1200 + split)
    g = gammas("per_head", H)
    cut = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    o1, s1 = fast(cut(q, 0, split), cut(k, 0, split), cut(v, 0, split), gamma=g)
    o2, s2 = fast(cut(q, split, n), cut(k, split, n), cut(v, split, n), gamma=g, init=s1)
    ro, _, rf = oracle.forward(q, k, v, gamma=g)
    e = row_err(torch.cat([o1, o2], dim=2).cpu(), ro)
    print(f"row error {e:.3e}")
    assert e <= TOL[BF]
    check_state(s2, rf, TOL[BF])


@pytest.mark.parametrize("B,H,n", [(1, 4, 64 * 37 + 11), (2, 128, 150), (1, 16, 2048)])
def test_arbitrary_initial_state(B, H, n):
    """An initial state that no prefix produces, with and without a final
    state (the outputs must be the same bits either way)."""
    import oracle
    q, k, v = inputs.qkv(B, H, n, D, D, BF, seed=1300 + n)
    g = gammas("decay", H)
    st = inputs.random_state_fp32(B * H, D, D, seed=1301 + n, scale=0.05)
    init = hla.State(*(t.to(DEV) for t in st))
    ref_init = oracle.State(*(t.double().numpy() for t in st))
    ro, _, rf = oracle.forward(q, k, v, gamma=g, init=ref_init)
    out, fin = fast(q, k, v, gamma=g, init=init)
    e = row_err(out.cpu(), ro)
    print(f"row error {e:.3e}")
    assert e <= TOL[BF]
    check_state(fin, rf, TOL[BF])
    out2, _ = fast(q, k, v, gamma=g, init=init, state=False)
    assert torch.equal(out2, out)


def test_composition_of_one_launch_segments():
    import oracle
    B, H, n, p = 1, 8, 3000, 1401
    q, k, v = inputs.qkv(B, H, n, D, D, BF, seed=1400)
    g = gammas("per_head", H)
    cut = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    _, sa = fast(cut(q, 0, p), cut(k, 0, p), cut(v, 0, p), gamma=g)
    _, sb = fast(cut(q, p, n), cut(k, p, n), cut(v, p, n), gamma=g)
    sab = hla.state_compose(sa, sb)
    _, _, rf = oracle.forward(q, k, v, gamma=g)
    g_ = {k: getattr(sab, k).cpu().double().numpy() for k in ("S", "C", "m", "G", "h")}
    sc, sm = naive_scales(rf.S, rf.C, rf.m)
    for k in ("S", "C", "m", "G", "h"):
        scale = sc if k == "G" else sm if k == "h" else None
        assert slab_err(g_[k], getattr(rf, k), scale=scale) <= TOL[BF], k


def test_state_outputs_match_the_plain_kernel_and_reuse_a_workspace():
    B, H, n = 1, 16, 4096
    q, k, v = inputs.qkv(B, H, n, D, D, BF, seed=1500)
    g = gammas("per_head", H)
    ws = torch.zeros(hla.workspace_size(B, H, n, D, D), dtype=torch.uint8, device=DEV)
    o_plain, _ = fast(q, k, v, gamma=g, state=False, ws=ws)
    o_state, f1 = fast(q, k, v, gamma=g, ws=ws)
    o_again, f2 = fast(q, k, v, gamma=g, ws=ws)
    assert row_err(o_state.cpu(), o_plain.cpu()) <= 1e-4
    assert torch.equal(o_state, o_again)
    for a, b in zip(f1.tensors(), f2.tensors()):
        assert torch.equal(a, b)


def test_forced_give_up_poisons_and_recovers():
    """Control word 4 = -1: every wait gives up without polling (and is
    counted); the launch ends normally, outputs and the final state built on
    a given-up carry are NaN, and with the limit restored the same workspace
    gives the reference again."""
    B, H, n = 1, 16, 4096
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, D, D, BF, seed=1600))
    ws = torch.zeros(hla.workspace_size(B, H, n, D, D), dtype=torch.uint8, device=DEV)
    words = ws[:64].view(torch.int32)
    words[4] = -1
    out, _, fin = hla.forward_chunked(q, k, v, return_state=True, workspace=ws)
    torch.cuda.synchronize()
    w = ctrl_words(ws)
    assert w[2] == 1 and w[3] > 0, w
    assert not torch.isfinite(fin.S).all()   # the last segments waited on others
    assert torch.isfinite(out[:, :, :256]).all()  # the first segment waits on nothing
    words[4] = 0
    words[3] = 0
    out2, _, fin2 = hla.forward_chunked(q, k, v, return_state=True, workspace=ws)
    ref, _, fref = hla.forward_chunked(q, k, v, return_state=True)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[3] == 0
    assert torch.equal(out2, ref)
    for a, b in zip(fin2.tensors(), fref.tensors()):
        assert torch.equal(a, b)

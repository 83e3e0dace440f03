"""GPU parity of the one-launch d = 64 forward when it takes an initial state
and/or returns a final state, against the fp64 oracle.

The state-carrying calls (bf16, d = dv = 64, chunk 64, every decay >= 0.75)
run the one-launch kernel's state variant: the initial state enters every
segment's carry, and the last segment of each head forms the final state
(S, C, m, G, h, rho) from its carry and its own sums.  Cases: the one-pass
grid and the looped grid, ragged tails, a single segment, a single token,
decay per head, ridge, denominator and ratio; continuation across a split
point that is not chunk-aligned; initial states that no prefix produces
(C and G independent of S); composition of GPU segment states; and the
failure path forced from the host.  The control block (launch count in
word 2, give-ups in word 3) shows that the one-launch kernel ran.
Masked second-order HLA: Higher-order Linear Attention (paperlayer.ai
summary), sec. 4 (carry-in prefixes of the chunk scan) and sec. 4.2 (the
masked state and its composition).
"""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import TOL, naive_scales, ratio_err, row_err, slab_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF = torch.bfloat16


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
        return inputs.gamma_list_fp32([0.97] * H)
    if kind == "per_head":
        return inputs.gamma_list_fp32([(0.75, 0.9, 0.99, 1.0, 0.999, 0.8, 0.95, 0.97)[h % 8] for h in range(H)])
    if kind == "strong":
        return inputs.gamma_list_fp32([0.75] * H)
    return None


def fast(q, k, v, *, gamma=None, ridge=0.0, normalize=False, den=False, init=None, state=True):
    """One call on a fresh workspace; asserts that the one-launch kernel ran
    and that no wait gave up."""
    B, H, n, d = q.shape
    qg, kg, vg = (x.to(DEV).contiguous() for x in (q, k, v))
    ws = torch.zeros(hla.workspace_size(B, H, n, d, d, chunk=64), dtype=torch.uint8, device=DEV)
    out, dn, fin = hla.forward_chunked(qg, kg, vg, gamma=gamma, ridge=ridge, normalize=normalize, chunk=64,
                                       init=init, return_state=state, return_den=den, workspace=ws)
    torch.cuda.synchronize()
    w = ctrl_words(ws)
    assert w[2] == 1, f"the one-launch path did not run: {w}"
    assert w[3] == 0, f"a wait gave up: {w}"
    return out, dn, fin


def check_state(gpu, ref, tol, names=("S", "C", "m", "G", "h")):
    g = {k: getattr(gpu, k).cpu().double().numpy() for k in ("S", "C", "m", "G", "h", "rho")}
    sc, sm = naive_scales(ref.S, ref.C, ref.m)
    for k in names:
        scale = sc if k == "G" else sm if k == "h" else None
        e = slab_err(g[k], getattr(ref, k), scale=scale)
        print(f"state {k}: slab error {e:.3e}")
        assert e <= tol, f"state {k}: slab error {e:.3e} > {tol:.0e}"
    ref_rho = np.asarray(ref.rho, dtype=np.float32).astype(np.float64)
    assert np.allclose(g["rho"], ref_rho, rtol=2e-5, atol=1.2e-38), "rho"
    S = gpu.S.cpu()
    assert torch.equal(S, S.transpose(1, 2)), "the final key moment is not exactly symmetric"


def check_out(out, dn, ro, rd, normalize, den):
    tol = TOL[BF]
    if normalize:
        e, excluded = ratio_err(out.cpu(), ro, rd)
        print(f"ratio row error {e:.3e} ({excluded} rows excluded)")
    else:
        e = row_err(out.cpu(), ro)
        print(f"row error {e:.3e}")
    assert e <= tol
    if den:
        ed = slab_err(dn.cpu(), rd, lead=2)
        print(f"den slab error {ed:.3e}")
        assert ed <= tol


GRIDS = [  # B, H, n: one-pass grid at the headline shape, one-pass ragged (14 segments per head),
    (4, 8, 2048), (2, 3, 64 * 13 + 37),  # looped grid ragged (288 segments on at most 256 workgroups),
    (4, 8, 64 * 32 + 37), (1, 1, 50), (1, 2, 1)]  # a single segment, a single token
OPTIONS = [  # gamma, ridge, den, normalize
    (None, 0.0, False, False), ("per_head", 1e-3, True, False), ("decay", 0.0, True, True),
    ("strong", 0.5, False, False)]


@pytest.mark.parametrize("B,H,n", GRIDS)
@pytest.mark.parametrize("gk,ridge,den,normalize", OPTIONS)
def test_final_state(B, H, n, gk, ridge, den, normalize):
    import oracle
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=700 + n + H)
    if normalize:
        q, k = (x.float().abs().add(0.1).to(BF) for x in (q, k))
    g = gammas(gk, H)
    ridge = inputs.ridge_fp32(ridge)
    out, dn, fin = fast(q, k, v, gamma=g, ridge=ridge, normalize=normalize, den=den)
    ro, rd, rf = oracle.forward(q, k, v, gamma=g, lam=ridge, normalize=normalize)
    check_out(out, dn, ro, rd, normalize, den)
    check_state(fin, rf, TOL[BF])


@pytest.mark.parametrize("B,H,n,split", [(2, 4, 1000, 133), (4, 8, 4096, 2048 + 37), (1, 2, 300, 64)])
@pytest.mark.parametrize("gk,ridge,normalize", [(None, 0.0, False), ("per_head", 1e-3, True)])
def test_continuation_across_a_split(B, H, n, split, gk, ridge, normalize):
    """Segment A's final state starts segment B; both calls take the one-launch
    kernel.  Together they equal the whole sequence."""
    import oracle
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=800 + split)
    if normalize:
        q, k = (x.float().abs().add(0.1).to(BF) for x in (q, k))
    g = gammas(gk, H)
    ridge = inputs.ridge_fp32(ridge)
    cut = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    o1, _, s1 = fast(cut(q, 0, split), cut(k, 0, split), cut(v, 0, split), gamma=g, ridge=ridge,
                     normalize=normalize)
    o2, _, s2 = fast(cut(q, split, n), cut(k, split, n), cut(v, split, n), gamma=g, ridge=ridge,
                     normalize=normalize, init=s1)
    ro, rd, rf = oracle.forward(q, k, v, gamma=g, lam=ridge, normalize=normalize)
    check_out(torch.cat([o1, o2], dim=2), None, ro, rd, normalize, False)
    check_state(s2, rf, TOL[BF])


@pytest.mark.parametrize("B,H,n", [(2, 3, 64 * 13 + 37), (4, 8, 64 * 32 + 37), (1, 2, 40)])
@pytest.mark.parametrize("gk,ridge,den,normalize", [(None, 0.0, True, False), ("per_head", 1e-3, True, False),
                                                    ("decay", 0.25, False, False)])
def test_arbitrary_initial_state(B, H, n, gk, ridge, den, normalize):
    """An initial state that no prefix produces (symmetric S; C, m, G, h and
    rho independent of it), with and without a final state."""
    import oracle
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=900 + n)
    g = gammas(gk, H)
    ridge = inputs.ridge_fp32(ridge)
    st = inputs.random_state_fp32(B * H, 64, 64, seed=901 + n, scale=0.1)
    init = hla.State(*(t.to(DEV) for t in st))
    ref_init = oracle.State(*(t.double().numpy() for t in st))
    ro, rd, rf = oracle.forward(q, k, v, gamma=g, lam=ridge, normalize=normalize, init=ref_init)
    out, dn, fin = fast(q, k, v, gamma=g, ridge=ridge, normalize=normalize, den=den, init=init)
    check_out(out, dn, ro, rd, normalize, den)
    check_state(fin, rf, TOL[BF])
    # the initial state alone (no final state): the same outputs
    out2, dn2, _ = fast(q, k, v, gamma=g, ridge=ridge, normalize=normalize, den=den, init=init, state=False)
    assert torch.equal(out2, out)
    if den:
        assert torch.equal(dn2, dn)


def test_composition_of_one_launch_segments():
    """Two segments' final states (one-launch kernel) composed on the GPU equal
    the whole sequence's state."""
    import oracle
    B, H, n, p = 2, 4, 1500, 701
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=950)
    g = gammas("per_head", H)
    cut = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    _, _, sa = fast(cut(q, 0, p), cut(k, 0, p), cut(v, 0, p), gamma=g)
    _, _, sb = fast(cut(q, p, n), cut(k, p, n), cut(v, p, n), gamma=g)
    sab = hla.state_compose(sa, sb)
    _, _, rf = oracle.forward(q, k, v, gamma=g)
    check_state(sab, rf, TOL[BF], names=("S", "C", "m", "G", "h"))


def test_state_variant_matches_the_plain_kernel():
    """Outputs with a final state requested agree with the plain one-launch
    kernel's.  They are not the same bits: the state variant is built on the
    denominator variant, which splits the S carry into three bf16 terms where
    the plain kernel takes two, so the two differ by the plain kernel's own
    rounding (about 1e-5 of a row against the fp64 oracle)."""
    B, H, n = 4, 8, 2048
    q, k, v = inputs.qkv(B, H, n, 64, 64, BF, seed=960)
    g = gammas("per_head", H)
    o_state, _, _ = fast(q, k, v, gamma=g)
    o_plain, _, _ = fast(q, k, v, gamma=g, state=False)
    assert row_err(o_state.cpu(), o_plain.cpu()) <= 1e-4


def test_state_calls_are_deterministic_and_reuse_a_workspace():
    B, H, n = 2, 3, 64 * 13 + 37
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, 64, 64, BF, seed=970))
    g = gammas("decay", H)
    st = inputs.random_state_fp32(B * H, 64, 64, seed=971, scale=0.1)
    init = hla.State(*(t.to(DEV) for t in st))
    ws = torch.zeros(hla.workspace_size(B, H, n, 64, 64, chunk=64), dtype=torch.uint8, device=DEV)
    r1 = hla.forward_chunked(q, k, v, gamma=g, chunk=64, init=init, return_state=True, workspace=ws)
    r2 = hla.forward_chunked(q, k, v, gamma=g, chunk=64, init=init, return_state=True, workspace=ws)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[2] == 2
    assert torch.equal(r1[0], r2[0])
    for a, b in zip(r1[2].tensors(), r2[2].tensors()):
        assert torch.equal(a, b)


def test_forced_give_up_poisons_the_state():
    """With control word 4 = -1 the waits give up after one unsuccessful poll:
    the launch ends normally, and any carry that was given up is NaN, in the
    outputs and in the final state built on it; nothing is a silently wrong
    number.  With the limit restored the same workspace gives the reference."""
    import oracle
    B, H, n = 4, 8, 2048
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, 64, 64, BF, seed=980))
    ws = torch.zeros(hla.workspace_size(B, H, n, 64, 64, chunk=64), dtype=torch.uint8, device=DEV)
    words = ws[:64].view(torch.int32)
    words[4] = -1
    out, _, fin = hla.forward_chunked(q, k, v, chunk=64, return_state=True, workspace=ws)
    torch.cuda.synchronize()
    w = ctrl_words(ws)
    assert w[2] == 1, w
    ro, _, rf = oracle.forward(q.cpu(), k.cpu(), v.cpu())
    o = out.cpu().double().numpy()
    bad = ~np.isfinite(o)
    # every finite row is right; if a wait gave up, some outputs are NaN
    good_rows = np.all(np.isfinite(o), axis=-1)
    num = np.max(np.abs(o[good_rows] - ro[good_rows]), axis=-1)
    assert np.all(num <= TOL[BF] * np.max(np.abs(ro[good_rows]), axis=-1))
    if w[3] > 0:
        assert bad.any()
    for t in fin.tensors()[:5]:  # a finite state is the right one
        x = t.cpu()
        if w[3] == 0:
            assert torch.isfinite(x).all()
    words[4] = 0
    words[3] = 0
    out2, _, fin2 = hla.forward_chunked(q, k, v, chunk=64, return_state=True, workspace=ws)
    ref, _, fref = hla.forward_chunked(q, k, v, chunk=64, return_state=True)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[3] == 0
    assert torch.equal(out2, ref)
    for a, b in zip(fin2.tensors(), fref.tensors()):
        assert torch.equal(a, b)

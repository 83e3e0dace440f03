"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
identical seeded inputs.  Every test here needs an MI355X and the built
libhla.so; none falls back to anything else.

Tolerances (tests/parity.py): 2e-3 for bf16 inputs, 1e-5 for fp32 inputs, on
the row error of outputs and the slab error of denominators and states.
"""
import math
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import TOL, naive_scales, ratio_err, row_err, slab_err

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


def state_np(st: hla.State):
    return {k: getattr(st, k).cpu().double().numpy() for k in ("S", "C", "m", "G", "h", "rho")}


def check_state(gpu: hla.State, ref, tol, names=("S", "C", "m", "G", "h")):
    g = state_np(gpu)
    sc, sm = naive_scales(ref.S, ref.C, ref.m)
    for k in names:
        scale = sc if k == "G" else sm if k == "h" else None
        e = slab_err(g[k], getattr(ref, k), scale=scale)
        assert e <= tol, f"state {k}: slab error {e:.3e} > {tol:.0e}"
    # rho = g^len can underflow fp32 (e.g. 0.96875^4096 ~ 3.5e-57): compare with
    # the fp64 value rounded to fp32, below fp32's normal range absolutely
    ref_rho = np.asarray(ref.rho, dtype=np.float32).astype(np.float64)
    assert np.allclose(g["rho"], ref_rho, rtol=1e-5, atol=1.2e-38), "rho"


def run_both(q, k, v, *, gamma=None, ridge=0.0, normalize=False, chunk=0, init_gpu=None,
             init_ref=None):
    qg, kg, vg = on_gpu(q, k, v)
    out, den, fin = hla.forward_chunked(qg, kg, vg, gamma=gamma, ridge=ridge, normalize=normalize,
                                        chunk=chunk, init=init_gpu, return_state=True,
                                        return_den=True)
    torch.cuda.synchronize()
    import oracle
    r_out, r_den, r_fin = oracle.forward(q, k, v, gamma=gamma, lam=ridge, normalize=normalize,
                                         init=init_ref)
    return (out.cpu(), den.cpu(), fin), (r_out, r_den, r_fin)


# ---------------------------------------------------------------------------
# the five workloads at their full sizes

@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("seed", [1000, 2000, 3000])
def test_small_fp32_workload(chunk, seed):
    w = inputs.SMALL_FP32
    q, k, v = inputs.workload_qkv(w, seed)
    (o, d, f), (ro, rd, rf) = run_both(q, k, v, chunk=chunk)
    tol = TOL[torch.float32]
    assert row_err(o, ro) <= tol
    assert slab_err(d, rd, lead=2) <= tol
    check_state(f, rf, tol)


@pytest.mark.parametrize("seed", [1001, 2001])
def test_fwd_d64_workload(seed):
    w = inputs.FWD_D64
    q, k, v = inputs.workload_qkv(w, seed)
    (o, d, f), (ro, rd, rf) = run_both(q, k, v, chunk=w.chunk)
    tol = TOL[torch.bfloat16]
    e = row_err(o, ro)
    print(f"row error {e:.3e}")
    assert e <= tol
    assert slab_err(d, rd, lead=2) <= tol
    check_state(f, rf, tol)


def test_ratio_decay_ridge_d64_workload():
    w = inputs.RATIO_DECAY_D64
    q, k, v = inputs.workload_qkv(w, 1002)
    (o, d, f), (ro, rd, rf) = run_both(q, k, v, gamma=w.gamma, ridge=w.ridge, normalize=True,
                                       chunk=w.chunk)
    tol = TOL[torch.bfloat16]
    e, excluded = ratio_err(o, ro, rd)
    print(f"ratio row error {e:.3e}, excluded rows {excluded}")
    assert e <= tol
    assert slab_err(d, rd, lead=2) <= tol
    check_state(f, rf, tol)
    # the numerator alone, gated row-wise
    qg, kg, vg = on_gpu(q, k, v)
    num, _, _ = hla.forward_chunked(qg, kg, vg, gamma=w.gamma, ridge=w.ridge, chunk=w.chunk)
    import oracle
    rnum, _, _ = oracle.forward(q, k, v, gamma=w.gamma, lam=w.ridge, want_state=False)
    assert row_err(num.cpu(), rnum) <= tol


def test_long_d128_workload():
    w = inputs.LONG_D128
    q, k, v = inputs.workload_qkv(w, 1003)
    (o, d, f), (ro, rd, rf) = run_both(q, k, v, gamma=w.gamma, chunk=w.chunk)
    tol = TOL[torch.bfloat16]
    e = row_err(o, ro)
    print(f"row error {e:.3e}")
    assert e <= tol
    assert slab_err(d, rd, lead=2) <= tol
    check_state(f, rf, tol)
    # the output alone takes the one-launch d = 128 path (two walks per segment)
    qg, kg, vg = on_gpu(q, k, v)
    ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk), dtype=torch.uint8,
                     device=DEV)
    before = ctrl_words(ws)
    fo, _, _ = hla.forward_chunked(qg, kg, vg, gamma=w.gamma, chunk=w.chunk, workspace=ws)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[2] != before[2], "the one-launch d=128 path did not run"
    ef = row_err(fo.cpu(), ro)
    print(f"fused d128 row error {ef:.3e}")
    assert ef <= tol


def decode_setup(B, H, prefix, d, dv, seed, gamma=None, ridge=0.0):
    """Fold a prefix with the oracle (fp64), round the states to fp32, and hand
    the same fp32 states to both sides."""
    import oracle
    (q, k, v), tok = inputs.decode_inputs(B, H, prefix, d, dv, torch.bfloat16, seed)
    _, _, st = oracle.forward(q, k, v, gamma=gamma, lam=ridge)
    st32 = {n: torch.from_numpy(getattr(st, n)).float() for n in ("S", "C", "m", "G", "h", "rho")}
    ref = oracle.State(*(st32[n].double().numpy() for n in ("S", "C", "m", "G", "h", "rho")))
    gpu = hla.State(*(st32[n].to(DEV) for n in ("S", "C", "m", "G", "h", "rho")))
    return tok, gpu, ref


def test_decode_workload():
    w = inputs.DECODE_D128
    tok, gpu, ref = decode_setup(w.B, w.H, w.n, w.d, w.dv, 1004)
    q1, k1, v1 = tok
    qg, kg, vg = on_gpu(q1, k1, v1)
    out, den = hla.decode_step(qg, kg, vg, gpu, return_den=True)
    torch.cuda.synchronize()
    import oracle
    r_out, r_den, r_st = oracle.decode(ref, q1, k1, v1)
    tol = TOL[torch.bfloat16]
    e = row_err(out.cpu(), r_out)
    print(f"decode row error {e:.3e}")
    assert e <= tol
    assert slab_err(den.cpu().reshape(-1, 1), r_den.reshape(-1, 1)) <= tol
    check_state(gpu, r_st, 1e-5)


@pytest.mark.parametrize("gamma,ridge,normalize", [(None, 0.0, False), (0.95, 0.5, True),
                                                   ("per_head", 1e-3, False)])
@pytest.mark.parametrize("d,dv", [(128, 128), (64, 32), (16, 128)])
def test_decode_variants(d, dv, gamma, ridge, normalize):
    B, H = 2, 8
    g = None
    if gamma == "per_head":
        g = inputs.gamma_list_fp32([1 - 2.0 ** -(3 + h) for h in range(H)])
    elif gamma is not None:
        g = inputs.gamma_list_fp32([gamma] * H)
    tok, gpu, ref = decode_setup(B, H, 64, d, dv, 77 + d + dv, gamma=g, ridge=ridge)
    qg, kg, vg = on_gpu(*tok)
    out, den = hla.decode_step(qg, kg, vg, gpu, gamma=g, ridge=ridge, normalize=normalize,
                               return_den=True)
    import oracle
    r_out, r_den, r_st = oracle.decode(ref, *tok, gamma=g, lam=ridge, normalize=normalize)
    tol = TOL[torch.bfloat16]
    assert row_err(out.cpu(), r_out) <= tol
    check_state(gpu, r_st, 1e-5)


# ---------------------------------------------------------------------------
# shape and option sweep at small sizes (several chunks and a ragged tail)

SWEEP = [
    # B, H, n,   d,   dv,  w,  dtype,           gamma,      ridge, normalize
    (1, 2, 100, 16, 16, 16, torch.float32, None, 0.0, False),
    (2, 2, 77, 32, 64, 32, torch.float32, "decay", 0.0, False),
    (1, 3, 130, 64, 16, 64, torch.float32, "per_head", 1.0, False),
    (1, 1, 300, 128, 128, 128, torch.float32, "decay", 0.0, True),
    (2, 2, 129, 64, 64, 64, torch.bfloat16, None, 0.0, False),
    (1, 2, 200, 64, 64, 16, torch.bfloat16, "per_head", 1e-3, True),
    (1, 2, 257, 128, 64, 128, torch.bfloat16, "decay", 0.0, False),
    (2, 1, 95, 16, 32, 32, torch.bfloat16, None, 1.0, True),
    (1, 2, 64, 64, 128, 64, torch.bfloat16, "decay", 0.0, False),
    (1, 1, 1, 64, 64, 64, torch.bfloat16, None, 0.3, False),
    (1, 2, 33, 32, 32, 128, torch.float32, None, 0.0, False),
]


@pytest.mark.parametrize("case", SWEEP, ids=[f"B{c[0]}H{c[1]}n{c[2]}d{c[3]}dv{c[4]}w{c[5]}"
                                              f"{'bf16' if c[6] == torch.bfloat16 else 'f32'}"
                                              f"{'-'+c[7] if c[7] else ''}-l{c[8]}{'-norm' if c[9] else ''}"
                                              for c in SWEEP])
def test_sweep(case):
    B, H, n, d, dv, w, dtype, gk, ridge, normalize = case
    q, k, v = inputs.qkv(B, H, n, d, dv, dtype, seed=500 + n + d + dv + w)
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.97] * H)
    elif gk == "per_head":
        g = inputs.gamma_list_fp32([1 - 2.0 ** -(3 + h) for h in range(H)])
    ridge = inputs.ridge_fp32(ridge)
    (o, dn, f), (ro, rd, rf) = run_both(q, k, v, gamma=g, ridge=ridge, normalize=normalize, chunk=w)
    tol = TOL[dtype]
    if normalize:
        e, _ = ratio_err(o, ro, rd)
    else:
        e = row_err(o, ro)
    assert e <= tol, f"output error {e:.3e}"
    assert slab_err(dn, rd, lead=2) <= tol
    check_state(f, rf, max(tol, 1e-5))


# ---------------------------------------------------------------------------
# streaming, state algebra and edge cases

def test_split_point_continuation_on_gpu():
    B, H, n, d, dv = 2, 4, 300, 64, 64
    q, k, v = inputs.qkv(B, H, n, d, dv, torch.bfloat16, seed=41)
    g = inputs.gamma_list_fp32([0.99, 0.995, 1.0, 0.98])
    qg, kg, vg = on_gpu(q, k, v)
    p = 133
    o1, _, s1 = hla.forward_chunked(qg[:, :, :p].contiguous(), kg[:, :, :p].contiguous(),
                                    vg[:, :, :p].contiguous(), gamma=g, return_state=True)
    o2, _, s2 = hla.forward_chunked(qg[:, :, p:].contiguous(), kg[:, :, p:].contiguous(),
                                    vg[:, :, p:].contiguous(), gamma=g, init=s1, return_state=True)
    import oracle
    ro, _, rf = oracle.forward(q, k, v, gamma=g)
    tol = TOL[torch.bfloat16]
    assert row_err(torch.cat([o1, o2], dim=2).cpu(), ro) <= tol
    check_state(s2, rf, tol)


@pytest.mark.parametrize("dtype,d,w", [(torch.float32, 32, 16), (torch.bfloat16, 64, 64), (torch.bfloat16, 128, 128)])
def test_final_key_moment_is_exactly_symmetric(dtype, d, w):
    """The decode step reads only S's upper tiles, so the forward must hand
    over an exactly symmetric S (every chunk sum and prefix keeps it so)."""
    q, k, v = inputs.qkv(2, 3, 301, d, d, dtype, seed=43)
    qg, kg, vg = on_gpu(q, k, v)
    g = inputs.gamma_list_fp32([0.97, 0.999, 1.0])
    _, _, st = hla.forward_chunked(qg, kg, vg, gamma=g, chunk=w, return_state=True)
    torch.cuda.synchronize()
    S = st.S.cpu()
    assert torch.equal(S, S.transpose(1, 2))


def test_forward_last_row_equals_decode_on_gpu():
    B, H, n, d, dv = 1, 4, 200, 64, 64
    q, k, v = inputs.qkv(B, H, n + 1, d, dv, torch.bfloat16, seed=42)
    qg, kg, vg = on_gpu(q, k, v)
    out, _, _ = hla.forward_chunked(qg, kg, vg)
    _, _, st = hla.forward_chunked(qg[:, :, :n].contiguous(), kg[:, :, :n].contiguous(),
                                   vg[:, :, :n].contiguous(), return_state=True)
    o1, _ = hla.decode_step(qg[:, :, n].contiguous(), kg[:, :, n].contiguous(),
                            vg[:, :, n].contiguous(), st)
    assert row_err(o1.cpu(), out[:, :, n].cpu()) <= 1e-4


def test_compose_matches_oracle():
    import oracle
    N, d, dv = 6, 64, 32
    a = inputs.random_state_fp32(N, d, dv, 1)
    b = inputs.random_state_fp32(N, d, dv, 2)
    ga = hla.State(*(t.to(DEV) for t in a))
    gb = hla.State(*(t.to(DEV) for t in b))
    r = hla.state_compose(ga, gb)
    ra = oracle.State(*(t.double().numpy() for t in a))
    rb = oracle.State(*(t.double().numpy() for t in b))
    rr = oracle.compose(ra, rb)
    check_state(r, rr, 1e-5)


@pytest.mark.parametrize("d,dv", [(16, 16), (128, 128), (32, 64)])
def test_compose_of_gpu_segments_equals_whole(d, dv):
    B, H, n = 1, 2, 150
    q, k, v = inputs.qkv(B, H, n, d, dv, torch.bfloat16, seed=43)
    g = inputs.gamma_list_fp32([0.98, 1.0])
    qg, kg, vg = on_gpu(q, k, v)
    p = 70
    _, _, sa = hla.forward_chunked(qg[:, :, :p].contiguous(), kg[:, :, :p].contiguous(),
                                   vg[:, :, :p].contiguous(), gamma=g, return_state=True)
    _, _, sb = hla.forward_chunked(qg[:, :, p:].contiguous(), kg[:, :, p:].contiguous(),
                                   vg[:, :, p:].contiguous(), gamma=g, return_state=True)
    sab = hla.state_compose(sa, sb)
    import oracle
    _, _, rf = oracle.forward(q, k, v, gamma=g)
    check_state(sab, rf, TOL[torch.bfloat16])


def test_empty_sequence_returns_init():
    N, d, dv = 3, 32, 16
    a = inputs.random_state_fp32(N, d, dv, 5)
    init = hla.State(*(t.to(DEV) for t in a))
    q = torch.empty(1, 3, 0, d, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(1, 3, 0, dv, dtype=torch.bfloat16, device=DEV)
    out, _, fin = hla.forward_chunked(q, q.clone(), v, init=init, return_state=True,
                                      gamma=[0.9, 0.8, 0.7])
    assert out.shape == (1, 3, 0, dv)
    for name in ("S", "C", "m"):
        assert torch.equal(getattr(fin, name), getattr(init, name))
    import oracle
    # G and h are rebuilt from X = S C - G on the way through: equal to rounding
    ref = oracle.State(*(t.double().numpy() for t in a))
    check_state(fin, ref, 1e-5)
    _, _, z = hla.forward_chunked(q, q.clone(), v, return_state=True)
    for t in z.tensors()[:5]:
        assert torch.count_nonzero(t) == 0
    assert torch.all(z.rho == 1)


def test_causality_bitwise():
    B, H, n, d, dv = 1, 2, 256, 64, 64
    q, k, v = inputs.qkv(B, H, n, d, dv, torch.bfloat16, seed=44)
    g = inputs.gamma_list_fp32([0.97, 1.0])
    qg, kg, vg = on_gpu(q, k, v)
    out, den, _ = hla.forward_chunked(qg, kg, vg, gamma=g, ridge=0.01, return_den=True)
    for t in (0, 63, 64, 100, 254):
        q2, k2, v2 = qg.clone(), kg.clone(), vg.clone()
        gen = torch.Generator(device="cpu").manual_seed(t)
        for x in (q2, k2, v2):
            noise = torch.randn(x[:, :, t + 1:].shape, generator=gen).to(x.dtype).to(DEV)
            x[:, :, t + 1:] += noise
        o2, d2, _ = hla.forward_chunked(q2, k2, v2, gamma=g, ridge=0.01, return_den=True)
        assert torch.equal(o2[:, :, : t + 1], out[:, :, : t + 1]), t
        assert torch.equal(d2[:, :, : t + 1], den[:, :, : t + 1]), t
        assert not torch.equal(o2[:, :, t + 1:], out[:, :, t + 1:])


def test_deterministic_and_writes_every_output():
    w = inputs.FWD_D64
    q, k, v = on_gpu(*inputs.workload_qkv(w, 7))
    out1 = torch.full((w.B, w.H, w.n, w.dv), float("nan"), device=DEV)
    den1 = torch.full((w.B, w.H, w.n), float("nan"), device=DEV)
    hla.forward_chunked(q, k, v, chunk=w.chunk, out=out1, den=den1)
    out2, den2, _ = hla.forward_chunked(q, k, v, chunk=w.chunk, return_den=True)
    assert torch.isfinite(out1).all() and torch.isfinite(den1).all()
    assert torch.equal(out1, out2) and torch.equal(den1, den2)


def test_bad_arguments_raise_before_launch():
    q = torch.zeros(1, 1, 8, 48, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(hla.HlaError, match="UNSUPPORTED"):
        hla.forward_chunked(q, q, q)
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(hla.HlaError, match="gamma"):
        hla.forward_chunked(q, q, q, gamma=[1.5])


# ---------------------------------------------------------------------------
# the one-launch MFMA path (bf16, d = dv = w = 64, out only)

def ctrl_words(ws):
    return ws[:16].view(torch.int32).cpu().tolist()


@pytest.mark.parametrize("B,H,n,gk", [
    (4, 8, 2048, None),            # the bench workload
    (1, 2, 64, None),              # one chunk per head
    (1, 3, 1, None),               # one token
    (2, 2, 100, "decay"),          # ragged tail, two chunks
    (1, 4, 1000, "per_head"),      # ragged, several segments per head
    (3, 5, 4095, "decay"),         # many segments, ragged
    (8, 8, 4096, "per_head"),      # more workgroups than CUs
    (8, 8, 4096, None),            # more workgroups than CUs, no decay
    (1, 2, 8192, None),            # more than eight earlier segments to sum, no decay
    (1, 1, 16384, "decay"),        # one head, long
    (4, 64, 256, None),            # 256 heads: the tail of q_0 . k_0 near zero at t = 0
    (5, 64, 200, "decay"),         # 320 one-segment heads: a grid larger than the CU count
])
def test_fused_forward(B, H, n, gk):
    q, k, v = inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=900 + n + H)
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.995] * H)
    elif gk == "per_head":
        g = inputs.gamma_list_fp32([1 - 2.0 ** -(5 + h % 8) for h in range(H)])
    qg, kg, vg = on_gpu(q, k, v)
    ws = torch.zeros(hla.workspace_size(B, H, n, 64, 64, chunk=64), dtype=torch.uint8, device=DEV)
    before = ctrl_words(ws)
    out, _, _ = hla.forward_chunked(qg, kg, vg, gamma=g, chunk=64, workspace=ws)
    torch.cuda.synchronize()
    after = ctrl_words(ws)
    assert after[2] != before[2], "the one-launch path did not run (epoch unchanged)"
    assert after[0] == 0 and after[1] == 0 and after[3] == 0, after
    import oracle
    ro, _, _ = oracle.forward(q, k, v, gamma=g, want_state=False)
    e = row_err(out.cpu(), ro)
    print(f"fused row error {e:.3e}")
    assert e <= TOL[torch.bfloat16]
    # a second call on the same workspace (ticket reset, new epoch) is identical
    out2, _, _ = hla.forward_chunked(qg, kg, vg, gamma=g, chunk=64, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert ctrl_words(ws)[2] != after[2]


def test_fused_matches_generic_path():
    B, H, n = 2, 4, 700
    q, k, v = on_gpu(*inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=31))
    g = inputs.gamma_list_fp32([0.99, 0.999, 1.0, 0.98])
    fused, fden, _ = hla.forward_chunked(q, k, v, gamma=g, ridge=1e-3, chunk=64, return_den=True)
    # the same inputs widened exactly to fp32 take the generic kernels
    generic, gden, _ = hla.forward_chunked(q.float(), k.float(), v.float(), gamma=g, ridge=1e-3, chunk=64,
                                           return_den=True)
    assert row_err(fused.cpu(), generic.cpu()) <= 2e-4
    assert slab_err(fden.cpu(), gden.cpu(), lead=2) <= 2e-4


@pytest.mark.parametrize("B,H,n", [(2, 3, 64 * 13 + 37), (4, 8, 64 * 32 + 37)])
@pytest.mark.parametrize("gk", [None, "per_head"])
@pytest.mark.parametrize("ridge,den,normalize", [
    (0.0, True, False), (1e-3, False, False), (1e-3, True, True), (1.0, True, False),
    (0.0, False, True),
])
def test_fused_options(B, H, n, gk, ridge, den, normalize):
    """Ridge, denominator and ratio on the one-launch path, with a ragged
    tail: 14 one-chunk segments per head (6 heads), or 9 segments of four
    chunks per head, the last one a partial chunk (32 heads)."""
    q, k, v = inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=700 + int(1000 * ridge) + H)
    g = None if gk is None else inputs.gamma_list_fp32([1 - 2.0 ** -(5 + h) for h in range(H)])
    lam = inputs.ridge_fp32(ridge)
    qg, kg, vg = on_gpu(q, k, v)
    ws = torch.zeros(hla.workspace_size(B, H, n, 64, 64, chunk=64), dtype=torch.uint8, device=DEV)
    before = ctrl_words(ws)
    out, dg, _ = hla.forward_chunked(qg, kg, vg, gamma=g, ridge=lam, normalize=normalize, chunk=64,
                                     return_den=den, workspace=ws)
    torch.cuda.synchronize()
    after = ctrl_words(ws)
    assert after[2] != before[2], "the one-launch path did not run"
    assert after[3] == 0, after
    import oracle
    ro, rd, _ = oracle.forward(q, k, v, gamma=g, lam=lam, normalize=normalize, want_state=False)
    tol = TOL[torch.bfloat16]
    if normalize:
        e, excluded = ratio_err(out.cpu(), ro, rd)
        print(f"ratio row error {e:.3e} ({excluded} rows excluded)")
    else:
        e = row_err(out.cpu(), ro)
        print(f"row error {e:.3e}")
    assert e <= tol
    if den:
        ed = slab_err(dg.cpu(), rd, lead=2)
        print(f"den slab error {ed:.3e}")
        assert ed <= tol


def test_fused_ratio_workload():
    """The ratio-normalised workload with per-head decay and ridge (B8 H8 n4096)
    through the one-launch path: out and den, no final state."""
    w = inputs.RATIO_DECAY_D64
    q, k, v = inputs.workload_qkv(w, 1002)
    qg, kg, vg = on_gpu(q, k, v)
    ws = torch.zeros(hla.workspace_size(w.B, w.H, w.n, w.d, w.dv, chunk=w.chunk), dtype=torch.uint8,
                     device=DEV)
    before = ctrl_words(ws)
    out, den, _ = hla.forward_chunked(qg, kg, vg, gamma=w.gamma, ridge=w.ridge, normalize=True,
                                      chunk=w.chunk, return_den=True, workspace=ws)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[2] != before[2], "the one-launch path did not run"
    import oracle
    ro, rd, _ = oracle.forward(q, k, v, gamma=w.gamma, lam=w.ridge, normalize=True, want_state=False)
    tol = TOL[torch.bfloat16]
    e, excluded = ratio_err(out.cpu(), ro, rd)
    ed = slab_err(den.cpu(), rd, lead=2)
    print(f"ratio row error {e:.3e} ({excluded} rows excluded), den slab error {ed:.3e}")
    assert e <= tol and ed <= tol


def test_fused_workspace_shared_across_shapes():
    ws = torch.zeros(hla.workspace_size(4, 8, 4096, 64, 64, chunk=64), dtype=torch.uint8, device=DEV)
    import oracle
    for (B, H, n) in [(4, 8, 4096), (1, 1, 300), (2, 3, 2048), (4, 8, 4096)]:
        q, k, v = inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=B * 100 + n)
        out, _, _ = hla.forward_chunked(*on_gpu(q, k, v), chunk=64, workspace=ws)
        ro, _, _ = oracle.forward(q, k, v, want_state=False)
        assert row_err(out.cpu(), ro) <= TOL[torch.bfloat16]
    assert ctrl_words(ws)[3] == 0


def test_fused_causality_bitwise():
    B, H, n = 1, 2, 512
    q, k, v = on_gpu(*inputs.qkv(B, H, n, 64, 64, torch.bfloat16, seed=45))
    out, _, _ = hla.forward_chunked(q, k, v, chunk=64)
    for t in (10, 64, 255, 300):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        for x in (q2, k2, v2):
            x[:, :, t + 1:] = -x[:, :, t + 1:]
        o2, _, _ = hla.forward_chunked(q2, k2, v2, chunk=64)
        assert torch.equal(o2[:, :, : t + 1], out[:, :, : t + 1]), t


# ---------------------------------------------------------------------------
# the one-launch d = dv = 128 path (bf16, out only)

@pytest.mark.parametrize("B,H,n,gk", [
    (1, 2, 64, None),           # one chunk, one segment: a single walk
    (1, 3, 1, "decay"),         # one token
    (4, 64, 256, None),         # 256 heads: one segment per head, no rounds
    (1, 16, 4096, "decay"),     # 16 segments of 4 chunks per head
    (2, 3, 1000, "per_head"),   # ragged, one chunk per segment
    (1, 1, 5000, "decay"),      # one head, 79 segments, ragged tail
    (1, 4, 300, None),          # ragged tail inside the only chunk row
    (5, 64, 70, "per_head"),    # 320 heads > 256 CUs: workgroups walk several heads
    (3, 96, 130, None),         # 288 heads, no decay, ragged third chunk
    (1, 100, 150, "decay"),     # 3 one-chunk segments per head: 300 > 256, with the exchange
])
def test_fused128_forward(B, H, n, gk):
    q, k, v = inputs.qkv(B, H, n, 128, 128, torch.bfloat16, seed=1300 + n + H)
    g = None
    if gk == "decay":
        g = inputs.gamma_list_fp32([0.999] * H)
    elif gk == "per_head":
        g = inputs.gamma_list_fp32([1 - 2.0 ** -(5 + h % 8) for h in range(H)])
    qg, kg, vg = on_gpu(q, k, v)
    ws = torch.zeros(hla.workspace_size(B, H, n, 128, 128), dtype=torch.uint8, device=DEV)
    before = ctrl_words(ws)
    out, _, _ = hla.forward_chunked(qg, kg, vg, gamma=g, workspace=ws)
    torch.cuda.synchronize()
    after = ctrl_words(ws)
    assert after[2] != before[2], "the one-launch d=128 path did not run"
    assert after[3] == 0, after
    import oracle
    ro, _, _ = oracle.forward(q, k, v, gamma=g, want_state=False)
    e = row_err(out.cpu(), ro)
    print(f"fused d128 row error {e:.3e}")
    assert e <= TOL[torch.bfloat16]
    out2, _, _ = hla.forward_chunked(qg, kg, vg, gamma=g, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_fused128_causality_bitwise():
    B, H, n = 1, 2, 700
    q, k, v = on_gpu(*inputs.qkv(B, H, n, 128, 128, torch.bfloat16, seed=46))
    out, _, _ = hla.forward_chunked(q, k, v)
    for t in (5, 64, 300, 650):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        for x in (q2, k2, v2):
            x[:, :, t + 1:] = -x[:, :, t + 1:]
        o2, _, _ = hla.forward_chunked(q2, k2, v2)
        assert torch.equal(o2[:, :, : t + 1], out[:, :, : t + 1]), t


@pytest.mark.parametrize("d,B,H,n", [(64, 4, 8, 2048), (128, 1, 16, 4096)])
def test_bounded_waits_give_up_and_are_counted(d, B, H, n):
    """Failure handling of the one-launch kernels, forced from the host: with
    control word 4 set to -1 the cross-workgroup waits give up (the d = 128
    kernel without polling, so some always do and are counted in word 3; the
    d = 64 kernel after one unsuccessful poll, so only those that find their
    flag down).  The launch must end normally either way, and with the limit
    restored the next call on the same workspace is bit-identical to one on a
    fresh workspace."""
    q, k, v = on_gpu(*inputs.qkv(B, H, n, d, d, torch.bfloat16, seed=47))
    ws = torch.zeros(hla.workspace_size(B, H, n, d, d), dtype=torch.uint8, device=DEV)
    words = ws[:64].view(torch.int32)
    words[4] = -1
    hla.forward_chunked(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    w = ctrl_words(ws)
    assert w[2] == 1, w          # the one-launch path ran, and ran to its end
    if d == 128:
        assert w[3] > 0, w       # every wait gave up without polling
    words[4] = 0
    words[3] = 0
    out, _, _ = hla.forward_chunked(q, k, v, workspace=ws)
    ref, _, _ = hla.forward_chunked(q, k, v)
    torch.cuda.synchronize()
    assert ctrl_words(ws)[3] == 0
    assert torch.equal(out, ref)


def test_final_state_into_a_given_state():
    """forward_chunked(final_state=...) writes the same state that
    return_state=True returns, into the caller's tensors."""
    q, k, v = on_gpu(*inputs.qkv(2, 3, 150, 32, 32, torch.float32, seed=48))
    g = inputs.gamma_list_fp32([0.95, 0.99, 1.0])
    _, _, ref = hla.forward_chunked(q, k, v, gamma=g, return_state=True)
    fin = hla.State.empty(6, 32, 32, DEV)
    _, _, got = hla.forward_chunked(q, k, v, gamma=g, final_state=fin)
    torch.cuda.synchronize()
    assert got is fin
    for a, b in zip(ref.tensors(), fin.tensors()):
        assert torch.equal(a, b)

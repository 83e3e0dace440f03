"""hla_forward_chunked_noalloc (through the C ABI) against hla_forward_chunked
on the same inputs: the same kernels run on the library's static scratch
instead of a caller's workspace, so the outputs must be the same bits.  Two
calls in a row, the second with a smaller input, on every kernel path (the
one-launch d = 64 and d = 128 forwards, the d = 64 kernel with initial and
final states, and the generic path with a final state), calls with other
params one after the other, then a call too large for the scratch, which must
fail before anything is enqueued."""
import sys

import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def both(q, k, v, **kw):
    ref_out, ref_den, ref_fin = hla.forward_chunked(q, k, v, **kw)
    B, H, n, _ = q.shape
    dv = v.shape[-1]
    out = torch.full((B, H, n, dv), float("nan"), device=DEV)
    den = torch.full((B, H, n), float("nan"), device=DEV) if kw.get("return_den") else None
    fin = None
    if kw.get("return_state"):
        fin = hla.State.empty(B * H, q.shape[-1], dv, DEV)
        for t in fin.tensors():
            t.fill_(float("nan"))
    kw2 = {x: y for x, y in kw.items() if x not in ("return_den", "return_state")}
    hla.forward_chunked_noalloc(q, k, v, out=out, den=den, final_state=fin, **kw2)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    if den is not None:
        assert torch.equal(den, ref_den)
    if fin is not None:
        for a, b in zip(fin.tensors(), ref_fin.tensors()):
            assert torch.equal(a, b)


def test_noalloc_two_calls_second_smaller():
    w = inputs.FWD_D64
    q, k, v = (x.to(DEV) for x in inputs.workload_qkv(w, 91))
    both(q, k, v, chunk=64)
    q2, k2, v2 = (x.to(DEV) for x in inputs.qkv(2, 3, 700, 64, 64, torch.bfloat16, seed=92))
    g = inputs.gamma_list_fp32([0.99, 0.9, 1.0])
    both(q2, k2, v2, chunk=64, gamma=g, ridge=1e-3, normalize=True, return_den=True)


def test_noalloc_d64_with_states():
    """The one-launch d = 64 kernel's state variant: a final state, then a
    smaller call that continues from it."""
    q, k, v = (x.to(DEV) for x in inputs.qkv(2, 4, 1000, 64, 64, torch.bfloat16, seed=97))
    g = inputs.gamma_list_fp32([0.99, 0.9, 1.0, 0.97])
    both(q, k, v, chunk=64, gamma=g, ridge=1e-3, return_den=True, return_state=True)
    _, _, st = hla.forward_chunked(q, k, v, chunk=64, gamma=g, return_state=True)
    q2, k2, v2 = (x.to(DEV) for x in inputs.qkv(2, 4, 300, 64, 64, torch.bfloat16, seed=98))
    both(q2, k2, v2, chunk=64, gamma=g, init=st, return_state=True)


def test_noalloc_d128_then_generic_with_state():
    q, k, v = (x.to(DEV) for x in inputs.qkv(1, 16, 4096, 128, 128, torch.bfloat16, seed=93))
    both(q, k, v, gamma=inputs.gamma_list_fp32([0.999] * 16))
    q2, k2, v2 = (x.to(DEV) for x in inputs.qkv(1, 2, 300, 32, 32, torch.float32, seed=94))
    both(q2, k2, v2, gamma=[0.97, 1.0], return_state=True, return_den=True)


def test_noalloc_short_sequences():
    """The short-sequence path (two direct maps) keeps its fp32 U in the
    scratch's data: the small fp32 workload, then a smaller bf16 call with
    other widths and per-head decay."""
    w = inputs.SMALL_FP32
    q, k, v = (x.to(DEV) for x in inputs.workload_qkv(w, 102))
    both(q, k, v)
    q2, k2, v2 = (x.to(DEV) for x in inputs.qkv(2, 3, 100, 32, 16, torch.bfloat16, seed=103))
    both(q2, k2, v2, gamma=inputs.gamma_list_fp32([0.9, 1.0, 0.5]))


def test_noalloc_generic_state_call_then_one_launch():
    """Calls with other params share the one scratch: a generic-path call (fp32
    inputs, an initial and a final state) keeps its data past the scratch's
    fixed flag region, so the one-launch call that follows (bf16 d = 64) finds
    only launch epochs in its flags.  Both match the caller-workspace path bit
    for bit."""
    q, k, v = (x.to(DEV) for x in inputs.qkv(2, 4, 1000, 64, 64, torch.float32, seed=99))
    init = hla.State(*(t.to(DEV).contiguous() for t in inputs.random_state_fp32(8, 64, 64, seed=100, scale=0.1)))
    both(q, k, v, chunk=64, gamma=[0.97, 0.9, 1.0, 0.99], init=init, return_state=True)
    q2, k2, v2 = (x.to(DEV) for x in inputs.qkv(4, 8, 2048, 64, 64, torch.bfloat16, seed=101))
    both(q2, k2, v2, chunk=64)


def test_noalloc_in_a_graph():
    """Calls of the entry point captured into a HIP graph (nothing is
    allocated inside the capture) replay to the eager result, with eager
    work and synchronisations between the replays."""
    q, k, v = (x.to(DEV) for x in inputs.qkv(2, 4, 1000, 64, 64, torch.bfloat16, seed=95))
    ref, _, _ = hla.forward_chunked(q, k, v, chunk=64)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # warm: the first call looks up the scratch address
        hla.forward_chunked_noalloc(q, k, v, chunk=64, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(3):
            hla.forward_chunked_noalloc(q, k, v, chunk=64, out=out)
    for rep in range(3):
        out.fill_(float("nan"))
        hla.forward_chunked(q, k, v, chunk=64)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep


def test_noalloc_rejects_a_call_beyond_the_scratch():
    """The generic path (fp32 inputs, a final state) at B4 H8 n2048 d64 needs
    more than the 64 MiB scratch: HLA_ERR_WORKSPACE before anything is
    enqueued, outputs untouched."""
    q, k, v = (x.to(DEV) for x in inputs.qkv(4, 8, 2048, 64, 64, torch.float32, seed=96))
    out = torch.full((4, 8, 2048, 64), 7.0, device=DEV)
    fin = hla.State.empty(32, 64, 64, DEV)
    with pytest.raises(hla.HlaError, match="WORKSPACE.*static scratch"):
        hla.forward_chunked_noalloc(q, k, v, chunk=64, out=out, final_state=fin)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

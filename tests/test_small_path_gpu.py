"""The short-sequence forward (n <= 256, d and dv in {16, 32}, no ridge,
denominator or states): two launches of a direct first-order map,
U = LA(Q, K, K; g) and out = LA(Q, U, V; g^2), checked through the C ABI
against the fp64 oracle (row error within the fp32 / bf16 gates).

The path keeps U (fp32, [B*H][n][d]) at the start of the workspace's data,
right after the control block, as these params have no flag region; the
tests read it back to confirm that the call took this path, and check it
against U computed from the oracle's inputs in fp64.
"""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs
from parity import TOL, row_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CTRL = 8192


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def u_fp64(q, k, gamma):
    """U = LA(Q, K, K; g) per head, in fp64 from the (exact) inputs."""
    q = q.double().numpy()
    k = k.double().numpy()
    B, H, n, d = q.shape
    t = np.arange(n)
    e = t[:, None] - t[None, :]
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            g = 1.0 if gamma is None else gamma[h]
            w = np.where(e >= 0, np.power(g, np.where(e >= 0, e, 0)), 0.0)
            out[b, h] = ((q[b, h] @ k[b, h].T) * w) @ k[b, h]
    return out


def run(B, H, n, d, dv, dtype, gamma, seed, chunk=0):
    import oracle
    q, k, v = inputs.qkv(B, H, n, d, dv, dtype, seed=seed)
    ws = torch.zeros(hla.workspace_size(B, H, n, d, dv, dtype=dtype, gamma=gamma), dtype=torch.uint8, device=DEV)
    out, den, st = hla.forward_chunked(q.to(DEV), k.to(DEV), v.to(DEV), gamma=gamma, chunk=chunk, workspace=ws)
    assert den is None and st is None
    torch.cuda.synchronize()
    ref = oracle.forward(q, k, v, gamma=gamma, want_state=False)[0]
    u = ws[CTRL:CTRL + 4 * B * H * n * d].view(torch.float32).reshape(B, H, n, d).cpu().double().numpy()
    return out.cpu(), ref, u, u_fp64(q, k, gamma), (q, k, v, ws)


@pytest.mark.parametrize("seed", [1000, 2000, 3000])
def test_small_fp32_workload_on_the_short_path(seed):
    w = inputs.SMALL_FP32
    out, ref, u, uref, _ = run(w.B, w.H, w.n, w.d, w.dv, w.dtype, None, seed)
    e = row_err(out, ref)
    print(f"row error {e:.3e}, U row error {row_err(u, uref):.3e}")
    assert e <= TOL[torch.float32]
    assert row_err(u, uref) <= TOL[torch.float32], "U is not where the short path keeps it: another path ran"


@pytest.mark.parametrize("B,H,n,d,dv", [
    (1, 1, 1, 16, 16),     # one token
    (2, 3, 15, 16, 32),    # less than one block
    (1, 2, 16, 32, 16),    # one whole block
    (2, 2, 17, 32, 32),    # one block and one token
    (1, 3, 100, 16, 16),   # ragged
    (3, 2, 255, 32, 32),   # the last row of the last block missing
    (1, 4, 256, 16, 32),   # the longest sequence the path takes
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("decay", ["none", "uniform", "per_head"])
def test_short_path_shapes_and_decays(B, H, n, d, dv, dtype, decay):
    gamma = {"none": None, "uniform": inputs.gamma_list_fp32([0.95] * H),
             "per_head": inputs.gamma_list_fp32([0.3, 0.9, 1.0, 0.75][:H] + [0.99] * max(0, H - 4))}[decay]
    out, ref, u, uref, _ = run(B, H, n, d, dv, dtype, gamma, seed=B * 131 + H * 17 + n)
    tol = TOL[dtype]
    e = row_err(out, ref)
    print(f"row error {e:.3e}")
    assert e <= tol
    assert row_err(u, uref) <= TOL[torch.float32]


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_the_chunk_setting_does_not_change_the_result(chunk):
    # the path has no chunks: every chunk setting gives the same bits
    a = run(1, 2, 200, 16, 16, torch.float32, [0.9, 1.0], seed=77)[0]
    b = run(1, 2, 200, 16, 16, torch.float32, [0.9, 1.0], seed=77, chunk=chunk)[0]
    assert torch.equal(a, b)


def test_short_path_agrees_with_the_chunked_path():
    # asking for den sends the same call to the chunked kernels; their out is the same numerator
    B, H, n, d, dv = 2, 2, 160, 32, 16
    g = inputs.gamma_list_fp32([0.9, 1.0])
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, dv, torch.float32, seed=5))
    o1, _, _ = hla.forward_chunked(q, k, v, gamma=g)
    o2, den, _ = hla.forward_chunked(q, k, v, gamma=g, return_den=True)
    assert den is not None
    assert row_err(o1.cpu(), o2.cpu().double()) <= 2 * TOL[torch.float32]


def test_longer_sequences_take_the_chunked_path():
    import oracle
    B, H, n, d = 1, 2, 257, 16
    q, k, v = inputs.qkv(B, H, n, d, d, torch.float32, seed=9)
    ws = torch.zeros(hla.workspace_size(B, H, n, d, d, dtype=torch.float32), dtype=torch.uint8, device=DEV)
    out, _, _ = hla.forward_chunked(q.to(DEV), k.to(DEV), v.to(DEV), workspace=ws)
    torch.cuda.synchronize()
    assert row_err(out.cpu(), oracle.forward(q, k, v, want_state=False)[0]) <= TOL[torch.float32]


def test_graph_replays_match_the_eager_call():
    B, H, n, d, dv = 1, 1, 256, 16, 16
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, dv, torch.float32, seed=1000))
    ws = torch.zeros(hla.workspace_size(B, H, n, d, dv, dtype=torch.float32), dtype=torch.uint8, device=DEV)
    out = torch.empty(B, H, n, dv, dtype=torch.float32, device=DEV)
    ref, _, _ = hla.forward_chunked(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        hla.forward_chunked(q, k, v, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hla.forward_chunked(q, k, v, workspace=ws, out=out)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        hla.forward_chunked(q, k, v, workspace=ws)  # eager work between the replays
        torch.cuda.synchronize()

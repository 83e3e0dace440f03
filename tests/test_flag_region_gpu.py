"""The one-launch kernels' flags hold launch epochs and nothing else.

A segment raises a flag by storing the running launch's epoch; a waiting
segment compares the flag with that epoch.  The epochs follow one 32-bit
linear congruential sequence (x -> 1664525 x + 1013904223 mod 2^32, from
zero), kept in the workspace's control block, so a flag left by an earlier
launch never matches.  Any other value in a flag word could match by
coincidence: the wait would pass early, and the segment would read sums not
yet published.  So every forward workspace keeps the flags in a region of
their own, after the control block, that no path's data reaches.  Through
the C ABI, these tests check that:

* the generic path's data misses the flags.  A d = 128 call with den takes
  the generic path, and its initial state is copied into the path's first
  data slot.  That state holds exactly the next launch's epoch.  The next
  one-launch call on the same workspace, with the same params, gives the
  same bits as on a fresh workspace, and the flag words hold only zeros and
  issued epochs;
* the same holds for AHLA, whose generic path copies its initial state
  first;
* the third-order forward keeps its two maps apart.  It runs a first-order
  map and then the second-order kernel in one call.  Afterwards, every word
  of the second kernel's flag region is zero or one of the two epochs.
"""
import sys

import numpy as np
import pytest
import torch

import associative_scan_sequence_amd as hla
import hla_inputs as inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF = torch.bfloat16
CTRL_WORDS = 8192 // 4  # the control block; the flag region follows it
EPOCH_WORD, LAUNCH_WORD, GIVE_UP_WORD = 65, 2, 3


@pytest.fixture(autouse=True)
def _name_the_case(request):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sys.stdout.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stdout.flush()
    yield
    torch.cuda.synchronize()


def next_epoch(e):
    return (e * 1664525 + 1013904223) & 0xFFFFFFFF


def issued(k):
    """The epochs of the first k launches on a zeroed control block."""
    out, e = [], 0
    for _ in range(k):
        e = next_epoch(e)
        out.append(e)
    return out


def words(ws, count):
    torch.cuda.synchronize()
    return ws[:4 * count].view(torch.int32).cpu().numpy().view(np.uint32)


def as_float(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def check_flags(ws, first, count, allowed):
    w = words(ws, first + count)[first:]
    bad = ~np.isin(w, np.array([0] + list(allowed), dtype=np.uint32))
    assert not bad.any(), f"{int(bad.sum())} flag words hold other values, first at {int(np.argmax(bad))}"


def segments(BH, nc, max_chunks):
    # about one workgroup per CU, at most max_chunks chunks per segment
    target = -(-256 // BH)
    L = min(max(-(-nc // target), 1), max_chunks)
    return -(-nc // L)


def higher_workspace(third, B, H, n, d, gamma):
    import ctypes
    b = hla._binding
    p, keep = b._params(B, H, n, d, d, 64, BF, gamma, 0.0, False)
    fn = b.load().hla_third_workspace_size if third else b.load().hla_ahla_workspace_size
    size = int(fn(ctypes.byref(p)))
    del keep
    return torch.zeros(size, dtype=torch.uint8, device=DEV)


def test_generic_state_call_leaves_the_d128_flags_alone():
    B, H, n, d = 1, 16, 2048, 128
    N = B * H
    g = inputs.gamma_list_fp32([0.99] * H)
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, d, BF, seed=3100))
    ws = torch.zeros(hla.workspace_size(B, H, n, d, d, dtype=BF, gamma=g), dtype=torch.uint8, device=DEV)
    ref, _, _ = hla.forward_chunked(q, k, v, gamma=g)  # a fresh workspace
    out1, _, _ = hla.forward_chunked(q, k, v, gamma=g, workspace=ws)
    assert torch.equal(out1, ref)
    ctrl = words(ws, CTRL_WORDS)
    e1 = issued(1)[0]
    assert ctrl[LAUNCH_WORD] == 1 and ctrl[EPOCH_WORD] == e1, "the d = 128 call did not take the one-launch kernel"
    # an initial state whose first head's S holds the next launch's epoch in every word
    init = inputs.random_state_fp32(N, d, d, seed=3101, scale=0.1)
    init = hla.State(*(t.to(DEV).contiguous() for t in init))
    init.S[0].fill_(float(as_float(next_epoch(e1))))
    hla.forward_chunked(q, k, v, gamma=g, init=init, return_den=True, workspace=ws)  # the generic path
    ctrl = words(ws, CTRL_WORDS)
    assert ctrl[LAUNCH_WORD] == 1, "the call with den ran a one-launch kernel"
    # the d = 128 kernel's flags: two words per segment, segments of whole 64-token chunks
    nc = -(-n // 64)
    p = min(max(-(-256 // N), 1), nc)
    P = -(-nc // -(-nc // p))
    check_flags(ws, CTRL_WORDS, 2 * N * P, [e1])
    out2, _, _ = hla.forward_chunked(q, k, v, gamma=g, workspace=ws)
    ctrl = words(ws, CTRL_WORDS)
    assert ctrl[LAUNCH_WORD] == 2 and ctrl[GIVE_UP_WORD] == 0
    assert torch.equal(out2, ref)


def test_generic_state_call_leaves_the_ahla_flags_alone():
    B, H, n, d = 2, 4, 700, 64
    N = B * H
    g = inputs.gamma_list_fp32([0.97, 0.9, 1.0, 0.99])
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, d, BF, seed=3200))
    ws = higher_workspace(False, B, H, n, d, g)
    ref, _, _ = hla.ahla_forward(q, k, v, gamma=g, chunk=64)
    out1, _, _ = hla.ahla_forward(q, k, v, gamma=g, chunk=64, workspace=ws)
    assert torch.equal(out1, ref)
    e1 = issued(1)[0]
    ctrl = words(ws, CTRL_WORDS)
    assert ctrl[LAUNCH_WORD] == 1 and ctrl[EPOCH_WORD] == e1, "AHLA did not take the one-launch kernel"
    st = hla.AhlaState.empty(N, d, d, DEV)
    gen = torch.Generator().manual_seed(3201)
    for t in st.tensors():
        t.copy_(0.1 * torch.randn(t.shape, generator=gen))
    st.rho.fill_(1.0)
    st.P[0].fill_(float(as_float(next_epoch(e1))))  # copied first into the generic path's data
    hla.ahla_forward(q, k, v, gamma=g, chunk=64, init=st, workspace=ws)
    ctrl = words(ws, CTRL_WORDS)
    assert ctrl[LAUNCH_WORD] == 1, "the call with a state ran a one-launch kernel"
    # the chained map's two flag sets: eight flags a line apart per segment each
    P = segments(N, -(-n // 64), 4)
    check_flags(ws, CTRL_WORDS, 2 * N * P * 8 * 32, [e1])
    out2, _, _ = hla.ahla_forward(q, k, v, gamma=g, chunk=64, workspace=ws)
    ctrl = words(ws, CTRL_WORDS)
    assert ctrl[LAUNCH_WORD] == 2 and ctrl[GIVE_UP_WORD] == 0
    assert torch.equal(out2, ref)


def test_third_order_maps_keep_their_flags_apart():
    B, H, n, d = 2, 4, 2048, 64
    N = B * H
    q, k, v = (x.to(DEV) for x in inputs.qkv(B, H, n, d, d, BF, seed=3300))
    ws = higher_workspace(True, B, H, n, d, None)
    ref, _, _ = hla.third_forward(q, k, v, chunk=64)
    for rep in range(2):
        out, _, _ = hla.third_forward(q, k, v, chunk=64, workspace=ws)
        assert torch.equal(out, ref), rep
        ctrl = words(ws, CTRL_WORDS)
        launches = 2 * (rep + 1)
        assert ctrl[LAUNCH_WORD] == launches and ctrl[GIVE_UP_WORD] == 0, "third order did not take the one-launch path"
        # the second-order kernel's flags: two rounds of eight flags a line apart per segment
        P = segments(N, -(-n // 64), 4)
        check_flags(ws, CTRL_WORDS, N * P * 2 * 8 * 32, issued(launches))

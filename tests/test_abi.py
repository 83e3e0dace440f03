"""The C ABI on the CPU: the library loads, exports every function that
include/hla.h declares, and rejects bad arguments on the host before any HIP
call (no test here launches a kernel, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import associative_scan_sequence_amd as hla
from associative_scan_sequence_amd._binding import CHiState, CParams, CState

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hla.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4

# Fake, 256-byte aligned, non-overlapping "device" addresses: validation only
# compares and range-checks them; every call below fails before any launch.
BASE = 0x7F0000000000


def addr(i):
    return BASE + i * (1 << 34)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return hla.load()


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("hla_forward_chunked", "hla_backward_chunked", "hla_decode_step", "hla_state_compose"):
        assert name in fns
    assert set(fns) == set(hla.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", hla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hla_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else with the public prefix leaks out
    assert exported == set(declared_functions())


def test_status_strings(lib):
    for code, name in hla._binding.STATUS.items():
        assert lib.hla_status_string(code).decode() == name


def params(**kw):
    d = dict(B=2, H=3, n=100, d=64, dv=32, chunk=0, dtype=1, gamma=None, ridge=0.0, normalize=0)
    d.update(kw)
    return CParams(d["B"], d["H"], d["n"], d["d"], d["dv"], d["chunk"], d["dtype"], d["gamma"],
                   d["ridge"], d["normalize"])


def fwd(lib, p, q=addr(1), k=addr(2), v=addr(3), out=addr(4), den=None, init=None, fin=None,
        ws=None, ws_bytes=None):
    need = lib.hla_forward_workspace_size(ctypes.byref(p))
    if ws is None:
        ws = addr(5)
    if ws_bytes is None:
        ws_bytes = need
    return lib.hla_forward_chunked(ctypes.byref(p), q, k, v, out, den,
                                   ctypes.byref(init) if init is not None else None,
                                   ctypes.byref(fin) if fin is not None else None, ws, ws_bytes, None)


def last(lib):
    return lib.hla_last_error().decode()


def test_workspace_size(lib):
    assert lib.hla_forward_workspace_size(ctypes.byref(params())) > 0
    assert lib.hla_forward_workspace_size(None) == 0
    assert lib.hla_forward_workspace_size(ctypes.byref(params(d=48))) == 0
    # grows with n and with the chunk count
    a = lib.hla_forward_workspace_size(ctypes.byref(params(n=1000)))
    b = lib.hla_forward_workspace_size(ctypes.byref(params(n=2000)))
    assert b > a


@pytest.mark.parametrize("d,w", [(16, 16), (32, 32), (64, 64), (128, 128)])
def test_default_chunk_is_d(lib, d, w):
    """chunk = 0 takes w = d (the chunk algebra costs O(w d + d^2) per token):
    the default call asks for the same workspace as the explicit chunk."""
    for dtype in (0, 1):
        size = lambda c: lib.hla_forward_workspace_size(  # noqa: E731
            ctypes.byref(params(d=d, dv=d, n=1000, chunk=c, dtype=dtype)))
        assert size(0) == size(w) > 0


@pytest.mark.parametrize("kw,code,frag", [
    (dict(B=0), INVALID, "B="),
    (dict(H=0), INVALID, "H="),
    (dict(n=-1), INVALID, "n="),
    (dict(d=48), UNSUPPORTED, "d=48"),
    (dict(dv=256), UNSUPPORTED, "dv=256"),
    (dict(chunk=24), UNSUPPORTED, "chunk"),
    (dict(dtype=7), INVALID, "dtype"),
    (dict(ridge=-1.0), INVALID, "ridge"),
    (dict(ridge=float("nan")), INVALID, "ridge"),
    (dict(normalize=2), INVALID, "normalize"),
    (dict(B=300, H=300), UNSUPPORTED, "65535"),
])
def test_forward_rejects_bad_params(lib, kw, code, frag):
    p = params(**kw)
    assert fwd(lib, p) == code
    assert frag in last(lib)


@pytest.mark.parametrize("g", [0.0, -0.5, 1.5, float("nan"), float("inf")])
def test_forward_rejects_bad_gamma(lib, g):
    arr = (ctypes.c_float * 3)(0.9, g, 0.9)
    p = params(gamma=ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)))
    assert fwd(lib, p) == INVALID
    assert "gamma[1]" in last(lib)


def test_forward_rejects_null_and_misaligned(lib):
    p = params()
    assert fwd(lib, p, q=None) == INVALID and "q is NULL" in last(lib)
    assert fwd(lib, p, out=None) == INVALID and "out is NULL" in last(lib)
    assert fwd(lib, p, k=addr(2) + 4) == ALIGN and "k is not" in last(lib)
    assert fwd(lib, p, den=addr(6) + 8) == ALIGN and "den" in last(lib)


def test_forward_rejects_small_or_missing_workspace(lib):
    p = params()
    need = lib.hla_forward_workspace_size(ctypes.byref(p))
    assert fwd(lib, p, ws_bytes=need - 1) == WORKSPACE
    assert lib.hla_forward_chunked(ctypes.byref(p), addr(1), addr(2), addr(3), addr(4), None, None,
                                   None, None, need, None) == WORKSPACE
    assert fwd(lib, p, ws=addr(5) + 16) == ALIGN


def test_forward_rejects_aliasing(lib):
    p = params()
    # out overlapping q
    assert fwd(lib, p, out=addr(1) + 256) == INVALID and "out overlaps q" in last(lib)
    # den overlapping out
    assert fwd(lib, p, den=addr(4) + 1024) == INVALID and "overlaps" in last(lib)
    # workspace overlapping v
    assert fwd(lib, p, ws=addr(3)) == INVALID and "workspace overlaps v" in last(lib)
    # final state overlapping init
    st = CState(addr(7), addr(8), addr(9), addr(10), addr(11), None)
    st2 = CState(addr(12), addr(13), addr(14), addr(10), addr(15), None)
    assert fwd(lib, p, init=st, fin=st2) == INVALID and "overlaps init.G" in last(lib)


def test_forward_rejects_incomplete_state(lib):
    p = params()
    st = CState(addr(7), addr(8), None, addr(10), addr(11), None)
    assert fwd(lib, p, init=st) == INVALID and "init->m is NULL" in last(lib)
    st = CState(addr(7), addr(8), addr(9), addr(10) + 4, addr(11), None)
    assert fwd(lib, p, fin=st) == ALIGN and "final_state->G" in last(lib)


def test_forward_empty_sequence_without_state_is_a_no_op(lib):
    p = params(n=0)
    assert lib.hla_forward_chunked(ctypes.byref(p), None, None, None, None, None, None, None,
                                   addr(5), lib.hla_forward_workspace_size(ctypes.byref(p)),
                                   None) == OK


def bwd(lib, p, q=addr(1), k=addr(2), v=addr(3), dout=addr(4), dq=addr(5), dk=addr(6), dv=addr(7),
        ws=None, ws_bytes=None, init=None, dinit=None, dfinal=None):
    need = lib.hla_backward_workspace_size(ctypes.byref(p))
    if ws is None:
        ws = addr(8)
    if ws_bytes is None:
        ws_bytes = need
    return lib.hla_backward_chunked(ctypes.byref(p), q, k, v, ctypes.byref(init) if init is not None else None,
                                    dout, dq, dk, dv, ctypes.byref(dfinal) if dfinal is not None else None,
                                    ctypes.byref(dinit) if dinit is not None else None,
                                    ws, ws_bytes, None)


def test_backward_workspace_size(lib):
    assert lib.hla_backward_workspace_size(ctypes.byref(params())) > 0
    assert lib.hla_backward_workspace_size(None) == 0
    assert lib.hla_backward_workspace_size(ctypes.byref(params(d=48))) == 0
    assert lib.hla_backward_workspace_size(ctypes.byref(params(n=0))) == 0
    a = lib.hla_backward_workspace_size(ctypes.byref(params(n=1000)))
    assert lib.hla_backward_workspace_size(ctypes.byref(params(n=2000))) > a


@pytest.mark.parametrize("kw,code,frag", [
    (dict(B=0), INVALID, "B="),
    (dict(n=-1), INVALID, "n="),
    (dict(d=48), UNSUPPORTED, "d=48"),
    (dict(chunk=24), UNSUPPORTED, "chunk"),
    (dict(ridge=-1.0), INVALID, "ridge"),
    (dict(normalize=2), INVALID, "normalize"),
])
def test_backward_rejects_bad_params(lib, kw, code, frag):
    assert bwd(lib, params(**kw)) == code
    assert frag in last(lib)


def test_backward_rejects_bad_pointers_and_workspace(lib):
    p = params()
    assert bwd(lib, p, dout=None) == INVALID and "dout is NULL" in last(lib)
    assert bwd(lib, p, dk=None) == INVALID and "dk is NULL" in last(lib)
    assert bwd(lib, p, dv=addr(7) + 4) == ALIGN and "dv is not" in last(lib)
    need = lib.hla_backward_workspace_size(ctypes.byref(p))
    assert bwd(lib, p, ws_bytes=need - 1) == WORKSPACE
    assert bwd(lib, p, ws=addr(8) + 16) == ALIGN and "256-byte" in last(lib)
    assert lib.hla_backward_chunked(ctypes.byref(p), addr(1), addr(2), addr(3), None, addr(4), addr(5),
                                    addr(6), addr(7), None, None, None, need, None) == WORKSPACE
    bad = CState(addr(9), addr(10), None, addr(12), addr(13), None)
    assert bwd(lib, p, dinit=bad) == INVALID and "dinit->m is NULL" in last(lib)
    bad = CState(addr(9) + 4, addr(10), addr(11), addr(12), addr(13), None)
    assert bwd(lib, p, dinit=bad) == ALIGN and "dinit->S is not" in last(lib)


def test_backward_rejects_aliasing(lib):
    p = params()
    assert bwd(lib, p, dq=addr(1) + 256) == INVALID and "dq overlaps q" in last(lib)
    assert bwd(lib, p, dk=addr(5) + 512) == INVALID and "overlaps" in last(lib)
    assert bwd(lib, p, dv=addr(4)) == INVALID and "dv overlaps dout" in last(lib)
    assert bwd(lib, p, ws=addr(2)) == INVALID and "workspace overlaps k" in last(lib)
    st = CState(addr(9), addr(10), addr(11), addr(12), addr(13), None)
    assert bwd(lib, p, dq=addr(10), init=st) == INVALID and "dq overlaps init.C" in last(lib)
    assert bwd(lib, p, init=CState(addr(9), None, addr(11), addr(12), addr(13), None)) == INVALID
    assert "init->C is NULL" in last(lib)
    dst = CState(addr(14), addr(15), addr(16), addr(17), addr(18), None)
    assert bwd(lib, p, init=st, dinit=CState(addr(9), addr(15), addr(16), addr(17), addr(18), None)) \
        == INVALID and "dinit.S overlaps init.S" in last(lib)
    assert bwd(lib, p, dinit=CState(addr(14), addr(15), addr(16), addr(17), addr(18), addr(5))) \
        == INVALID and "overlaps" in last(lib)
    assert bwd(lib, p, dq=addr(14), dinit=dst) == INVALID and "overlaps" in last(lib)
    fst = CState(addr(19), addr(20), addr(21), addr(22), addr(23), None)
    assert bwd(lib, p, dfinal=CState(addr(19), None, addr(21), addr(22), addr(23), None)) == INVALID
    assert "dfinal->C is NULL" in last(lib)
    assert bwd(lib, p, dfinal=fst, dinit=CState(addr(14), addr(20), addr(16), addr(17), addr(18), None)) \
        == INVALID and "dinit.C overlaps dfinal.C" in last(lib)
    assert bwd(lib, p, dfinal=fst, dk=addr(21)) == INVALID and "dk overlaps dfinal.m" in last(lib)
    g = (ctypes.c_float * 2)(0.9, 1e-7)
    pg = params(H=2, gamma=ctypes.cast(g, ctypes.POINTER(ctypes.c_float)))
    assert bwd(lib, pg, dfinal=fst) == UNSUPPORTED and "gamma[1]" in last(lib)


def test_backward_empty_sequence_is_a_no_op(lib):
    p = params(n=0)
    assert lib.hla_backward_chunked(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                                    None, None, 0, None) == OK


def dec(lib, p, state, q=addr(1), k=addr(2), v=addr(3), out=addr(4), den=None):
    return lib.hla_decode_step(ctypes.byref(p), q, k, v,
                               ctypes.byref(state) if state is not None else None, out, den, None)


def test_decode_rejects_bad_arguments(lib):
    st = CState(addr(7), addr(8), addr(9), addr(10), addr(11), addr(12))
    assert dec(lib, params(n=2), st) == INVALID and "n = 1" in last(lib)
    assert dec(lib, params(n=1, d=8), st) == UNSUPPORTED
    assert dec(lib, params(n=1), None) == INVALID
    assert dec(lib, params(n=1), st, q=None) == INVALID
    assert dec(lib, params(n=1), st, out=addr(8)) == INVALID and "overlaps" in last(lib)
    assert dec(lib, params(n=1), CState(addr(7), addr(8), addr(9), None, addr(11), None)) == INVALID
    assert dec(lib, params(n=1), st, v=addr(3) + 2) == ALIGN


def test_compose_rejects_bad_arguments(lib):
    a = CState(addr(1), addr(2), addr(3), addr(4), addr(5), None)
    b = CState(addr(6), addr(7), addr(8), addr(9), addr(10), None)
    r = CState(addr(11), addr(12), addr(13), addr(14), addr(15), None)
    comp = lambda cnt, d, dv, x, y, z: lib.hla_state_compose(  # noqa: E731
        cnt, d, dv, ctypes.byref(x) if x else None, ctypes.byref(y) if y else None,
        ctypes.byref(z) if z else None, None)
    assert comp(-1, 64, 64, a, b, r) == INVALID
    assert comp(4, 64, 80, a, b, r) == UNSUPPORTED
    assert comp(4, 64, 64, a, None, r) == INVALID
    assert comp(0, 64, 64, a, b, r) == OK  # empty batch: nothing to do
    assert comp(4, 64, 64, a, b, CState(addr(11), addr(2), addr(13), addr(14), addr(15), None)) == INVALID
    assert "result.C overlaps earlier.C" in last(lib)


def test_last_error_is_cleared_by_success(lib):
    assert fwd(lib, params(B=0)) == INVALID
    assert last(lib) != ""
    p = params(n=0)
    assert lib.hla_forward_chunked(ctypes.byref(p), None, None, None, None, None, None, None,
                                   addr(5), 1 << 30, None) == OK
    assert last(lib) == ""


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError, match="HIP device"):
        hla.forward_chunked(q, q, q)


def test_noalloc_validates_before_any_device_call(lib):
    """hla_forward_chunked_noalloc takes the forward's arguments without a
    workspace; bad arguments and calls whose path needs more than the static
    scratch fail on the host, before the scratch is looked up on a device."""
    def call(p, **kw):
        a = dict(q=addr(1), k=addr(2), v=addr(3), out=addr(4), den=None, init=None, fin=None)
        a.update(kw)
        return lib.hla_forward_chunked_noalloc(ctypes.byref(p), a["q"], a["k"], a["v"], a["out"], a["den"],
                                               ctypes.byref(a["init"]) if a["init"] is not None else None,
                                               ctypes.byref(a["fin"]) if a["fin"] is not None else None, None)
    assert call(params(d=48)) == UNSUPPORTED
    assert call(params(), q=None) == INVALID and "q is NULL" in last(lib)
    # the generic path (fp32, a final state) at B4 H8 n2048 d64 needs more than 64 MiB
    fin = CState(*[addr(10 + i) for i in range(6)])
    p = params(B=4, H=8, n=2048, d=64, dv=64, chunk=64, dtype=0)
    assert call(p, fin=fin) == WORKSPACE
    assert "static scratch" in last(lib) and str(hla._binding.NOALLOC_SCRATCH_BYTES) in last(lib)


def mq(lib, p, kv_heads, state, q=addr(1), k=addr(2), v=addr(3), out=addr(4), den=None):
    return lib.hla_decode_step_mq(ctypes.byref(p), kv_heads, q, k, v,
                                  ctypes.byref(state) if state is not None else None, out, den, None)


def test_decode_mq_rejects_bad_arguments(lib):
    st = CState(addr(7), addr(8), addr(9), addr(10), addr(11), addr(12))
    p = params(B=2, H=4, n=1, d=64, dv=64)
    assert mq(lib, p, 3, st) == INVALID and "divide H=4" in last(lib)
    assert mq(lib, p, 0, st) == INVALID and "kv_heads=0" in last(lib)
    assert mq(lib, params(B=2, H=4, n=1, d=16, dv=64), 2, st) == UNSUPPORTED and "packed" in last(lib)
    assert mq(lib, params(B=2, H=4, n=2, d=64, dv=64), 2, st) == INVALID and "n = 1" in last(lib)
    # one decay per group of heads that share a key moment
    g = (ctypes.c_float * 4)(0.9, 0.8, 0.7, 0.7)
    pg = params(B=2, H=4, n=1, d=64, dv=64, gamma=ctypes.cast(g, ctypes.POINTER(ctypes.c_float)))
    assert mq(lib, pg, 2, st) == INVALID and "gamma[1]" in last(lib)
    assert mq(lib, p, 2, None) == INVALID and "state is NULL" in last(lib)
    assert mq(lib, p, 2, st, q=None) == INVALID and "q is NULL" in last(lib)
    assert mq(lib, p, 2, st, k=addr(2) + 4) == ALIGN and "k is not" in last(lib)
    assert mq(lib, p, 2, CState(addr(7), addr(8), None, addr(10), addr(11), None)) == INVALID
    # out written over the (packed, per-group) key moment
    assert mq(lib, p, 2, st, out=addr(7) + 1024) == INVALID and "overlaps" in last(lib)


def test_key_moment_pack_rejects_bad_arguments(lib):
    for fn in (lib.hla_key_moment_pack, lib.hla_key_moment_unpack):
        assert fn(-1, 64, addr(1), addr(2), None) == INVALID
        assert fn(4, 48, addr(1), addr(2), None) == UNSUPPORTED and "d=48" in last(lib)
        assert fn(0, 64, None, None, None) == OK  # nothing to do
        assert fn(4, 64, None, addr(2), None) == INVALID and "NULL" in last(lib)
        assert fn(4, 64, addr(1) + 8, addr(2), None) == ALIGN
        assert fn(4, 64, addr(1), addr(1) + 4096, None) == INVALID and "aliasing" in last(lib)
        assert fn(1 << 20, 128, addr(1), addr(2), None) == UNSUPPORTED and "too large" in last(lib)


def hi_fwd(lib, fn, size_fn, p, q=addr(1), k=addr(2), v=addr(3), out=addr(4), den=None, init=None,
           fin=None, ws=None, ws_bytes=None):
    need = size_fn(ctypes.byref(p))
    return fn(ctypes.byref(p), q, k, v, out, den, ctypes.byref(init) if init is not None else None,
              ctypes.byref(fin) if fin is not None else None, addr(5) if ws is None else ws,
              need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("third", [False, True])
def test_ahla_and_third_forward_reject_bad_arguments(lib, third):
    fn = lib.hla_third_forward if third else lib.hla_ahla_forward
    size_fn = lib.hla_third_workspace_size if third else lib.hla_ahla_workspace_size
    call = lambda p, **kw: hi_fwd(lib, fn, size_fn, p, **kw)  # noqa: E731
    p = params(n=200, d=64, dv=64)
    assert size_fn(ctypes.byref(p)) > 0
    assert size_fn(None) == 0 and size_fn(ctypes.byref(params(d=48))) == 0
    assert size_fn(ctypes.byref(params(dtype=7))) == 0
    assert fn(None, addr(1), addr(2), addr(3), addr(4), None, None, None, addr(5), 1 << 30, None) == INVALID
    assert call(params(B=0)) == INVALID and "B=" in last(lib)
    assert call(params(dtype=7)) == INVALID and "dtype" in last(lib)
    assert call(params(d=48)) == UNSUPPORTED
    # neither operator has a ridge term
    assert call(params(ridge=0.5)) == UNSUPPORTED and "ridge" in last(lib)
    g = (ctypes.c_float * 3)(1.0, 0.9, 1.0)
    pg = params(gamma=ctypes.cast(g, ctypes.POINTER(ctypes.c_float)))
    if third:  # masked third order here is the undecayed operator
        assert call(pg) == UNSUPPORTED and "gamma[1]" in last(lib)
    else:
        assert call(pg, ws_bytes=0) == WORKSPACE  # a decay is fine for AHLA: the next check fires
    assert call(p, q=None) == INVALID and "q is NULL" in last(lib)
    assert call(p, v=addr(3) + 4) == ALIGN and "v is not" in last(lib)
    need = size_fn(ctypes.byref(p))
    assert call(p, ws_bytes=need - 1) == WORKSPACE
    assert call(p, ws=addr(5) + 16) == ALIGN and "workspace" in last(lib)
    assert call(p, out=addr(2) + 256) == INVALID and "out overlaps k" in last(lib)
    # field order: hla_third_state (S, P, m, F, Fd), hla_ahla_state (P, m, E, n, rho)
    names = ("S", "P", "m", "F", "Fd") if third else ("P", "m", "E", "n", "rho")
    full = CHiState(addr(7), addr(8), addr(9), addr(10), addr(11))
    gap = CHiState(addr(7), None, addr(9), addr(10), addr(11))
    assert call(p, init=gap) == INVALID and f"init->{names[1]} is NULL" in last(lib)
    mis = CHiState(addr(7), addr(8), addr(9) + 4, addr(10), addr(11))
    assert call(p, fin=mis) == ALIGN and f"final_state->{names[2]}" in last(lib)
    # a final-state array written over an init array; the message uses the header's names
    fin = CHiState(addr(12), addr(13), addr(14), addr(10), addr(15))
    assert call(p, init=full, fin=fin) == INVALID
    assert f"final_state.{names[3]} overlaps init.{names[3]}" in last(lib)
    # nothing to do: no tokens and no final state
    assert call(params(n=0), q=None, k=None, v=None, out=None, ws=None) == OK


@pytest.mark.parametrize("third", [False, True])
def test_ahla_and_third_decode_reject_bad_arguments(lib, third):
    fn = lib.hla_third_decode_step if third else lib.hla_ahla_decode_step
    st = CHiState(addr(7), addr(8), addr(9), addr(10), addr(11))
    call = lambda p, state=st, q=addr(1), out=addr(4): fn(  # noqa: E731
        ctypes.byref(p) if p is not None else None, q, addr(2), addr(3),
        ctypes.byref(state) if state is not None else None, out, None, None)
    assert call(params(n=1), state=None) == INVALID and "state is NULL" in last(lib)
    assert call(None) == INVALID and "params is NULL" in last(lib)
    assert call(params(n=2)) == INVALID and "n = 1" in last(lib)
    assert call(params(n=1, ridge=1.0)) == UNSUPPORTED
    assert call(params(n=1), q=None) == INVALID and "q is NULL" in last(lib)
    assert call(params(n=1), q=addr(1) + 2) == ALIGN
    hole = CHiState(addr(7), addr(8), addr(9), None, addr(11))
    assert call(params(n=1), state=hole) == INVALID and "is NULL" in last(lib)
    assert call(params(n=1), out=addr(8)) == INVALID and "overlaps" in last(lib)


def test_path_choice_with_a_state_at_every_width(lib):
    """Choosing the kernel path for a call with a state reads the batch size
    (the d = 128 one-launch kernel checks its segment count): every width,
    both dtypes, through the no-alloc entry point, whose validation chooses
    the path before anything touches a device.  A call either fits the static
    scratch (and then fails here, without a GPU, looking up its address) or is
    rejected for its size; it never reaches a kernel."""
    init = CState(*[addr(10 + i) for i in range(6)])
    fin = CState(*[addr(20 + i) for i in range(6)])
    for d in (16, 32, 64, 128):
        for dtype in (0, 1):
            for n in (1, 300, 4096):
                for ini in (None, init):
                    p = params(B=1, H=16, n=n, d=d, dv=d, dtype=dtype)
                    st = lib.hla_forward_chunked_noalloc(
                        ctypes.byref(p), addr(1), addr(2), addr(3), addr(4), None,
                        ctypes.byref(ini) if ini is not None else None, ctypes.byref(fin), None)
                    assert st in (WORKSPACE, 5), (d, dtype, n, st, last(lib))

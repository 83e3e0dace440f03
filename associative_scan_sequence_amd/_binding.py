"""ctypes binding of libhla.so (include/hla.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device addresses and the current HIP stream are passed to
the C ABI, and a non-OK status is raised as :class:`HlaError`.  Every step of
the computation runs in the library's HIP kernels; there is no fallback, and
a missing library raises at load time.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhla.so")

HLA_F32, HLA_BF16 = 0, 1
STATUS = {0: "HLA_OK", 1: "HLA_ERR_INVALID_ARGUMENT", 2: "HLA_ERR_UNSUPPORTED",
          3: "HLA_ERR_ALIGNMENT", 4: "HLA_ERR_WORKSPACE", 5: "HLA_ERR_DEVICE"}
EXPORTED = ("hla_forward_workspace_size", "hla_forward_chunked", "hla_forward_chunked_noalloc",
            "hla_backward_workspace_size", "hla_backward_chunked", "hla_decode_step", "hla_decode_step_mq",
            "hla_key_moment_pack", "hla_key_moment_unpack", "hla_state_compose", "hla_status_string",
            "hla_last_error", "hla_ahla_workspace_size", "hla_third_workspace_size", "hla_ahla_forward",
            "hla_third_forward", "hla_ahla_decode_step", "hla_third_decode_step")
NOALLOC_SCRATCH_BYTES = 64 << 20  # HLA_NOALLOC_SCRATCH_BYTES


class CState(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in ("S", "C", "m", "G", "h", "rho")]


class CHiState(ctypes.Structure):  # hla_ahla_state (P, m, E, n, rho) / hla_third_state (S, P, m, F, Fd)
    _fields_ = [(name, ctypes.c_void_p) for name in ("a", "b", "c", "d", "e")]


class CParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("n", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("gamma", ctypes.POINTER(ctypes.c_float)),
                ("ridge", ctypes.c_float), ("normalize", ctypes.c_int32)]


class HlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {detail}")


_lib = None


def load(path: str = LIB_PATH):
    """Load libhla.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m associative_scan_sequence_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp, ps = ctypes.POINTER(CParams), ctypes.POINTER(CState)
    lib.hla_forward_workspace_size.argtypes = [pp]
    lib.hla_forward_workspace_size.restype = sz
    lib.hla_forward_chunked.argtypes = [pp, vp, vp, vp, vp, vp, ps, ps, vp, sz, vp]
    lib.hla_forward_chunked.restype = ctypes.c_int
    lib.hla_forward_chunked_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, ps, ps, vp]
    lib.hla_forward_chunked_noalloc.restype = ctypes.c_int
    lib.hla_backward_workspace_size.argtypes = [pp]
    lib.hla_backward_workspace_size.restype = sz
    lib.hla_backward_chunked.argtypes = [pp, vp, vp, vp, ps, vp, vp, vp, vp, ps, ps, vp, sz, vp]
    lib.hla_backward_chunked.restype = ctypes.c_int
    lib.hla_decode_step.argtypes = [pp, vp, vp, vp, ps, vp, vp, vp]
    lib.hla_decode_step.restype = ctypes.c_int
    lib.hla_decode_step_mq.argtypes = [pp, ctypes.c_int32, vp, vp, vp, ps, vp, vp, vp]
    lib.hla_decode_step_mq.restype = ctypes.c_int
    for fn in (lib.hla_key_moment_pack, lib.hla_key_moment_unpack):
        fn.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
        fn.restype = ctypes.c_int
    lib.hla_state_compose.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ps, ps, ps, vp]
    lib.hla_state_compose.restype = ctypes.c_int
    for fn in (lib.hla_ahla_workspace_size, lib.hla_third_workspace_size):
        fn.argtypes = [pp]
        fn.restype = sz
    p5 = ctypes.POINTER(CHiState)
    for fn in (lib.hla_ahla_forward, lib.hla_third_forward):
        fn.argtypes = [pp, vp, vp, vp, vp, vp, p5, p5, vp, sz, vp]
        fn.restype = ctypes.c_int
    for fn in (lib.hla_ahla_decode_step, lib.hla_third_decode_step):
        fn.argtypes = [pp, vp, vp, vp, p5, vp, vp, vp]
        fn.restype = ctypes.c_int
    lib.hla_status_string.argtypes = [ctypes.c_int]
    lib.hla_status_string.restype = ctypes.c_char_p
    lib.hla_last_error.argtypes = []
    lib.hla_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise HlaError(status, load().hla_last_error().decode())


@dataclass
class State:
    """Segment summary for B*H heads, fp32 device tensors:
    S [N,d,d], C [N,d,dv], m [N,d], G [N,d,dv], h [N,d], rho [N] (or None)."""
    S: torch.Tensor
    C: torch.Tensor
    m: torch.Tensor
    G: torch.Tensor
    h: torch.Tensor
    rho: Optional[torch.Tensor] = None

    @staticmethod
    def empty(N: int, d: int, dv: int, device, with_rho: bool = True) -> "State":
        f = dict(dtype=torch.float32, device=device)
        return State(torch.empty(N, d, d, **f), torch.empty(N, d, dv, **f), torch.empty(N, d, **f),
                     torch.empty(N, d, dv, **f), torch.empty(N, d, **f),
                     torch.empty(N, **f) if with_rho else None)

    @staticmethod
    def zeros(N: int, d: int, dv: int, device) -> "State":
        s = State.empty(N, d, dv, device)
        for t in (s.S, s.C, s.m, s.G, s.h):
            t.zero_()
        s.rho.fill_(1.0)
        return s

    def tensors(self):
        return (self.S, self.C, self.m, self.G, self.h, self.rho)

    def c(self) -> CState:
        for t in self.tensors():
            if t is not None:
                _need(t, "state", (torch.float32,))
        return CState(*[t.data_ptr() if t is not None else None for t in self.tensors()])

    def clone(self) -> "State":
        return State(*[t.clone() if t is not None else None for t in self.tensors()])


def _need(t: torch.Tensor, name: str, dtypes):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _params(B, H, n, d, dv, chunk, dtype, gamma, ridge, normalize):
    if dtype == torch.bfloat16:
        dt = HLA_BF16
    elif dtype == torch.float32:
        dt = HLA_F32
    else:
        raise TypeError(f"q/k/v dtype must be bfloat16 or float32, got {dtype}")
    garr = None
    keep = None
    if gamma is not None:
        g = [float(x) for x in (gamma if isinstance(gamma, Sequence) or hasattr(gamma, "__len__") else [gamma] * H)]
        if len(g) == 1 and H > 1:
            g = g * H
        if len(g) != H:
            raise ValueError(f"gamma has {len(g)} entries for H={H}")
        keep = (ctypes.c_float * H)(*g)
        garr = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    p = CParams(B, H, n, d, dv, int(chunk), dt, garr, float(ridge), int(bool(normalize)))
    return p, keep


def give_ups(workspace: torch.Tensor) -> int:
    """Waits that gave up in the one-launch kernels that ran on this
    forward workspace (control word 3; synchronises with the device).  A
    give-up makes the outputs that depend on it NaN; zero is the normal
    value."""
    return int(workspace[12:16].view(torch.int32).item())


def workspace_size(B, H, n, d, dv, *, chunk=0, dtype=torch.bfloat16, gamma=None, ridge=0.0,
                   normalize=False) -> int:
    """Bytes of forward workspace; allocate it zero-filled (``torch.zeros``)."""
    p, _keep = _params(B, H, n, d, dv, chunk, dtype, gamma, ridge, normalize)
    return int(load().hla_forward_workspace_size(ctypes.byref(p)))


def forward_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, gamma=None,
                    ridge: float = 0.0, normalize: bool = False, chunk: int = 0,
                    init: Optional[State] = None, return_state: bool = False,
                    return_den: bool = False, out: Optional[torch.Tensor] = None,
                    den: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    final_state: Optional[State] = None):
    """Masked second-order HLA forward through ``hla_forward_chunked``.

    q, k: [B,H,n,d]; v: [B,H,n,dv] (bf16 or fp32, same dtype, on one device).
    ``final_state``: a State to write the final state into (implies
    return_state; otherwise one is allocated when return_state is set).
    Returns (out [B,H,n,dv] fp32, den [B,H,n] fp32 or None, final State or None).
    """
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (torch.bfloat16, torch.float32))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}: "
                         "expected q,k [B,H,n,d] and v [B,H,n,dv]")
    B, H, n, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    p, _keep = _params(B, H, n, d, dv, chunk, q.dtype, gamma, ridge, normalize)
    need = int(lib.hla_forward_workspace_size(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty(B, H, n, dv, dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,))
    if den is None and return_den:
        den = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    if den is not None:
        _need(den, "den", (torch.float32,))
    fin = final_state if final_state is not None else (State.empty(B * H, d, dv, dev) if return_state else None)
    ini_c = init.c() if init is not None else None
    fin_c = fin.c() if fin is not None else None
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.hla_forward_chunked(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 out.data_ptr(), den.data_ptr() if den is not None else None,
                                 ctypes.byref(ini_c) if ini_c is not None else None,
                                 ctypes.byref(fin_c) if fin_c is not None else None,
                                 ws_ptr, ws_bytes, _stream(dev))
    _check(st)
    return out, den, fin


def forward_chunked_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, gamma=None,
                            ridge: float = 0.0, normalize: bool = False, chunk: int = 0,
                            init: Optional[State] = None, out: Optional[torch.Tensor] = None,
                            den: Optional[torch.Tensor] = None, final_state: Optional[State] = None):
    """The forward through ``hla_forward_chunked_noalloc``: no workspace, the
    library's static scratch instead (calls on one GPU must not overlap in
    time).  With ``out``, ``den`` and ``final_state`` given nothing is
    allocated here either.  Returns (out, den or None, final_state or None)."""
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (torch.bfloat16, torch.float32))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}: "
                         "expected q,k [B,H,n,d] and v [B,H,n,dv]")
    B, H, n, d = q.shape
    dv = v.shape[-1]
    p, _keep = _params(B, H, n, d, dv, chunk, q.dtype, gamma, ridge, normalize)
    if out is None:
        out = torch.empty(B, H, n, dv, dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,))
    if den is not None:
        _need(den, "den", (torch.float32,))
    ini_c = init.c() if init is not None else None
    fin_c = final_state.c() if final_state is not None else None
    st = lib.hla_forward_chunked_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         out.data_ptr(), den.data_ptr() if den is not None else None,
                                         ctypes.byref(ini_c) if ini_c is not None else None,
                                         ctypes.byref(fin_c) if fin_c is not None else None,
                                         _stream(q.device))
    _check(st)
    return out, den, final_state


def backward_workspace_size(B, H, n, d, dv, *, chunk=0, dtype=torch.bfloat16, gamma=None,
                            ridge=0.0, normalize=False) -> int:
    """Bytes of backward workspace (any contents; no zero fill needed)."""
    p, _keep = _params(B, H, n, d, dv, chunk, dtype, gamma, ridge, normalize)
    return int(load().hla_backward_workspace_size(ctypes.byref(p)))


def backward_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, *,
                     gamma=None, ridge: float = 0.0, normalize: bool = False, chunk: int = 0,
                     init: Optional[State] = None, workspace: Optional[torch.Tensor] = None,
                     grads=None, dinit: Optional[State] = None, dfinal: Optional[State] = None):
    """Gradients of sum(out * dout) through ``hla_backward_chunked``, from the
    zero state or from ``init``.  q, k: [B,H,n,d]; v, dout: [B,H,n,dv] (dout
    fp32).  Returns (dq, dk, dv), fp32, shaped like q, k, v; ``grads`` may
    supply them.  ``dinit``, if given, receives the gradient with respect to
    the initial state (``init``, or the zero state); ``dfinal``, if given, is
    a gradient flowing into the final state (added to the loss as
    sum <final part, dfinal part>)."""
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (torch.bfloat16, torch.float32))
    _need(dout, "dout", (torch.float32,))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3] \
            or dout.shape != v.shape:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} "
                         f"dout{tuple(dout.shape)}: expected q,k [B,H,n,d], v,dout [B,H,n,dv]")
    B, H, n, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    p, _keep = _params(B, H, n, d, dv, chunk, q.dtype, gamma, ridge, normalize)
    need = int(lib.hla_backward_workspace_size(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if grads is None:
        grads = (torch.empty(B, H, n, d, dtype=torch.float32, device=dev),
                 torch.empty(B, H, n, d, dtype=torch.float32, device=dev),
                 torch.empty(B, H, n, dv, dtype=torch.float32, device=dev))
    for name, t in zip(("dq", "dk", "dv"), grads):
        _need(t, name, (torch.float32,))
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ini_c = init.c() if init is not None else None
    dini_c = dinit.c() if dinit is not None else None
    dfin_c = dfinal.c() if dfinal is not None else None
    st = lib.hla_backward_chunked(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  ctypes.byref(ini_c) if ini_c is not None else None, dout.data_ptr(),
                                  grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                                  ctypes.byref(dfin_c) if dfin_c is not None else None,
                                  ctypes.byref(dini_c) if dini_c is not None else None,
                                  ws_ptr, ws_bytes, _stream(dev))
    _check(st)
    return grads


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: State, *, gamma=None,
                ridge: float = 0.0, normalize: bool = False, return_den: bool = False,
                out: Optional[torch.Tensor] = None, den: Optional[torch.Tensor] = None):
    """One token per state through ``hla_decode_step``; ``state`` is updated in
    place.  q, k: [B,H,d]; v: [B,H,dv].  Returns (out [B,H,dv], den [B,H] or None)."""
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (torch.bfloat16, torch.float32))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q,k [B,H,d] and v [B,H,dv]")
    B, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    p, _keep = _params(B, H, 1, d, dv, 0, q.dtype, gamma, ridge, normalize)
    if out is None:
        out = torch.empty(B, H, dv, dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,))
    if den is None and return_den:
        den = torch.empty(B, H, dtype=torch.float32, device=dev)
    sc = state.c()
    st = lib.hla_decode_step(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             ctypes.byref(sc), out.data_ptr(),
                             den.data_ptr() if den is not None else None, _stream(dev))
    _check(st)
    return out, den


@dataclass
class MqState:
    """Decode state with the key moment shared by groups of query heads and
    stored packed (hla_mq_state): S [B*kv_heads, d*(d+1)/2]; C, G
    [B*H, d, dv]; m, h [B*H, d]; rho [B*kv_heads] or None (fp32, device)."""
    S: torch.Tensor
    C: torch.Tensor
    m: torch.Tensor
    G: torch.Tensor
    h: torch.Tensor
    rho: Optional[torch.Tensor] = None

    def tensors(self):
        return (self.S, self.C, self.m, self.G, self.h, self.rho)

    def c(self) -> CState:
        for t in self.tensors():
            if t is not None:
                _need(t, "state", (torch.float32,))
        return CState(*[t.data_ptr() if t is not None else None for t in self.tensors()])


def packed_size(d: int) -> int:
    return d * (d + 1) // 2


def key_moment_pack(S: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Full symmetric key moments [N,d,d] -> packed [N, d(d+1)/2] (``hla_key_moment_pack``)."""
    _need(S, "S", (torch.float32,))
    N, d, _ = S.shape
    if out is None:
        out = torch.empty(N, packed_size(d), dtype=torch.float32, device=S.device)
    _need(out, "out", (torch.float32,))
    _check(load().hla_key_moment_pack(N, d, S.data_ptr(), out.data_ptr(), _stream(S.device)))
    return out


def key_moment_unpack(P: torch.Tensor, d: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed key moments [N, d(d+1)/2] -> full symmetric [N,d,d] (``hla_key_moment_unpack``)."""
    _need(P, "P", (torch.float32,))
    N = P.shape[0]
    if out is None:
        out = torch.empty(N, d, d, dtype=torch.float32, device=P.device)
    _need(out, "out", (torch.float32,))
    _check(load().hla_key_moment_unpack(N, d, P.data_ptr(), out.data_ptr(), _stream(P.device)))
    return out


def decode_step_mq(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, state: MqState, *, gamma=None,
                   ridge: float = 0.0, normalize: bool = False, return_den: bool = False,
                   out: Optional[torch.Tensor] = None, den: Optional[torch.Tensor] = None):
    """One token per query head through ``hla_decode_step_mq``: q [B,H,d];
    k [B,G,d] and v [B,G,dv] for G groups of query heads (G divides H);
    ``state`` (an MqState) is updated in place.  Returns (out [B,H,dv], den [B,H] or None)."""
    lib = load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (torch.bfloat16, torch.float32))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or k.shape[0] != q.shape[0] or v.shape[:2] != k.shape[:2] \
            or k.shape[2] != q.shape[2]:
        raise ValueError("expected q [B,H,d], k [B,G,d] and v [B,G,dv]")
    B, H, d = q.shape
    G, dv = k.shape[1], v.shape[-1]
    p, _keep = _params(B, H, 1, d, dv, 0, q.dtype, gamma, ridge, normalize)
    if out is None:
        out = torch.empty(B, H, dv, dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,))
    if den is None and return_den:
        den = torch.empty(B, H, dtype=torch.float32, device=q.device)
    sc = state.c()
    st = lib.hla_decode_step_mq(ctypes.byref(p), G, q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(sc),
                                out.data_ptr(), den.data_ptr() if den is not None else None, _stream(q.device))
    _check(st)
    return out, den


@dataclass
class AhlaState:
    """AHLA streaming summaries for B*H heads (fp32, device): P [N,d,dv],
    m [N,d], E [N,d,dv], n [N,d], rho [N] or None."""
    P: torch.Tensor
    m: torch.Tensor
    E: torch.Tensor
    n: torch.Tensor
    rho: Optional[torch.Tensor] = None

    @staticmethod
    def empty(N, d, dv, device):
        f = dict(dtype=torch.float32, device=device)
        return AhlaState(torch.empty(N, d, dv, **f), torch.empty(N, d, **f), torch.empty(N, d, dv, **f),
                         torch.empty(N, d, **f), torch.empty(N, **f))

    def tensors(self):
        return (self.P, self.m, self.E, self.n, self.rho)


@dataclass
class ThirdState:
    """Third-order streaming state for B*H heads (fp32, device): S [N,d,d],
    P [N,d,dv], m [N,d], F [N,d,dv], Fd [N,d]."""
    S: torch.Tensor
    P: torch.Tensor
    m: torch.Tensor
    F: torch.Tensor
    Fd: torch.Tensor

    @staticmethod
    def empty(N, d, dv, device):
        f = dict(dtype=torch.float32, device=device)
        return ThirdState(torch.empty(N, d, d, **f), torch.empty(N, d, dv, **f), torch.empty(N, d, **f),
                          torch.empty(N, d, dv, **f), torch.empty(N, d, **f))

    def tensors(self):
        return (self.S, self.P, self.m, self.F, self.Fd)


def _hi_c(st):
    if st is None:
        return None
    for t in st.tensors():
        if t is not None:
            _need(t, "state", (torch.float32,))
    return CHiState(*[t.data_ptr() if t is not None else None for t in st.tensors()])


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (torch.bfloat16, torch.float32))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")


def _higher_forward(third, q, k, v, gamma, normalize, chunk, init, return_state, return_den, out, den,
                    workspace, final_state):
    lib = load()
    _check_qkv(q, k, v)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q,k [B,H,n,d] and v [B,H,n,dv]")
    B, H, n, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    p, _keep = _params(B, H, n, d, dv, chunk, q.dtype, gamma, 0.0, normalize)
    size_fn = lib.hla_third_workspace_size if third else lib.hla_ahla_workspace_size
    need = int(size_fn(ctypes.byref(p)))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)  # zero-filled before first use
    if out is None:
        out = torch.empty(B, H, n, dv, dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,))
    if den is None and return_den:
        den = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    if den is not None:
        _need(den, "den", (torch.float32,))
    cls = ThirdState if third else AhlaState
    fin = final_state if final_state is not None else (cls.empty(B * H, d, dv, dev) if return_state else None)
    ic, fc = _hi_c(init), _hi_c(fin)
    fn = lib.hla_third_forward if third else lib.hla_ahla_forward
    st = fn(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            den.data_ptr() if den is not None else None, ctypes.byref(ic) if ic is not None else None,
            ctypes.byref(fc) if fc is not None else None, workspace.data_ptr() if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, _stream(dev))
    _check(st)
    return out, den, fin


def ahla_forward(q, k, v, *, gamma=None, normalize=False, chunk=0, init: Optional[AhlaState] = None,
                 return_state=False, return_den=False, out=None, den=None, workspace=None,
                 final_state: Optional[AhlaState] = None):
    """The asymmetric variant (AHLA) through ``hla_ahla_forward``: q, k [B,H,n,d],
    v [B,H,n,dv].  Returns (out, den or None, final AhlaState or None)."""
    return _higher_forward(False, q, k, v, gamma, normalize, chunk, init, return_state, return_den, out, den,
                           workspace, final_state)


def third_forward(q, k, v, *, normalize=False, chunk=0, init: Optional[ThirdState] = None, return_state=False,
                  return_den=False, out=None, den=None, workspace=None, final_state: Optional[ThirdState] = None):
    """Masked third-order HLA through ``hla_third_forward`` (no decay).
    Returns (out, den or None, final ThirdState or None)."""
    return _higher_forward(True, q, k, v, None, normalize, chunk, init, return_state, return_den, out, den,
                           workspace, final_state)


def _higher_decode(third, q, k, v, state, gamma, normalize, return_den, out, den):
    lib = load()
    _check_qkv(q, k, v)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q,k [B,H,d] and v [B,H,dv]")
    B, H, d = q.shape
    dv = v.shape[-1]
    p, _keep = _params(B, H, 1, d, dv, 0, q.dtype, gamma, 0.0, normalize)
    if out is None:
        out = torch.empty(B, H, dv, dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,))
    if den is None and return_den:
        den = torch.empty(B, H, dtype=torch.float32, device=q.device)
    sc = _hi_c(state)
    fn = lib.hla_third_decode_step if third else lib.hla_ahla_decode_step
    _check(fn(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(sc), out.data_ptr(),
              den.data_ptr() if den is not None else None, _stream(q.device)))
    return out, den


def ahla_decode_step(q, k, v, state: AhlaState, *, gamma=None, normalize=False, return_den=False, out=None,
                     den=None):
    """One AHLA token per state (``hla_ahla_decode_step``); ``state`` updated in place."""
    return _higher_decode(False, q, k, v, state, gamma, normalize, return_den, out, den)


def third_decode_step(q, k, v, state: ThirdState, *, normalize=False, return_den=False, out=None, den=None):
    """One third-order token per state (``hla_third_decode_step``); ``state`` updated in place."""
    return _higher_decode(True, q, k, v, state, None, normalize, return_den, out, den)


def state_compose(earlier: State, later: State, result: Optional[State] = None) -> State:
    """Masked semidirect product (earlier, then later) through ``hla_state_compose``."""
    lib = load()
    N, d, dv = earlier.C.shape
    if result is None:
        result = State.empty(N, d, dv, earlier.C.device)
    a, b, r = earlier.c(), later.c(), result.c()
    st = lib.hla_state_compose(N, d, dv, ctypes.byref(a), ctypes.byref(b), ctypes.byref(r),
                               _stream(earlier.C.device))
    _check(st)
    return result


class _HLAFunction(torch.autograd.Function):
    """Forward through ``hla_forward_chunked``, backward through
    ``hla_backward_chunked`` (both C ABI calls; nothing is computed here)."""

    @staticmethod
    def forward(ctx, q, k, v, gamma, ridge, normalize, chunk):
        out, _, _ = forward_chunked(q, k, v, gamma=gamma, ridge=ridge, normalize=normalize, chunk=chunk)
        ctx.save_for_backward(q, k, v)
        ctx.opts = (gamma, ridge, normalize, chunk)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v = ctx.saved_tensors
        gamma, ridge, normalize, chunk = ctx.opts
        dq, dk, dv = backward_chunked(q, k, v, dout.float().contiguous(), gamma=gamma, ridge=ridge,
                                      normalize=normalize, chunk=chunk)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None


class _HLAStateFunction(torch.autograd.Function):
    """The forward from an initial state, returning out and the final state's
    five parts; the backward takes the final state's gradient as dfinal and
    returns the initial state's as dinit (both C ABI calls)."""

    @staticmethod
    def forward(ctx, q, k, v, S, C, m, G, h, gamma, ridge, normalize, chunk):
        out, _, fin = forward_chunked(q, k, v, gamma=gamma, ridge=ridge, normalize=normalize, chunk=chunk,
                                      init=State(S, C, m, G, h), return_state=True)
        ctx.save_for_backward(q, k, v, S, C, m, G, h)
        ctx.opts = (gamma, ridge, normalize, chunk)
        ctx.set_materialize_grads(False)  # unused outputs arrive as None, not zeros
        return out, fin.S, fin.C, fin.m, fin.G, fin.h

    @staticmethod
    def backward(ctx, dout, dS, dC, dm, dG, dh):
        q, k, v, S, C, m, G, h = ctx.saved_tensors
        gamma, ridge, normalize, chunk = ctx.opts
        parts = (dS, dC, dm, dG, dh)
        dfinal = None
        if any(x is not None for x in parts):  # the final state is used downstream
            like = (S, C, m, G, h)
            dfinal = State(*(torch.zeros_like(t, dtype=torch.float32) if x is None else x.float().contiguous()
                             for x, t in zip(parts, like)))
        if dout is None:
            dout = torch.zeros(v.shape, dtype=torch.float32, device=v.device)
        dini = None
        if any(ctx.needs_input_grad[3:8]):  # some part of the initial state wants its gradient
            dini = State.empty(S.shape[0], q.shape[-1], v.shape[-1], q.device, with_rho=False)
        dq, dk, dv = backward_chunked(q, k, v, dout.float().contiguous(), gamma=gamma, ridge=ridge,
                                      normalize=normalize, chunk=chunk, init=State(S, C, m, G, h),
                                      dinit=dini, dfinal=dfinal)
        dst = (None,) * 5 if dini is None else (dini.S, dini.C, dini.m, dini.G, dini.h)
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), *dst, None, None, None, None)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, gamma=None, ridge: float = 0.0,
              normalize: bool = False, chunk: int = 0, init: Optional[State] = None):
    """Masked second-order HLA as a differentiable op: out [B,H,n,dv] fp32 from
    q, k [B,H,n,d] and v [B,H,n,dv] (bf16 or fp32); gradients flow to q, k, v
    through ``hla_backward_chunked`` and are returned in the inputs' dtype.

    Without ``init`` the sequence starts from the zero state and only out is
    returned.  With ``init`` (a State of fp32 tensors, which may require
    grad) it returns (out, final State): gradients reach the initial state's
    parts and flow back from the final state's, so sequence segments chain
    (``attention(..., init=final_of_previous)``) and train as one sequence.
    That path needs every decay >= 1e-6.

    The key moment S of a state is symmetric (a sum of k k^T), and the
    library reads it as such.  The op therefore uses the symmetric part
    (S + S^T)/2 of the given S, so a learnable initial S that an optimizer
    step has moved off the symmetric matrices still gives the function the
    gradient describes, and the gradient it receives is itself symmetric."""
    if init is None:
        return _HLAFunction.apply(q, k, v, gamma, ridge, normalize, chunk)
    S = 0.5 * (init.S + init.S.transpose(-1, -2))
    out, *fin = _HLAStateFunction.apply(q, k, v, S.contiguous(), init.C, init.m, init.G, init.h, gamma,
                                        ridge, normalize, chunk)
    return out, State(*fin)


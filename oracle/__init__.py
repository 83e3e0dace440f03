"""Plain fp64 CPU oracle for masked second-order Higher-order Linear Attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this package; the HIP library never does, and this
package never imports the HIP library.  The arithmetic lives in
``hla_oracle.c`` (plain C, double precision, one serial recurrence per head);
this module only compiles it, loads it with ctypes and marshals numpy arrays.

Functions (each follows the pages' identities; see ``hla_oracle.c``):

* :func:`forward` -- serial per-token recurrence (prefix moments S, C, m and
  the cross summaries G, h; output ``q_t^T (S_t C_t - G_t)`` plus ridge and
  optional ratio), Higher-order Linear Attention, paperlayer.ai page
  sec. 3.1 / 5.1 and gist.science page "Methodik" item 1.
* :func:`decode` -- the same update for one new token per state.
* :func:`decode_mq` -- the decode step when groups of query heads share keys
  and values (and so the key moment): the per-head step with the group's k, v.
* :mod:`oracle.higher` -- the asymmetric variant (AHLA) and third-order HLA
  (``higher_oracle.c``): serial recurrences, one decode step, composition.
* :func:`compose` -- the masked semidirect product of two segment summaries,
  paperlayer.ai page sec. 4.2 and gist.science page "Assoziative Operatoren".
* :func:`oracle.backward.backward` (module ``backward.py``) -- gradients of
  sum(out * dout) with respect to q, k, v: fp64 torch autograd through the
  same serial recurrence written with plain tensor ops.

Parity of every function is pinned by the ``-m "not gpu"`` tests against a
brute-force evaluation of the masked definition, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hla_oracle.c")
_SRC_HIGHER = os.path.join(_HERE, "higher_oracle.c")
_LIB = os.path.join(_HERE, "libhla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < _src_mtime():
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_HIGHER], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _src_mtime() -> float:
    return max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_HIGHER))


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < _src_mtime():
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i, d = ctypes.c_int, ctypes.c_double
        _lib.hla_oracle_forward.argtypes = [i, i, i, i, i, dp, dp, dp, dp, d, i,
                                            dp, dp, dp, dp, dp, dp, dp, dp,
                                            dp, dp, dp, dp, dp, dp, i]
        _lib.hla_oracle_forward.restype = i
        _lib.hla_oracle_decode.argtypes = [i, i, i, i, dp, dp, dp, dp, d, i,
                                           dp, dp, dp, dp, dp, dp, dp, dp, i]
        _lib.hla_oracle_decode.restype = i
        _lib.hla_oracle_compose.argtypes = [i, i, i] + [dp] * 18
        _lib.hla_oracle_compose.restype = i
        _lib.hla_oracle_ahla_forward.argtypes = [i, i, i, i, i, dp, dp, dp, dp, i] + [dp] * 5 + [dp, dp] + [dp] * 6 + [i]
        _lib.hla_oracle_ahla_forward.restype = i
        _lib.hla_oracle_ahla_compose.argtypes = [i, i, i] + [dp] * 18
        _lib.hla_oracle_ahla_compose.restype = i
        _lib.hla_oracle_ho3_forward.argtypes = [i, i, i, i, i, dp, dp, dp, i] + [dp] * 5 + [dp, dp] + [dp] * 9 + [i]
        _lib.hla_oracle_ho3_forward.restype = i
        _lib.hla_oracle_ho3_compose.argtypes = [i, i, i] + [dp] * 27
        _lib.hla_oracle_ho3_compose.restype = i
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, capped
    at 16 (the CPU share of one GPU on the GPU hosts)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f64(a) -> np.ndarray:
    """Exact conversion to a contiguous float64 array (bf16/fp32 -> fp64 is exact)."""
    try:
        import torch  # noqa: F401  (only to recognise tensors)
        if hasattr(a, "detach"):
            a = a.detach().to("cpu").double().numpy()
    except ImportError:
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


@dataclass
class State:
    """Segment summary (S, C, m, G, h, rho) for a batch of heads, float64.

    Shapes: S [N,d,d], C [N,d,dv], m [N,d], G [N,d,dv], h [N,d], rho [N].
    """
    S: np.ndarray
    C: np.ndarray
    m: np.ndarray
    G: np.ndarray
    h: np.ndarray
    rho: np.ndarray

    @staticmethod
    def zeros(N: int, d: int, dv: int) -> "State":
        return State(np.zeros((N, d, d)), np.zeros((N, d, dv)), np.zeros((N, d)),
                     np.zeros((N, d, dv)), np.zeros((N, d)), np.ones(N))

    def copy(self) -> "State":
        return State(*(np.array(x, dtype=np.float64, copy=True) for x in
                       (self.S, self.C, self.m, self.G, self.h, self.rho)))

    def flat(self):
        return (self.S, self.C, self.m, self.G, self.h, self.rho)


def _as_state(st, N, d, dv) -> State:
    out = State(*(_f64(x) for x in (st.S, st.C, st.m, st.G, st.h,
                                     st.rho if st.rho is not None else np.ones(N))))
    out.S = out.S.reshape(N, d, d); out.C = out.C.reshape(N, d, dv)
    out.m = out.m.reshape(N, d); out.G = out.G.reshape(N, d, dv)
    out.h = out.h.reshape(N, d); out.rho = out.rho.reshape(N)
    return out


def forward(q, k, v, gamma=None, lam: float = 0.0, normalize: bool = False,
            init: Optional[State] = None, want_state: bool = True,
            threads: Optional[int] = None):
    """Serial-recurrence forward.

    q, k: [B,H,n,d]; v: [B,H,n,dv] (any real dtype; converted exactly to fp64).
    gamma: None or a length-H sequence of decays in (0, 1].
    Returns (out [B,H,n,dv], den [B,H,n], final State or None).
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, d = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, n, d) and v.shape == (B, H, n, dv)
    g = None if gamma is None else _f64(np.asarray(gamma, dtype=np.float64).reshape(H))
    out = np.empty((B, H, n, dv))
    den = np.empty((B, H, n))
    N = B * H
    ini = _as_state(init, N, d, dv) if init is not None else None
    fin = State.zeros(N, d, dv) if want_state else None
    threads = threads or default_threads()
    ip = [None] * 6 if ini is None else [_ptr(x) for x in ini.flat()]
    fp = [None] * 6 if fin is None else [_ptr(x) for x in fin.flat()]
    rc = lib.hla_oracle_forward(B, H, n, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                float(lam), int(bool(normalize)), *ip,
                                _ptr(out), _ptr(den), *fp, int(threads))
    if rc != 0:
        raise ValueError("hla_oracle_forward: bad sizes")
    return out, den, fin


def decode(state: State, q, k, v, gamma=None, lam: float = 0.0,
           normalize: bool = False, threads: Optional[int] = None):
    """One token per state.  q, k: [B,H,d]; v: [B,H,dv].  Returns
    (out [B,H,dv], den [B,H], new State); the input state is not modified."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, d = q.shape
    dv = v.shape[-1]
    N = B * H
    st = _as_state(state, N, d, dv).copy()
    g = None if gamma is None else _f64(np.asarray(gamma, dtype=np.float64).reshape(H))
    out = np.empty((B, H, dv))
    den = np.empty((B, H))
    threads = threads or default_threads()
    rc = lib.hla_oracle_decode(B, H, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                               float(lam), int(bool(normalize)),
                               *[_ptr(x) for x in st.flat()], _ptr(out), _ptr(den),
                               int(threads))
    if rc != 0:
        raise ValueError("hla_oracle_decode: bad sizes")
    return out, den, st


def decode_mq(state: State, q, k, v, gamma=None, lam: float = 0.0, normalize: bool = False,
              threads: Optional[int] = None):
    """One token per query head when groups of query heads share keys and
    values (paperlayer.ai summary sec. 5.2, multi-query sharing).  The key
    moment S depends on the keys alone, so heads that share keys share it,
    and each head's step is the ordinary one (:func:`decode`) with its
    group's k and v.  q: [B,H,d]; k: [B,G,d]; v: [B,G,dv] with G dividing H
    (group j = query heads j*R .. j*R+R-1, R = H/G); ``state`` holds one
    full state per query head (S equal within a group).  Returns (out
    [B,H,dv], den [B,H], new per-head State); S stays equal within a group."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, d = q.shape
    G = k.shape[1]
    assert H % G == 0 and k.shape == (B, G, d) and v.shape[:2] == (B, G)
    R = H // G
    kk = np.ascontiguousarray(np.repeat(k, R, axis=1))
    vv = np.ascontiguousarray(np.repeat(v, R, axis=1))
    out, den, st = decode(state, q, kk, vv, gamma=gamma, lam=lam, normalize=normalize, threads=threads)
    S = st.S.reshape(B, G, R, d, d)
    assert np.array_equal(S, np.broadcast_to(S[:, :, :1], S.shape)), "S differs within a group"
    return out, den, st


def compose(a: State, b: State) -> State:
    """Masked semidirect product a then b, batched over the leading axis."""
    lib = _load()
    N, d, dv = np.asarray(a.C).shape
    a = _as_state(a, N, d, dv)
    b = _as_state(b, N, d, dv)
    r = State.zeros(N, d, dv)
    rc = lib.hla_oracle_compose(N, d, dv, *[_ptr(x) for x in a.flat()],
                                *[_ptr(x) for x in b.flat()], *[_ptr(x) for x in r.flat()])
    if rc != 0:
        raise ValueError("hla_oracle_compose: bad sizes")
    return r

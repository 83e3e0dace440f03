"""fp64 CPU oracle of the asymmetric variant (AHLA) and of third-order HLA.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The arithmetic lives
in ``higher_oracle.c`` (plain C, double precision, one serial recurrence per
head, the formulas in its header); this module marshals numpy arrays.

* :func:`ahla_forward` -- AHLA, the masked left-cascaded product
  Q (K^T Q)(K^T V) with decay (paperlayer.ai page sec. 6, 6.1, 6.3;
  gist.science page "Methodik" item 2), streaming summaries (P, m, E, n).
* :func:`ahla_decode` -- one token per state (the same recurrence, n = 1).
* :func:`ahla_compose` -- composition of AHLA segment summaries (sec. 6.2),
  which carries the segment sum R = sum k q^T.
* :func:`third_forward` -- masked third order A A^T A V, no decay
  (paperlayer.ai page sec. 7, 7.1, 7.2; gist.science page "Methodik" item 3),
  streaming state (S, P, m, F, Fd) and, from the zero state, the segment
  aggregates (SQ, M, N, Nd) that composition needs.
* :func:`third_decode`, :func:`third_compose` -- likewise (sec. 7.3).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import _f64, _load, _ptr, default_threads


@dataclass
class AhlaState:
    """P [N,d,dv], m [N,d], E [N,d,dv], n [N,d], R [N,d,d] (segment sum
    k q^T; composition only, may be None), rho [N]."""
    P: np.ndarray
    m: np.ndarray
    E: np.ndarray
    n: np.ndarray
    R: Optional[np.ndarray]
    rho: np.ndarray

    @staticmethod
    def zeros(N, d, dv):
        return AhlaState(np.zeros((N, d, dv)), np.zeros((N, d)), np.zeros((N, d, dv)), np.zeros((N, d)),
                         np.zeros((N, d, d)), np.ones(N))


def _gam(gamma, H):
    return None if gamma is None else _f64(np.asarray(gamma, dtype=np.float64).reshape(H))


def ahla_forward(q, k, v, gamma=None, normalize: bool = False, init: Optional[AhlaState] = None,
                 want_state: bool = True, threads: Optional[int] = None):
    """Serial AHLA recurrence.  q, k [B,H,n,d], v [B,H,n,dv].  Returns
    (out [B,H,n,dv], den [B,H,n], final AhlaState or None); the final R is the
    sum of k q^T over this call's tokens."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, d = q.shape
    dv = v.shape[-1]
    N = B * H
    out, den = np.empty((B, H, n, dv)), np.empty((B, H, n))
    ini = None
    if init is not None:
        ini = [_f64(x).reshape(s) for x, s in ((init.P, (N, d, dv)), (init.m, (N, d)), (init.E, (N, d, dv)),
                                              (init.n, (N, d)))]
        ini.append(_f64(init.rho).reshape(N) if init.rho is not None else np.ones(N))
    fin = AhlaState.zeros(N, d, dv) if want_state else None
    ip = [None] * 5 if ini is None else [_ptr(x) for x in ini]
    fp = [None] * 6 if fin is None else [_ptr(x) for x in (fin.P, fin.m, fin.E, fin.n, fin.R, fin.rho)]
    rc = lib.hla_oracle_ahla_forward(B, H, n, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(_gam(gamma, H)),
                                     int(bool(normalize)), *ip, _ptr(out), _ptr(den), *fp,
                                     int(threads or default_threads()))
    if rc != 0:
        raise ValueError("hla_oracle_ahla_forward: bad sizes")
    return out, den, fin


def ahla_decode(state: AhlaState, q, k, v, gamma=None, normalize: bool = False):
    """One token per state: q, k [B,H,d], v [B,H,dv].  Returns (out [B,H,dv],
    den [B,H], new AhlaState)."""
    q, k, v = (_f64(x)[:, :, None] for x in (q, k, v))
    out, den, st = ahla_forward(q, k, v, gamma=gamma, normalize=normalize, init=state)
    return out[:, :, 0], den[:, :, 0], st


def ahla_compose(a: AhlaState, b: AhlaState) -> AhlaState:
    """Earlier segment a, then b (each with its R), batched over the leading axis."""
    lib = _load()
    N, d, dv = np.asarray(a.P).shape
    A = [_f64(x) for x in (a.P, a.m, a.E, a.n, a.R, a.rho)]
    Bb = [_f64(x) for x in (b.P, b.m, b.E, b.n, b.R, b.rho)]
    r = AhlaState.zeros(N, d, dv)
    rc = lib.hla_oracle_ahla_compose(N, d, dv, *[_ptr(x) for x in A], *[_ptr(x) for x in Bb],
                                     *[_ptr(x) for x in (r.P, r.m, r.E, r.n, r.R, r.rho)])
    if rc != 0:
        raise ValueError("hla_oracle_ahla_compose: bad sizes")
    return r


@dataclass
class ThirdState:
    """Streaming S [N,d,d], P [N,d,dv], m [N,d], F [N,d,dv], Fd [N,d]; segment
    aggregates SQ [N,d,d], M [N,d,d], Nq [N,d,dv], Nd [N,d] (or None)."""
    S: np.ndarray
    P: np.ndarray
    m: np.ndarray
    F: np.ndarray
    Fd: np.ndarray
    SQ: Optional[np.ndarray] = None
    M: Optional[np.ndarray] = None
    Nq: Optional[np.ndarray] = None
    Nd: Optional[np.ndarray] = None

    @staticmethod
    def zeros(N, d, dv, aggregates=True):
        z = lambda *s: np.zeros(s)
        return ThirdState(z(N, d, d), z(N, d, dv), z(N, d), z(N, d, dv), z(N, d),
                          *((z(N, d, d), z(N, d, d), z(N, d, dv), z(N, d)) if aggregates else (None,) * 4))

    def streaming(self):
        return (self.S, self.P, self.m, self.F, self.Fd)

    def parts(self):
        return (self.S, self.P, self.m, self.F, self.Fd, self.SQ, self.M, self.Nq, self.Nd)


def third_forward(q, k, v, normalize: bool = False, init: Optional[ThirdState] = None,
                  want_state: bool = True, threads: Optional[int] = None):
    """Serial third-order recurrence (no decay).  Returns (out, den, final
    ThirdState or None); from the zero state the final state carries the
    segment aggregates too."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, d = q.shape
    dv = v.shape[-1]
    N = B * H
    out, den = np.empty((B, H, n, dv)), np.empty((B, H, n))
    ip = [None] * 5
    if init is not None:
        ini = [_f64(x).reshape(s) for x, s in zip(init.streaming(), ((N, d, d), (N, d, dv), (N, d), (N, d, dv), (N, d)))]
        ip = [_ptr(x) for x in ini]
    fin = ThirdState.zeros(N, d, dv, aggregates=init is None) if want_state else None
    fp = [None] * 9 if fin is None else [_ptr(x) for x in fin.parts()]
    rc = lib.hla_oracle_ho3_forward(B, H, n, d, dv, _ptr(q), _ptr(k), _ptr(v), int(bool(normalize)), *ip,
                                    _ptr(out), _ptr(den), *fp, int(threads or default_threads()))
    if rc != 0:
        raise ValueError("hla_oracle_ho3_forward: bad sizes")
    return out, den, fin


def third_decode(state: ThirdState, q, k, v, normalize: bool = False):
    """One token per state: q, k [B,H,d], v [B,H,dv]."""
    q, k, v = (_f64(x)[:, :, None] for x in (q, k, v))
    out, den, st = third_forward(q, k, v, normalize=normalize, init=state)
    return out[:, :, 0], den[:, :, 0], st


def third_compose(a: ThirdState, b: ThirdState) -> ThirdState:
    """Earlier segment a, then b (both with their aggregates)."""
    lib = _load()
    N, d, dv = np.asarray(a.P).shape
    A = [_f64(x) for x in a.parts()]
    Bb = [_f64(x) for x in b.parts()]
    r = ThirdState.zeros(N, d, dv)
    rc = lib.hla_oracle_ho3_compose(N, d, dv, *[_ptr(x) for x in A], *[_ptr(x) for x in Bb],
                                    *[_ptr(x) for x in r.parts()])
    if rc != 0:
        raise ValueError("hla_oracle_ho3_compose: bad sizes")
    return r

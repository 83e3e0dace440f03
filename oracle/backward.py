"""Reverse-mode gradients of the masked second-order HLA forward, fp64 CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests, the
smoke check and the bench's CPU baseline may use it; the HIP library never
does.

What it computes.  The forward is the serial per-token recurrence of the
pages (Higher-order Linear Attention; paperlayer.ai page sec. 3.1 for the
masked prefix summaries and the cross summaries, sec. 4.3 for the decay as an
attenuation factor, sec. 5.1 for the ridge and the optional ratio;
gist.science page "Methodik" item 1 for the read-out q^T(S C - G)):

    S_t = g S_{t-1} + k_t k_t^T          C_t = g C_{t-1} + q_t v_t^T
    m_t = g m_{t-1} + q_t
    G_t = g^2 G_{t-1} + g k_t (k_t^T C_{t-1})
    h_t = g^2 h_{t-1} + g k_t (k_t . m_{t-1})
    num_t = q_t^T ((S_t + lam I) C_t - G_t)
    den_t = q_t^T ((S_t + lam I) m_t - h_t)
    out_t = num_t, or num_t / den_t with normalize

starting from the zero state or from a given state (S, C, m, G, h) at
position -1 (held constant, or, on request, differentiated as well).  The pages' training claim is that this scan
is differentiated like any other layer; here the gradient of the scalar
sum_t <out_t, dout_t> with respect to q, k and v is taken by torch's
autograd through exactly these updates, written with plain tensor ops in
float64 (autograd is the library primitive; there is no hand-derived
gradient in this file).  Everything is batched over the (batch, head)
units only; the token loop stays serial.

Pinned by the CPU tests against central finite differences of the C oracle's
forward (``hla_oracle.c``, independent code), against the exact linearity of
out in v, and by its own forward against the C oracle's.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch


def _t64(a) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.float64).contiguous()
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def _part(a) -> torch.Tensor:
    """A state part: kept as is when it is a float64 tensor that requires a
    gradient (so autograd reaches it), else converted like any input."""
    if isinstance(a, torch.Tensor) and a.requires_grad:
        return a
    return _t64(a)


def forward_recurrence(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       gamma: Optional[Sequence[float]] = None, lam: float = 0.0,
                       normalize: bool = False, init=None, return_state: bool = False):
    """The serial recurrence in float64 torch ops (differentiable).

    q, k: [B,H,n,d]; v: [B,H,n,dv]; init: None or an object with S [N,d,d],
    C [N,d,dv], m [N,d], G [N,d,dv], h [N,d] (N = B*H), the state before
    token 0.  Returns (out [B,H,n,dv], den [B,H,n]), and with ``return_state``
    also the final state as a tuple (S, C, m, G, h) shaped as ``init``'s parts."""
    B, H, n, d = q.shape
    dv = v.shape[-1]
    N = B * H
    qf, kf, vf = q.reshape(N, n, d), k.reshape(N, n, d), v.reshape(N, n, dv)
    g = torch.ones(N, dtype=torch.float64) if gamma is None else \
        torch.as_tensor(np.asarray(gamma, dtype=np.float64)).repeat(B)
    g1, g2 = g.view(N, 1, 1), (g * g).view(N, 1, 1)
    gv1, gv2 = g.view(N, 1), (g * g).view(N, 1)
    if init is None:
        S = torch.zeros(N, d, d, dtype=torch.float64)
        C = torch.zeros(N, d, dv, dtype=torch.float64)
        G = torch.zeros(N, d, dv, dtype=torch.float64)
        m = torch.zeros(N, d, dtype=torch.float64)
        h = torch.zeros(N, d, dtype=torch.float64)
    else:
        S, C, G = (_part(x).reshape(N, d, w) for x, w in ((init.S, d), (init.C, dv), (init.G, dv)))
        m, h = (_part(x).reshape(N, d) for x in (init.m, init.h))
    outs, dens = [], []
    for t in range(n):
        qt, kt, vt = qf[:, t], kf[:, t], vf[:, t]
        # cross summaries use the moments before token t
        r = torch.einsum("na,naj->nj", kt, C)          # k_t^T C_{t-1}
        s = (kt * m).sum(-1, keepdim=True)              # k_t . m_{t-1}
        G = g2 * G + g1 * kt.unsqueeze(-1) * r.unsqueeze(1)
        h = gv2 * h + gv1 * s * kt
        S = g1 * S + kt.unsqueeze(-1) * kt.unsqueeze(1)
        C = g1 * C + qt.unsqueeze(-1) * vt.unsqueeze(1)
        m = gv1 * m + qt
        a = torch.einsum("nab,nb->na", S, qt) + lam * qt   # (S_t + lam I) q_t
        num = torch.einsum("na,naj->nj", a, C) - torch.einsum("na,naj->nj", qt, G)
        den = (a * m).sum(-1) - (qt * h).sum(-1)
        outs.append(num / den.unsqueeze(-1) if normalize else num)
        dens.append(den)
    if n == 0:
        out = torch.zeros(B, H, 0, dv, dtype=torch.float64)
        den = torch.zeros(B, H, 0, dtype=torch.float64)
    else:
        out = torch.stack(outs, 1).reshape(B, H, n, dv)
        den = torch.stack(dens, 1).reshape(B, H, n)
    if return_state:
        return out, den, (S, C, m, G, h)
    return out, den


class _Init:
    def __init__(self, S, C, m, G, h):
        self.S, self.C, self.m, self.G, self.h = S, C, m, G, h


def backward(q, k, v, dout, gamma: Optional[Sequence[float]] = None, lam: float = 0.0,
             normalize: bool = False, init=None, init_grad: bool = False, dfinal=None):
    """Gradients (dq, dk, dv) of sum(out * dout), from the zero state or from
    ``init`` (see :func:`forward_recurrence`).

    q, k: [B,H,n,d]; v, dout: [B,H,n,dv]; any real dtype (converted exactly to
    float64).  Returns float64 numpy arrays shaped like q, k, v.  With
    ``init_grad`` a fourth item is returned: a dict of the gradients with
    respect to the initial state's parts, S [N,d,d], C [N,d,dv], m [N,d],
    G [N,d,dv], h [N,d] (N = B*H; a zero initial state when ``init`` is None).
    Every entry of S counts as its own variable, with the read-out written as
    (S_t q_t)^T C_t.  ``dfinal``, an object with S, C, m, G, h shaped as a
    state, adds sum over the parts of <final part, dfinal part> to the loss:
    the gradient a later segment hands back for the final state."""
    q, k, v, dout = (_t64(x).clone().requires_grad_(i < 3) for i, x in enumerate((q, k, v, dout)))
    B, H, n, d = q.shape
    dv = v.shape[-1]
    N = B * H
    ini = init
    if init_grad:
        if init is None:
            parts = [torch.zeros(N, d, d), torch.zeros(N, d, dv), torch.zeros(N, d),
                     torch.zeros(N, d, dv), torch.zeros(N, d)]
            parts = [x.to(torch.float64) for x in parts]
        else:
            parts = [_t64(x).reshape(shape) for x, shape in
                     ((init.S, (N, d, d)), (init.C, (N, d, dv)), (init.m, (N, d)),
                      (init.G, (N, d, dv)), (init.h, (N, d)))]
        parts = [x.clone().requires_grad_(True) for x in parts]
        ini = _Init(*parts)
    if n == 0 and dfinal is None:
        grads = (np.zeros(tuple(q.shape)), np.zeros(tuple(k.shape)), np.zeros(tuple(v.shape)))
        if init_grad:
            return grads + ({key: np.zeros(tuple(x.shape)) for key, x in
                             zip(("S", "C", "m", "G", "h"), parts)},)
        return grads
    out, _, fin = forward_recurrence(q, k, v, gamma, lam, normalize, ini, return_state=True)
    loss = (out * dout).sum()
    if dfinal is not None:
        for x, name in zip(fin, ("S", "C", "m", "G", "h")):
            loss = loss + (x * _t64(getattr(dfinal, name)).reshape(x.shape)).sum()
    if loss.requires_grad:
        loss.backward()
    grads = tuple(x.grad.numpy() if x.grad is not None else np.zeros(tuple(x.shape)) for x in (q, k, v))
    if init_grad:
        return grads + ({key: x.grad.numpy() if x.grad is not None else np.zeros(tuple(x.shape))
                         for key, x in zip(("S", "C", "m", "G", "h"), parts)},)
    return grads

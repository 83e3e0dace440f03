"""Parity metrics between the HIP path and the fp64 oracle.

* row error: max over rows of ||x_r - ref_r||_inf / ||ref_r||_inf, a row being
  one (b, h, t) output vector -- the gate for unnormalised outputs;
* slab error: per (b, h), max_t |x - ref| / max_t |ref|, maximised over (b, h)
  -- the gate for the denominator and for state tensors;
* cross summaries G and h: they remove the future pairs from the naive
  products S C and S m, and can be exactly zero (one token) while those
  products are not, so their slab error is taken relative to
  max(max |ref|, max |S_ref C_ref|) (resp. S_ref m_ref) per slab;
* ratio outputs: the row error on rows whose reference denominator satisfies
  |den| >= 1e-2 * median |den| of their (b, h) slab (the ratio is ill
  conditioned near den = 0, which the method does not rule out).
Tolerances: 2e-3 for bf16 inputs, 1e-5 for fp32 inputs.
"""
import numpy as np
import torch

TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def _np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def row_err(x, ref) -> float:
    x, ref = _np(x), _np(ref)
    x = x.reshape(-1, x.shape[-1])
    ref = ref.reshape(x.shape)
    num = np.max(np.abs(x - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.max(num / np.maximum(den, 1e-300)))


def slab_err(x, ref, lead: int = 1, scale=None) -> float:
    """Error per slab, where a slab is the leading `lead` axes' index; `scale`
    (one value per slab) is a floor for the denominator."""
    x, ref = _np(x), _np(ref)
    if not np.all(np.isfinite(x)):
        return float("inf")
    shp = int(np.prod(x.shape[:lead]))
    x = x.reshape(shp, -1)
    ref = ref.reshape(shp, -1)
    num = np.max(np.abs(x - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    if scale is not None:
        den = np.maximum(den, np.asarray(scale, dtype=np.float64).reshape(shp))
    return float(np.max(num / np.maximum(den, 1e-300)))


def naive_scales(S, C, m):
    """Per-slab max |S C| and max |S m| for states S [N,d,d], C [N,d,dv], m [N,d]."""
    S, C, m = _np(S), _np(C), _np(m)
    sc = np.max(np.abs(S @ C).reshape(S.shape[0], -1), axis=1)
    sm = np.max(np.abs(np.einsum("nij,nj->ni", S, m)), axis=1)
    return sc, sm


def ratio_err(out, ref_out, ref_den):
    """(error, excluded rows) for ratio outputs [B,H,n,dv] with ref den [B,H,n]."""
    out, ref_out, ref_den = _np(out), _np(ref_out), _np(ref_den)
    B, H, n, dv = ref_out.shape
    med = np.median(np.abs(ref_den), axis=2, keepdims=True)
    keep = np.abs(ref_den) >= 1e-2 * med
    x = out[keep]
    r = ref_out[keep]
    if x.size == 0:
        return 0.0, int((~keep).sum())
    return row_err(x, r), int((~keep).sum())

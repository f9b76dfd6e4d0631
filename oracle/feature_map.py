"""CPU oracle for the Hedgehog feature map of the GLA branch and for the layer
that consumes it in log space.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

What it computes, with the passages it follows (gist.science explainer of
"Lizard: An Efficient Linearization Framework for Large Language Models"):

* The GLA branch keeps its state from feature-mapped keys, S_t = Gamma_t
  S_{t-1} + phi(k_t) v_t^T, and reads it with phi(q_t) (English page §2.A,
  state update).  The pages name the map a Hedgehog feature map and use its
  non-negativity to absorb the cumulative gate into the query and key
  projections in log space (Chinese page §2.3, hardware-aware algorithm;
  English page §2.C; French page: the gate terms enter the feature space
  through logarithms).  The pages do not print the map; the reading taken
  here is the published two-sided softmax form of the Hedgehog map,
      phi(x) = [softmax(x W), softmax(-x W)],   W [d, d/2] per head,
  whose logarithm is exact and finite:
      log phi(x) = [x W - lse(x W), -x W - lse(-x W)].
* The layer with the map: the GLA branch runs on phi(q), phi(k) (given as
  their logarithms lq, lk), the anchor window on the raw q, k (its softmax
  attention is the teacher's own form), both on the same v:
      o = gla(exp(lq), exp(lk), v, g) + mix * window(q, k, v).
  With the gate folded in log space the GLA operands are exp(lq + b) and
  exp(lk - b) for the chunk-local gate prefix b; in exact arithmetic that is
  the same product, which is what this oracle evaluates.
* Backward (the pages give none): with dq^gla = dL/d phi(q), the gradient of
  the log features is dlq = phi(q) * dq^gla (likewise dlk); the map's own
  backward is that of a log-softmax on each half, then dx = dz W^T and
  dW = sum over tokens of x^T dz.

Plain numpy in float64.
"""
from __future__ import annotations

import numpy as np

from . import lizard_oracle as orc

__all__ = ["hedgehog_log_features", "hedgehog_log_features_backward", "hybrid_forward_features",
           "hybrid_backward_features", "decode_step_features"]


def _lse(z):
    m = z.max(axis=-1, keepdims=True)
    return m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))


def hedgehog_log_features(x, w):
    """log phi(x) for x [B,H,L,d] and per-head weights w [H,d,d/2]; returns [B,H,L,d]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    z = np.einsum("bhtd,hdf->bhtf", x, w)
    return np.concatenate([z - _lse(z), -z - _lse(-z)], axis=-1)


def hedgehog_log_features_backward(x, w, dl):
    """Gradients (dx, dw) of sum(dl * log phi(x)).

    For y = z - lse(z): dz = g - softmax(z) * sum(g); the second half is the same map of -z,
    so its contribution enters with the opposite sign."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dl = np.asarray(dl, np.float64)
    f = w.shape[-1]
    z = np.einsum("bhtd,hdf->bhtf", x, w)
    gp, gm = dl[..., :f], dl[..., f:]
    pp = np.exp(z - _lse(z))
    pm = np.exp(-z - _lse(-z))
    dz = (gp - pp * gp.sum(-1, keepdims=True)) - (gm - pm * gm.sum(-1, keepdims=True))
    dx = np.einsum("bhtf,hdf->bhtd", dz, w)
    dw = np.einsum("bhtd,bhtf->hdf", x, dz)
    return dx, dw


def hybrid_forward_features(q, k, v, lq, lk, g, meta_k, meta_v=None, *, window, scale, mix=1.0):
    """o = gla(exp(lq), exp(lk), v, g) + mix * window(q, k, v); also o_swa, lse, state."""
    fq, fk = np.exp(np.asarray(lq, np.float64)), np.exp(np.asarray(lk, np.float64))
    o_gla, S = orc.gla_forward(fq, fk, v, g)
    o_swa, lse = orc.window_forward(q, k, v, meta_k, meta_v, window, scale)
    return dict(o=o_gla + mix * o_swa, o_gla=o_gla, o_swa=o_swa, lse=lse, state=S)


def hybrid_backward_features(q, k, v, lq, lk, g, meta_k, meta_v, dO, *, window, scale, mix=1.0):
    """Gradients of sum(dO * o) for hybrid_forward_features: dq, dk (window only), dv (both
    branches), dlq, dlk (GLA through the features), dg, dmeta_k, dmeta_v."""
    fq, fk = np.exp(np.asarray(lq, np.float64)), np.exp(np.asarray(lk, np.float64))
    gq, gk, gv, dg = orc.gla_backward(fq, fk, v, g, dO)
    wq, wk, wv, dmk, dmv = orc.window_backward(q, k, v, meta_k, meta_v, dO, window, scale, mix)
    return dict(dq=wq, dk=wk, dv=gv + wv, dlq=fq * gq, dlk=fk * gk, dg=dg, dmeta_k=dmk, dmeta_v=dmv)


def decode_step_features(st, q, k, v, lq, lk, g, meta_k, meta_v, *, scale, mix=1.0):
    """One decode step of the layer with GLA log features: S <- diag(exp g) S + exp(lk)^T v,
    o_gla = exp(lq) S; the anchor window on the raw q, k (ring of raw keys and values);
    o = o_gla + mix * o_swa; pos += 1.  q, k, v, lq, lk, g: [B,H,d]."""
    fq, fk = np.exp(np.asarray(lq, np.float64)), np.exp(np.asarray(lk, np.float64))
    v64 = np.asarray(v, np.float64)
    st.S = np.exp(np.asarray(g, np.float64))[..., None] * st.S + fk[..., :, None] * v64[..., None, :]
    o_gla = np.matmul(fq[:, :, None, :], st.S)[:, :, 0, :]
    o_swa = orc.decode_window(st, q, k, v, meta_k, meta_v, scale=scale)
    st.pos += 1
    return o_gla + mix * o_swa

"""CPU oracle for the gate projection of the Lizard layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

What it computes, with the passage it follows.  The explainer pages for
"Lizard: An Efficient Linearization Framework for Large Language Models"
(gist.science) give the learnable gating module as Gamma_i = sigmoid(W_gamma x_i)
(English page §2.A "Adaptive Memory Control"; French page §2.A; Chinese page
§2.1, innovation bullet on the learnable gating module), and handle the gate in
log space (English page §2.C).  The layer therefore consumes

    g = log(sigmoid(x W^T)) / tau

with x [B, L, d_model] the layer input, W [Ng, d_model] (row n = h*d_k + i for
one gate per key dimension, n = h for the Chinese page's scalar gate), and tau
a temperature (tau = 1 is the pages' gate; a larger tau slows the decay, and
the synthetic workloads of this project draw gates as logsigmoid(.)/16).
The pages give no bias term, so there is none.

The backward is the exact derivative (the pages give none):
    dz = dg * (1 - sigmoid(z)) / tau,   dx = dz W,   dW = sum over tokens of dz^T x.

Plain numpy in float64.  ``gate_projection`` returns g in the layer's gate
layout, [B, H, L, d_k] or [B, H, L].
"""
from __future__ import annotations

import numpy as np

__all__ = ["logsigmoid", "gate_projection", "gate_projection_backward"]


def logsigmoid(z):
    """log(1 / (1 + exp(-z))), evaluated without overflow for any real z."""
    return -np.logaddexp(0.0, -z)


def _to_gate_layout(y, heads, scalar):
    """[B, L, Ng] -> [B, H, L, d_k] (Ng = H*d_k) or [B, H, L] (Ng = H)."""
    B, L, Ng = y.shape
    if scalar:
        assert Ng == heads
        return np.ascontiguousarray(y.transpose(0, 2, 1))
    dk = Ng // heads
    assert dk * heads == Ng
    return np.ascontiguousarray(y.reshape(B, L, heads, dk).transpose(0, 2, 1, 3))


def _from_gate_layout(g, scalar):
    """Inverse of _to_gate_layout."""
    if scalar:
        return g.transpose(0, 2, 1)
    B, H, L, dk = g.shape
    return g.transpose(0, 2, 1, 3).reshape(B, L, H * dk)


def gate_projection(x, w, heads, *, tau=1.0, scalar=False):
    """g = log sigmoid(x W^T) / tau, in the layer's gate layout.

    x: [B, L, d_model]; w: [Ng, d_model] with Ng = heads * d_k (per key
    dimension) or heads (scalar gate).
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    z = x @ w.T
    return _to_gate_layout(logsigmoid(z) / tau, heads, scalar)


def gate_projection_backward(x, w, heads, dg, *, tau=1.0, scalar=False):
    """Gradients of sum(dg * g) for g = gate_projection(x, w, heads, tau, scalar).

    With z = x W^T: dg/dz = (1 - sigmoid(z)) / tau = sigmoid(-z) / tau, so
    dz = dg_tokens * sigmoid(-z) / tau (dg re-laid out token-major), and
    dx = dz W, dW = sum_{b,t} dz[b,t]^T x[b,t].  Returns (dx, dw).
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dgt = _from_gate_layout(np.asarray(dg, np.float64), scalar)
    z = x @ w.T
    dz = dgt * np.exp(logsigmoid(-z)) / tau
    dx = dz @ w
    dw = np.einsum("bln,blm->nm", dz, x)
    return dx, dw

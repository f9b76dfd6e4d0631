"""Pins of the Hedgehog feature-map oracle and of the layer that consumes log
features: log-softmax closed forms and normalisation, torch autograd, finite
differences, and the reduction to the plain layer when the features are the
raw q, k (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import feature_map as fm
from oracle import lizard_oracle as orc


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def test_closed_forms_and_normalisation():
    rng = np.random.default_rng(0)
    B, H, L, d = 2, 3, 5, 8
    x = rnd(rng, B, H, L, d)
    # W = 0: both halves are uniform over d/2 features
    lz = fm.hedgehog_log_features(x, np.zeros((H, d, d // 2)))
    assert np.allclose(lz, -math.log(d // 2), rtol=0, atol=1e-15)
    # each half is a probability vector, and the two halves mirror each other's order
    w = rnd(rng, H, d, d // 2)
    lf = fm.hedgehog_log_features(x, w)
    assert np.allclose(np.exp(lf[..., : d // 2]).sum(-1), 1.0, rtol=1e-14, atol=0)
    assert np.allclose(np.exp(lf[..., d // 2:]).sum(-1), 1.0, rtol=1e-14, atol=0)
    assert (lf <= 0).all()
    # a token whose projection is e_0 * c: phi+ puts weight e^c / (e^c + f - 1) on feature 0
    c, f = 2.0, d // 2
    x1 = np.zeros((1, 1, 1, d)); x1[..., 0] = 1.0
    w1 = np.zeros((1, d, f)); w1[0, 0, 0] = c
    l1 = fm.hedgehog_log_features(x1, w1)[0, 0, 0]
    assert abs(l1[0] - (c - math.log(math.exp(c) + f - 1))) < 1e-14
    assert abs(l1[f] - (-c - math.log(math.exp(-c) + f - 1))) < 1e-14


def test_feature_map_against_torch_autograd():
    rng = np.random.default_rng(1)
    B, H, L, d = 2, 2, 7, 8
    x, w, dl = rnd(rng, B, H, L, d), rnd(rng, H, d, d // 2), rnd(rng, B, H, L, d)
    lf = fm.hedgehog_log_features(x, w)
    dx, dw = fm.hedgehog_log_features_backward(x, w, dl)
    xt, wt = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
    z = torch.einsum("bhtd,hdf->bhtf", xt, wt)
    y = torch.cat([torch.log_softmax(z, -1), torch.log_softmax(-z, -1)], -1)
    (y * torch.tensor(dl)).sum().backward()
    assert np.allclose(lf, y.detach().numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_feature_map_finite_differences():
    rng = np.random.default_rng(2)
    B, H, L, d = 1, 2, 3, 4
    x, w, dl = rnd(rng, B, H, L, d), rnd(rng, H, d, d // 2), rnd(rng, B, H, L, d)
    dx, dw = fm.hedgehog_log_features_backward(x, w, dl)
    f = lambda xx, ww: float((fm.hedgehog_log_features(xx, ww) * dl).sum())
    h = 1e-6
    for arr, grad, is_x in ((x, dx, True), (w, dw, False)):
        for _ in range(5):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            fd = (f(ap, w) - f(am, w)) / (2 * h) if is_x else (f(x, ap) - f(x, am)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd))


def test_layer_with_raw_features_is_the_plain_layer():
    """lq = log q, lk = log k with positive q, k reproduces the plain layer exactly."""
    rng = np.random.default_rng(3)
    B, H, L, d, M, W = 1, 2, 20, 4, 2, 6
    q, k = np.abs(rnd(rng, B, H, L, d)) + 0.1, np.abs(rnd(rng, B, H, L, d)) + 0.1
    v, dO = rnd(rng, B, H, L, d), rnd(rng, B, H, L, d)
    g = -np.abs(rnd(rng, B, H, L, d, s=0.2))
    mk = rnd(rng, H, M, d)
    a = fm.hybrid_forward_features(q, k, v, np.log(q), np.log(k), g, mk, window=W, scale=0.5)
    b = orc.hybrid_forward(q, k, v, g, mk, window=W, scale=0.5)
    assert np.allclose(a["o"], b["o"], rtol=1e-12, atol=1e-13)
    ga = fm.hybrid_backward_features(q, k, v, np.log(q), np.log(k), g, mk, None, dO, window=W, scale=0.5)
    gb = orc.hybrid_backward(q, k, v, g, mk, None, dO, window=W, scale=0.5)
    # chain rule through q = exp(lq): the plain layer's dq splits into the window part and dlq / q
    assert np.allclose(ga["dq"] + ga["dlq"] / q, gb["dq"], rtol=1e-10, atol=1e-12)
    assert np.allclose(ga["dk"] + ga["dlk"] / k, gb["dk"], rtol=1e-10, atol=1e-12)
    for n in ("dv", "dg", "dmeta_k"):
        assert np.allclose(ga[n], gb[n], rtol=1e-12, atol=1e-13), n


def test_layer_with_features_finite_differences():
    rng = np.random.default_rng(4)
    B, H, L, d, M, W = 1, 1, 9, 4, 1, 4
    q, k, v, dO = (rnd(rng, B, H, L, d) for _ in range(4))
    lq, lk = rnd(rng, B, H, L, d, s=0.5) - 1.0, rnd(rng, B, H, L, d, s=0.5) - 1.0
    g = -np.abs(rnd(rng, B, H, L, d, s=0.2))
    mk = rnd(rng, H, M, d)
    out = fm.hybrid_backward_features(q, k, v, lq, lk, g, mk, None, dO, window=W, scale=0.5)
    args = {"q": q, "k": k, "v": v, "lq": lq, "lk": lk, "g": g}

    def loss(**kw):
        a = dict(args)
        a.update(kw)
        o = fm.hybrid_forward_features(a["q"], a["k"], a["v"], a["lq"], a["lk"], a["g"], mk, window=W,
                                       scale=0.5)["o"]
        return float((o * dO).sum())

    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("lq", "dlq"), ("lk", "dlk"), ("g", "dg")):
        for _ in range(3):
            idx = tuple(rng.integers(0, s) for s in args[name].shape)
            ap, am = args[name].copy(), args[name].copy()
            ap[idx] += h
            am[idx] -= h
            fd = (loss(**{name: ap}) - loss(**{name: am})) / (2 * h)
            assert abs(fd - out[gname][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx)


def test_feature_decode_continues_the_sequence():
    """A prefill of P tokens, then decode steps with log features, equal the whole-sequence
    log-feature forward at the decoded positions (W smaller and larger than P)."""
    rng = np.random.default_rng(6)
    B, H, L, d, M = 2, 2, 14, 4, 2
    q, k, v = (rnd(rng, B, H, L, d) for _ in range(3))
    lq, lk = rnd(rng, B, H, L, d, s=0.5) - 1.0, rnd(rng, B, H, L, d, s=0.5) - 1.0
    g = -np.abs(rnd(rng, B, H, L, d, s=0.3))
    mk = rnd(rng, H, M, d)
    for W, P in ((4, 9), (20, 5)):
        full = fm.hybrid_forward_features(q, k, v, lq, lk, g, mk, window=W, scale=0.5)
        pre = fm.hybrid_forward_features(q[:, :, :P], k[:, :, :P], v[:, :, :P], lq[:, :, :P], lk[:, :, :P],
                                         g[:, :, :P], mk, window=W, scale=0.5)
        st = orc.DecodeState.from_prefix(k[:, :, :P], v[:, :, :P], pre["state"], W)
        for t in range(P, L):
            o = fm.decode_step_features(st, q[:, :, t], k[:, :, t], v[:, :, t], lq[:, :, t], lk[:, :, t], g[:, :, t],
                                        mk, None, scale=0.5)
            assert np.allclose(o, full["o"][:, :, t], rtol=1e-12, atol=1e-12), (W, P, t)
        assert np.allclose(st.S, full["state"], rtol=1e-12, atol=1e-12)

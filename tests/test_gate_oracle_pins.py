"""Pins of the gate-projection oracle against closed forms, a library routine,
finite differences and its invariants (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle.gate_projection import gate_projection, gate_projection_backward, logsigmoid


def test_logsigmoid_closed_forms():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4; far tails: -e^{-z} and z
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0])
    want = np.array([-math.log(2.0), math.log(0.75), math.log(0.25), -math.exp(-40.0), -40.0])
    got = logsigmoid(z)
    assert np.allclose(got[:3], want[:3], rtol=1e-15, atol=0)
    assert abs(got[3] - want[3]) <= 1e-15 * abs(want[3])          # relative, not absolute, accuracy
    assert abs(got[4] - want[4]) <= 1e-15 * 40.0


def test_gate_values_through_the_projection():
    # d_model = 1, x = 1: g is logsigmoid of the weight itself, divided by tau
    x = np.ones((1, 1, 1))
    w = np.array([[0.0], [math.log(3.0)]])
    g = gate_projection(x, w, heads=1, tau=2.0)
    assert g.shape == (1, 1, 1, 2)
    assert np.allclose(g[0, 0, 0], [-math.log(2.0) / 2, math.log(0.75) / 2], rtol=1e-15, atol=0)


@pytest.mark.parametrize("scalar", [False, True])
def test_layout_elementwise(scalar):
    """Each sampled output element recomputed on its own with Python floats."""
    rng = np.random.default_rng(3)
    B, H, L, dk, Dm, tau = 2, 3, 5, 2, 7, 4.0
    Ng = H if scalar else H * dk
    x = rng.standard_normal((B, L, Dm))
    w = rng.standard_normal((Ng, Dm))
    g = gate_projection(x, w, H, tau=tau, scalar=scalar)
    assert g.shape == ((B, H, L) if scalar else (B, H, L, dk))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for i in range(1 if scalar else dk):
                    n = h if scalar else h * dk + i
                    z = sum(float(x[b, t, m]) * float(w[n, m]) for m in range(Dm))
                    want = -math.log1p(math.exp(-z)) / tau
                    got = g[b, h, t] if scalar else g[b, h, t, i]
                    assert abs(got - want) <= 1e-13 * max(1.0, abs(want)), (b, h, t, i)


@pytest.mark.parametrize("scalar", [False, True])
def test_against_torch_autograd(scalar):
    rng = np.random.default_rng(11)
    B, H, L, dk, Dm, tau = 2, 4, 9, 8, 24, 16.0
    Ng = H if scalar else H * dk
    x = rng.standard_normal((B, L, Dm))
    w = rng.standard_normal((Ng, Dm)) / math.sqrt(Dm)
    dg = rng.standard_normal((B, H, L) if scalar else (B, H, L, dk))
    g = gate_projection(x, w, H, tau=tau, scalar=scalar)
    dx, dw = gate_projection_backward(x, w, H, dg, tau=tau, scalar=scalar)

    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = torch.nn.functional.logsigmoid(torch.nn.functional.linear(xt, wt)) / tau     # [B, L, Ng]
    yg = y.permute(0, 2, 1) if scalar else y.reshape(B, L, H, dk).permute(0, 2, 1, 3)
    (yg * torch.tensor(dg)).sum().backward()
    assert np.allclose(g, yg.detach().numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-13)
    assert np.allclose(dw, wt.grad.numpy(), rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("scalar", [False, True])
def test_backward_finite_differences(scalar):
    rng = np.random.default_rng(5)
    B, H, L, dk, Dm, tau = 1, 2, 4, 4, 6, 3.0
    Ng = H if scalar else H * dk
    x = rng.standard_normal((B, L, Dm))
    w = rng.standard_normal((Ng, Dm))
    dg = rng.standard_normal((B, H, L) if scalar else (B, H, L, dk))
    dx, dw = gate_projection_backward(x, w, H, dg, tau=tau, scalar=scalar)
    f = lambda xx, ww: float((gate_projection(xx, ww, H, tau=tau, scalar=scalar) * dg).sum())
    h = 1e-6
    for _ in range(6):
        idx = tuple(rng.integers(0, s) for s in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        assert abs((f(xp, w) - f(xm, w)) / (2 * h) - dx[idx]) <= 1e-7 * max(1.0, abs(dx[idx]))
        jdx = tuple(rng.integers(0, s) for s in w.shape)
        wp, wm = w.copy(), w.copy()
        wp[jdx] += h
        wm[jdx] -= h
        assert abs((f(x, wp) - f(x, wm)) / (2 * h) - dw[jdx]) <= 1e-7 * max(1.0, abs(dw[jdx]))


def test_invariants():
    rng = np.random.default_rng(8)
    B, H, L, dk, Dm = 2, 2, 6, 4, 10
    x = rng.standard_normal((B, L, Dm)) * 3
    w = rng.standard_normal((H * dk, Dm))
    g1 = gate_projection(x, w, H, tau=1.0)
    g16 = gate_projection(x, w, H, tau=16.0)
    assert (g1 <= 0).all()                          # sigmoid < 1: the decay never grows the state
    assert np.allclose(g16, g1 / 16.0, rtol=1e-15, atol=0)
    # the scalar gate built from rows h*dk of the per-dimension weight is that column of g
    gs = gate_projection(x, w[::dk], H, tau=1.0, scalar=True)
    assert np.allclose(gs, g1[..., 0], rtol=1e-15, atol=0)

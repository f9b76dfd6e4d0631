"""Pins of the stage-1 (attention approximation) oracle: the teacher attention
against torch's scaled-dot-product attention and closed forms, the loss and its
gradient against autograd and finite differences, the composed step against
finite differences of its loss (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import distill as dst
from oracle import lizard_oracle as orc


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


@pytest.mark.parametrize("L", [1, 7, 40])
def test_teacher_is_causal_sdpa(L):
    rng = np.random.default_rng(L)
    q, k, v = (rnd(rng, 2, 3, L, 8) for _ in range(3))
    o = dst.teacher_attention(q, k, v, scale=0.4)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                                           is_causal=True, scale=0.4).numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_teacher_rows_match_full():
    rng = np.random.default_rng(9)
    q, k, v = (rnd(rng, 1, 1, 30, 6) for _ in range(3))
    full = dst.teacher_attention(q, k, v, scale=0.3)
    rows = [0, 7, 29]
    assert np.allclose(dst.teacher_attention_rows(q[0, 0], k[0, 0], v[0, 0], rows, scale=0.3), full[0, 0, rows],
                       rtol=1e-13, atol=1e-14)


def test_teacher_closed_forms():
    rng = np.random.default_rng(1)
    L = 9
    k, v = rnd(rng, 1, 2, L, 4), rnd(rng, 1, 2, L, 4)
    # zero queries: uniform weights over the prefix, o_t = mean of v_0..v_t
    o = dst.teacher_attention(np.zeros((1, 2, L, 4)), k, v, scale=1.0)
    assert np.allclose(o, np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None], rtol=1e-13, atol=0)
    # the first token attends only to itself
    q = rnd(rng, 1, 2, L, 4)
    assert np.allclose(dst.teacher_attention(q, k, v, scale=0.5)[:, :, 0], v[:, :, 0], rtol=1e-14, atol=0)
    # adding one vector to every key shifts each row's logits by a constant: no change
    o1 = dst.teacher_attention(q, k, v, scale=0.5)
    o2 = dst.teacher_attention(q, k + rnd(rng, 1, 2, 1, 4), v, scale=0.5)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)


def test_mse_and_grad():
    rng = np.random.default_rng(2)
    a, b = rnd(rng, 2, 2, 5, 3), rnd(rng, 2, 2, 5, 3)
    loss, dO = dst.mse_and_grad(a, b)
    at = torch.tensor(a, requires_grad=True)
    lt = torch.nn.functional.mse_loss(at, torch.tensor(b))
    lt.backward()
    assert abs(loss - lt.item()) <= 1e-15 * max(1.0, loss)
    assert np.allclose(dO, at.grad.numpy(), rtol=1e-13, atol=0)
    # closed form on a 2-element case: ((3-1)^2 + (0-2)^2)/2 = 4
    l2, d2 = dst.mse_and_grad(np.array([3.0, 0.0]), np.array([1.0, 2.0]))
    assert l2 == 4.0 and np.array_equal(d2, np.array([2.0, -2.0]))


def test_stage1_step_finite_differences():
    """The step's gradients are those of its own loss with the teacher held fixed."""
    rng = np.random.default_rng(3)
    B, H, L, D, M, W, scale = 1, 2, 12, 4, 2, 5, 0.5
    q, k, v = (rnd(rng, B, H, L, D, s=0.5) for _ in range(3))
    teacher = tuple(rnd(rng, B, H, L, D, s=0.5) for _ in range(3))
    g = -np.abs(rnd(rng, B, H, L, D, s=0.3))
    mk = rnd(rng, H, M, D, s=0.5)
    out = dst.stage1_step(q, k, v, g, mk, None, window=W, scale=scale, teacher=teacher)
    o_t = dst.teacher_attention(*teacher, scale=scale)

    def loss_of(qq, kk, vv, gg, mm):
        o = orc.hybrid_forward(qq, kk, vv, gg, mm, None, window=W, scale=scale)["o"]
        return dst.mse_and_grad(o, o_t)[0]

    assert abs(loss_of(q, k, v, g, mk) - out["loss"]) <= 1e-15
    h = 1e-6
    args = [q, k, v, g, mk]
    for ai, name in enumerate(["dq", "dk", "dv", "dg", "dmeta_k"]):
        for _ in range(3):
            idx = tuple(rng.integers(0, s) for s in args[ai].shape)
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[ai][idx] += h
            am[ai][idx] -= h
            fd = (loss_of(*ap) - loss_of(*am)) / (2 * h)
            assert abs(fd - out[name][idx]) <= 1e-6 * max(1e-3, abs(fd)), (name, idx, fd, out[name][idx])

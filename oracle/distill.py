"""CPU oracle for the stage-1 attention-approximation step of Lizard.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

What it computes, with the passages it follows (gist.science explainer of
"Lizard: An Efficient Linearization Framework for Large Language Models"):
the first training stage fits the linearized layer to the teacher's softmax
attention output with a mean squared error (English page §2, "Stage 1:
Attention Approximation"; French page "Étape 1"; Spanish page "Etapa 1";
Chinese page, first training stage).  At the level of one attention layer:

    o_T  = causal softmax attention of the teacher's q, k, v (scale 1/sqrt(d))
    o_S  = the Lizard layer's output (GLA branch + anchor window)
    loss = mean over every element of (o_S - o_T)^2
    dO   = d loss / d o_S = 2 (o_S - o_T) / N,   N = B*H*L*d_v

and the layer's backward from dO gives the gradients that train the
student's gates and meta tokens.  The teacher is frozen: no gradient flows
into o_T.  The teacher attention is the anchor window of the layer with a
window that covers the whole prefix and no meta tokens (its oracle reading:
W >= L is full causal attention), so it is evaluated with that oracle
function, whose pins include torch's scaled-dot-product attention.
"""
from __future__ import annotations

import numpy as np

from . import lizard_oracle as orc

__all__ = ["teacher_attention", "teacher_attention_rows", "mse_and_grad", "stage1_step"]


def teacher_attention(q, k, v, *, scale):
    """o_T[t] = sum_{s <= t} softmax_s(scale * q_t . k_s) v_s for every (b, h)."""
    q = np.asarray(q, np.float64)
    H, L, D = q.shape[1], q.shape[2], q.shape[3]
    no_meta = np.zeros((H, 0, D))
    o, _ = orc.window_forward(q, k, v, no_meta, None, max(L, 1), scale)
    return o


def teacher_attention_rows(q, k, v, rows, *, scale):
    """Rows ``rows`` of teacher_attention for one (b, h): q, k, v [L, d]; returns [len(rows), d].
    The same definition evaluated only where asked (for sampled checks at long L)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    out = np.empty((len(rows), v.shape[-1]))
    for n, t in enumerate(rows):
        logits = scale * (k[:t + 1] @ q[t])
        p = np.exp(logits - logits.max())
        out[n] = (p / p.sum()) @ v[:t + 1]
    return out


def mse_and_grad(o_student, o_teacher):
    """loss = mean((o_S - o_T)^2) over every element; dO = 2 (o_S - o_T) / N."""
    d = np.asarray(o_student, np.float64) - np.asarray(o_teacher, np.float64)
    n = d.size
    return float(np.sum(d * d) / n), 2.0 * d / n


def stage1_step(q, k, v, g, meta_k, meta_v, *, window, scale, mix=1.0, teacher=None):
    """One attention-approximation step: the student forward, the teacher attention, the
    loss and its gradient dO, and the student backward from dO.

    ``teacher``: (q_T, k_T, v_T) of the teacher, or None to use the student's own q, k, v.
    Returns a dict with loss, dO, o (student), o_teacher and the student gradients
    dq, dk, dv, dg, dmeta_k (and dmeta_v when meta_v is given)."""
    qt, kt, vt = (q, k, v) if teacher is None else teacher
    fwd = orc.hybrid_forward(q, k, v, g, meta_k, meta_v, window=window, scale=scale, mix=mix)
    o_t = teacher_attention(qt, kt, vt, scale=scale)
    loss, dO = mse_and_grad(fwd["o"], o_t)
    grads = orc.hybrid_backward(q, k, v, g, meta_k, meta_v, dO, window=window, scale=scale, mix=mix)
    out = {"loss": loss, "dO": dO, "o": fwd["o"], "o_teacher": o_t}
    out.update(grads)
    return out

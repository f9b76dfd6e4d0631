"""CPU oracle for the Lizard hybrid attention layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product path.

What it computes, with the passage each step follows.  Sources are the
explainer pages for "Lizard: An Efficient Linearization Framework for Large
Language Models" (gist.science, English / French / Spanish / Chinese):

* GLA branch -- English page, §2.A "Hybrid Attention Architecture", state
  update S_i = Gamma_i S_{i-1} + phi(k_i) v_i^T with Gamma_i = sigmoid(W x_i)
  (French page §2.A, Chinese page §2.1 give the same gate).  The gate enters
  here as its logarithm g = log Gamma (English page §2.C "Hardware-Aware
  Algorithm": the gate is handled in log space), one value per key dimension,
  so Gamma_i = diag(exp g_i).  q and k arrive after any feature map phi.  The
  output reads the updated state: o_t = q_t S_t.
* Scalar gate -- the Chinese page's ablation (section on ablation experiments)
  finds a lightweight scalar gate works better than richer gate structures:
  one log-gate per head and token, g [B,H,L], Gamma_t = exp(g_t) I.  Every
  function below accepts it wherever it accepts a per-dimension gate; its
  gradient is the derivative with respect to that one value.
* Anchor-window branch -- English page §2.A: a local sliding window plus
  learnable meta-memory tokens that act as sinks in the softmax denominator
  without contributing directly to the output value (French page §2.A: the
  window is local; its lay text gives ~128 tokens).  Query t attends to keys
  s in [t-W+1, t] (W counts the current token) plus M meta keys shared across
  the batch; meta values are zero unless given.  Logit scale 1/sqrt(d_k).
* Output -- English page §2.A "Final Output": Y = Y_gate + alpha * Y_anchor.
* Backward -- the pages give none; it is the exact gradient of the forward
  above, derived by hand (formulas in each function's docstring).
* Decode -- English page §4 "Efficiency" (constant memory at any length) and
  French page §2.A (O(1) inference by updating an incremental hidden state):
  the state S plus a ring of the last W keys/values is the whole decode state.

Everything is plain numpy, evaluated in float64 by default (``dtype`` selects
float32 for the CPU-baseline timing only).  Loops run token by token exactly
as the definitions read; numpy vectorises only over batch and heads.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "gla_forward", "window_forward", "hybrid_forward",
    "gla_backward", "window_backward", "hybrid_backward",
    "DecodeState", "decode_step", "decode_window",
]


def _as(x, dtype):
    return None if x is None else np.asarray(x, dtype=dtype)


def _decay(g, ndim_tok):
    """exp(g) shaped to scale state rows: a per-dimension gate [..., dk] keeps its
    last axis; a scalar gate (one fewer axis than q) gains a unit axis."""
    a = np.exp(g)
    return a if g.ndim == ndim_tok else a[..., None]


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def gla_forward(q, k, v, g, *, dtype=np.float64, initial_state=None, return_states=False):
    """Gated linear attention, token by token (English page §2.A).

    S_{-1} = initial_state (zero by default);
    S_t = diag(exp g_t) S_{t-1} + k_t^T v_t ;  o_t = q_t S_t.

    q, k: [B,H,L,dk]; v: [B,H,L,dv]; g: [B,H,L,dk] or scalar per head [B,H,L].
    Returns (o [B,H,L,dv], S_final [B,H,dk,dv]) and, with ``return_states``,
    the list of every S_t.
    """
    q, k, v, g = (_as(a, dtype) for a in (q, k, v, g))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv), dtype) if initial_state is None else np.array(initial_state, dtype)
    a = _decay(g, q.ndim)
    o = np.empty((B, H, L, dv), dtype)
    states = []
    for t in range(L):
        S = a[:, :, t, :, None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        o[:, :, t, :] = np.matmul(q[:, :, t, None, :], S)[:, :, 0, :]
        if return_states:
            states.append(S.copy())
    if return_states:
        return o, S, states
    return o, S


def _window_row(q_t, k, v, meta_k, meta_v, lo, hi, scale):
    """Softmax weights of one query row over M meta keys plus keys [lo, hi]."""
    kw = k[:, :, lo:hi + 1, :]                                  # [B,H,n,dk]
    lw = scale * np.matmul(kw, q_t[..., None])[..., 0]          # [B,H,n]
    lm = scale * np.einsum("bhd,hmd->bhm", q_t, meta_k)         # [B,H,M]
    logits = np.concatenate([lm, lw], axis=-1)
    mx = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - mx)
    l = e.sum(axis=-1, keepdims=True)
    p = e / l
    lse = (mx + np.log(l))[..., 0]
    return p, lse


def window_forward(q, k, v, meta_k, meta_v, window, scale, *, dtype=np.float64):
    """Anchor-window softmax branch (English page §2.A, anchor window).

    For query t: logits scale*q_t.k_s for s in [max(0,t-W+1), t] and
    scale*q_t.mk_m for every meta key m; p = softmax over those M+n entries;
    o_t = sum_s p_ts v_s + sum_m p_tm mv_m (mv = 0 when ``meta_v`` is None).
    Returns (o_swa [B,H,L,dv], lse [B,H,L]).
    """
    q, k, v, meta_k, meta_v = (_as(a, dtype) for a in (q, k, v, meta_k, meta_v))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    M = meta_k.shape[1]
    o = np.empty((B, H, L, dv), dtype)
    lse = np.empty((B, H, L), dtype)
    for t in range(L):
        lo = max(0, t - window + 1)
        p, lse[:, :, t] = _window_row(q[:, :, t], k, v, meta_k, meta_v, lo, t, scale)
        ot = np.matmul(p[:, :, None, M:], v[:, :, lo:t + 1, :])[:, :, 0, :]
        if meta_v is not None and M > 0:
            ot = ot + np.einsum("bhm,hmd->bhd", p[:, :, :M], meta_v)
        o[:, :, t, :] = ot
    return o, lse


def hybrid_forward(q, k, v, g, meta_k, meta_v=None, *, window, scale, mix=1.0,
                   dtype=np.float64, initial_state=None):
    """Lizard output o = o_gla + mix * o_swa (English page §2.A "Final Output").

    Returns dict(o, o_gla, o_swa, lse, state) with ``state`` the GLA state
    after the last token (the prefill-to-decode hand-off).
    """
    o_gla, S = gla_forward(q, k, v, g, dtype=dtype, initial_state=initial_state)
    o_swa, lse = window_forward(q, k, v, meta_k, meta_v, window, scale, dtype=dtype)
    return dict(o=o_gla + mix * o_swa, o_gla=o_gla, o_swa=o_swa, lse=lse, state=S)


# --------------------------------------------------------------------------
# Backward (exact gradients of the forward above; the pages print no backward)
# --------------------------------------------------------------------------

def gla_backward(q, k, v, g, dO, *, dtype=np.float64):
    """Gradient of sum_t dO_t . o^gla_t with respect to q, k, v, g.

    Forward sweep:  dq_t = dO_t S_t^T   (dq_t[i] = sum_j S_t[i,j] dO_t[j]).
    Reverse sweep:  dS_t = q_t^T dO_t + diag(exp g_{t+1}) dS_{t+1}, dS_L = 0;
                    dk_t = v_t dS_t^T,  dv_t = k_t dS_t.
    Gates: with b_t = sum_{r<=t} g_r, o depends on g only through
    exp(b_t - b_s); dL/db_u = q_u*dq_u - k_u*dk_u, hence
    dg_r = sum_{u>=r} (q_u*dq_u - k_u*dk_u)  (a reverse cumulative sum).
    A scalar gate [B,H,L] scales every key dimension by the same b_t, so its
    dL/db_u is the sum of those terms over the key dimensions.
    """
    q, k, v, g, dO = (_as(a, dtype) for a in (q, k, v, g, dO))
    B, H, L, dk_ = q.shape
    dv_ = v.shape[-1]
    a = _decay(g, q.ndim)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    S = np.zeros((B, H, dk_, dv_), dtype)
    for t in range(L):
        S = a[:, :, t, :, None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        dq[:, :, t, :] = np.matmul(S, dO[:, :, t, :, None])[..., 0]
    carry = np.zeros((B, H, dk_, dv_), dtype)       # diag(a_{t+1}) dS_{t+1}
    for t in range(L - 1, -1, -1):
        dS = q[:, :, t, :, None] * dO[:, :, t, None, :] + carry
        dk[:, :, t, :] = np.matmul(dS, v[:, :, t, :, None])[..., 0]
        dv[:, :, t, :] = np.matmul(k[:, :, t, None, :], dS)[:, :, 0, :]
        carry = a[:, :, t, :, None] * dS
    contrib = q * dq - k * dk
    if g.ndim != q.ndim:
        contrib = contrib.sum(-1)
    dg = np.flip(np.cumsum(np.flip(contrib, axis=2), axis=2), axis=2)
    return dq, dk, dv, dg


def window_backward(q, k, v, meta_k, meta_v, dO, window, scale, mix, *, dtype=np.float64):
    """Gradient of sum_t (mix*dO_t) . o^swa_t (explicit softmax Jacobian).

    With ob_t = mix*dO_t and p the forward softmax weights of row t:
    dp_ts = ob_t.v_s, dp_tm = ob_t.mv_m (0 without meta values),
    D_t = sum_x p_tx dp_tx,  dl_tx = p_tx (dp_tx - D_t);
    dq_t = scale * (sum_s dl_ts k_s + sum_m dl_tm mk_m),
    dk_s += scale dl_ts q_t,  dv_s += p_ts ob_t,
    dmk_m = sum_{b,t} scale dl_tm q_t,  dmv_m = sum_{b,t} p_tm ob_t.
    Returns (dq, dk, dv, dmeta_k [H,M,dk], dmeta_v [H,M,dv] or None).
    """
    q, k, v, meta_k, meta_v, dO = (_as(a, dtype) for a in (q, k, v, meta_k, meta_v, dO))
    B, H, L, dk_ = q.shape
    M = meta_k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dmk = np.zeros_like(meta_k)
    dmv = None if meta_v is None else np.zeros_like(meta_v)
    for t in range(L):
        lo = max(0, t - window + 1)
        p, _ = _window_row(q[:, :, t], k, v, meta_k, meta_v, lo, t, scale)
        ob = mix * dO[:, :, t, :]                                          # [B,H,dv]
        dp_w = np.matmul(v[:, :, lo:t + 1, :], ob[..., None])[..., 0]      # [B,H,n]
        if meta_v is not None:
            dp_m = np.einsum("bhd,hmd->bhm", ob, meta_v)
        else:
            dp_m = np.zeros((B, H, M), dtype)
        dp = np.concatenate([dp_m, dp_w], axis=-1)
        Dt = (p * dp).sum(axis=-1, keepdims=True)
        dl = p * (dp - Dt)
        dq[:, :, t, :] = scale * (np.matmul(dl[:, :, None, M:], k[:, :, lo:t + 1, :])[:, :, 0, :]
                                  + np.einsum("bhm,hmd->bhd", dl[:, :, :M], meta_k))
        dk[:, :, lo:t + 1, :] += scale * dl[:, :, M:, None] * q[:, :, t, None, :]
        dv[:, :, lo:t + 1, :] += p[:, :, M:, None] * ob[:, :, None, :]
        dmk += scale * np.einsum("bhm,bhd->hmd", dl[:, :, :M], q[:, :, t, :])
        if dmv is not None:
            dmv += np.einsum("bhm,bhd->hmd", p[:, :, :M], ob)
    return dq, dk, dv, dmk, dmv


def hybrid_backward(q, k, v, g, meta_k, meta_v, dO, *, window, scale, mix=1.0, dtype=np.float64):
    """Gradients of sum_t dO_t . o_t for o = o_gla + mix * o_swa.

    Returns dict(dq, dk, dv, dg, dmeta_k, dmeta_v).
    """
    gq, gk, gv, dg = gla_backward(q, k, v, g, dO, dtype=dtype)
    wq, wk, wv, dmk, dmv = window_backward(q, k, v, meta_k, meta_v, dO, window, scale, mix,
                                           dtype=dtype)
    return dict(dq=gq + wq, dk=gk + wk, dv=gv + wv, dg=dg, dmeta_k=dmk, dmeta_v=dmv)


# --------------------------------------------------------------------------
# Constant-memory decode
# --------------------------------------------------------------------------

class DecodeState:
    """Whole decode state: GLA state S, a ring of the last W keys/values, pos.

    Slot of token number ``pos`` is ``pos mod W``; ``pos`` counts the tokens
    already consumed by each sequence.
    """

    def __init__(self, B, H, dk, dv, window, dtype=np.float64):
        self.S = np.zeros((B, H, dk, dv), dtype)
        self.ring_k = np.zeros((B, H, window, dk), dtype)
        self.ring_v = np.zeros((B, H, window, dv), dtype)
        self.pos = np.zeros((B,), np.int64)
        self.window = window
        self.dtype = dtype

    @classmethod
    def from_prefix(cls, k, v, state, window, dtype=np.float64):
        """Hand-off after a prefill of L tokens: GLA state plus the last
        min(L, W) keys/values placed in their ring slots."""
        k, v = _as(k, dtype), _as(v, dtype)
        B, H, L, dk = k.shape
        st = cls(B, H, dk, v.shape[-1], window, dtype)
        st.S = np.array(state, dtype)
        for t in range(max(0, L - window), L):
            st.ring_k[:, :, t % window] = k[:, :, t]
            st.ring_v[:, :, t % window] = v[:, :, t]
        st.pos[:] = L
        return st


def decode_window(st: DecodeState, q, k, v, meta_k, meta_v, *, scale):
    """The anchor window of one decode step: the new key/value goes to slot pos mod W, then
    softmax attention of q over the M meta keys and the min(pos+1, W) filled ring slots.
    Returns o_swa [B,H,dv]; pos is not advanced."""
    dt = st.dtype
    q, k, v, meta_k, meta_v = (_as(a, dt) for a in (q, k, v, meta_k, meta_v))
    B = q.shape[0]
    M = meta_k.shape[1]
    W = st.window
    o_swa = np.empty(v.shape, dt)
    for b in range(B):
        slot = int(st.pos[b] % W)
        st.ring_k[b, :, slot] = k[b]
        st.ring_v[b, :, slot] = v[b]
        n = int(min(st.pos[b] + 1, W))
        keys = st.ring_k[b, :, :n]                                    # [H,n,dk]
        vals = st.ring_v[b, :, :n]
        lw = scale * np.einsum("hd,hnd->hn", q[b], keys)
        lm = scale * np.einsum("hd,hmd->hm", q[b], meta_k)
        logits = np.concatenate([lm, lw], axis=-1)
        e = np.exp(logits - logits.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)
        ob = np.einsum("hn,hnd->hd", p[:, M:], vals)
        if meta_v is not None and M > 0:
            ob = ob + np.einsum("hm,hmd->hd", p[:, :M], meta_v)
        o_swa[b] = ob
    return o_swa


def decode_step(st: DecodeState, q, k, v, g, meta_k, meta_v, *, scale, mix=1.0):
    """One token for every sequence (q, k, v: [B,H,d]; g: [B,H,d] or scalar [B,H]);
    returns o [B,H,dv].

    S <- diag(exp g) S + k^T v; o_gla = q S; the new key/value goes to slot
    pos mod W; o_swa = softmax attention of q over the M meta keys and the
    min(pos+1, W) filled ring slots; o = o_gla + mix*o_swa; pos += 1.
    """
    dt = st.dtype
    q, k, v, g = (_as(a, dt) for a in (q, k, v, g))
    st.S = _decay(g, q.ndim)[..., None] * st.S + k[..., :, None] * v[..., None, :]
    o_gla = np.matmul(q[:, :, None, :], st.S)[:, :, 0, :]
    o_swa = decode_window(st, q, k, v, meta_k, meta_v, scale=scale)
    st.pos += 1
    return o_gla + mix * o_swa

"""GPU parity of lizard_attn_fwd_continue (chunked prefill resuming from a carried
state, key/value ring and per-sequence position).  The continued forward must
equal the oracle's forward of the whole sequence restricted to the new tokens,
leave the carry the oracle's state after them, and agree bit for bit with the
one-shot forward where both compute the same thing."""
import math

import numpy as np
import pytest
import torch

from oracle import lizard_oracle as orc
from gated_linear_attention_chunkwise_amd import (continue_workspace, lizard_attn_decode_step,
                                                  lizard_attn_fwd, lizard_attn_fwd_continue)
from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs_device, make_small
from helpers import TOL, dev, host, rel_l2, tdtype

pytestmark = pytest.mark.gpu


def empty_carry(B, H, W, D, dt):
    state = torch.zeros(B, H, D, D, device="cuda", dtype=torch.float32)
    ring_k = torch.zeros(B, H, W, D, device="cuda", dtype=dt)
    return state, ring_k, torch.zeros_like(ring_k), torch.zeros(B, device="cuda", dtype=torch.int32)


def carry_after(T, b, P, mk, mv, W, scale, mix, seg):
    """Carry of sequence b after its first P tokens, built by continued segments of
    at most `seg` tokens from an empty carry."""
    H, D = T["q"].shape[1], T["q"].shape[3]
    carry = empty_carry(1, H, W, D, T["q"].dtype)
    for a in range(0, P, seg):
        e = min(P, a + seg)
        lizard_attn_fwd_continue(*(T[n][b:b + 1, :, a:e].contiguous() for n in "qkvg"), mk, mv, *carry,
                                 window=W, scale=scale, mix=mix)
    return carry


CASES = [
    # dtype, D, prefix lengths per sequence, segment length, W, M, meta values, prefix segment
    ("fp32", 64, (0, 37, 150), 70, 64, 4, False, 64),
    ("bf16", 64, (5, 0, 129), 64, 128, 4, True, 50),
    ("bf16", 128, (200, 63, 1), 100, 128, 4, False, 128),
    ("bf16", 128, (130, 3, 64), 1, 129, 16, True, 33),
    ("bf16", 64, (17, 0, 300), 130, 1, 0, False, 100),
    ("fp32", 64, (64, 128, 2), 200, 129, 2, True, 64),
    # a window of several chunks held in the ring
    ("bf16", 128, (300, 20, 0), 150, 260, 4, True, 90),
    # a segment long enough for the state sweep to run in sequence segments from the carried state
    ("bf16", 64, (100, 0, 3000), 2100, 64, 4, False, 1024),
]


@pytest.mark.parametrize("dtname,D,prefix,L,W,M,with_mv,seg", CASES)
def test_continue_matches_full_sequence(dtname, D, prefix, L, W, M, with_mv, seg):
    B, H = len(prefix), 2
    N = max(prefix) + L
    x = make_small(B, H, N, D, M, seed=N + 7 * L + W, bf16=(dtname == "bf16"), with_grad=False,
                   with_meta_v=with_mv)
    dt = tdtype(dtname)
    scale, mix = 1.0 / math.sqrt(D), 0.75
    T = {n: dev(x[n], dt) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], dt) if M > 0 else None
    mv = dev(x["meta_v"], dt) if with_mv else None
    # per-sequence carries (different lengths), stacked into one batch
    parts = [carry_after(T, b, prefix[b], mk, mv, W, scale, mix, seg) for b in range(B)]
    state, rk, rv, pos = (torch.cat([p[i] for p in parts]).contiguous() for i in range(4))
    # the next L tokens of every sequence: tokens prefix[b] .. prefix[b] + L
    seg_in = {n: torch.stack([T[n][b, :, prefix[b]:prefix[b] + L] for b in range(B)]).contiguous()
              for n in "qkvg"}
    o = lizard_attn_fwd_continue(*(seg_in[n] for n in "qkvg"), mk, mv, state, rk, rv, pos,
                                 window=W, scale=scale, mix=mix)
    torch.cuda.synchronize()
    for b in range(B):
        n = prefix[b] + L
        ref = orc.hybrid_forward(x["q"][b:b + 1, :, :n], x["k"][b:b + 1, :, :n], x["v"][b:b + 1, :, :n],
                                 x["g"][b:b + 1, :, :n], x["meta_k"], x.get("meta_v"),
                                 window=W, scale=scale, mix=mix)
        e_o = rel_l2(host(o[b:b + 1]), ref["o"][:, :, prefix[b]:])
        e_s = rel_l2(host(state[b:b + 1]), ref["state"])
        print(dtname, D, prefix[b], L, W, M, f"o {e_o:.2e} state {e_s:.2e}", flush=True)
        assert e_o <= TOL[dtname] and e_s <= TOL[dtname]
        # ring: the last min(n, W) keys / values of the sequence in slots t mod W, exactly
        ts = np.arange(max(0, n - W), n)
        assert torch.equal(rk[b][:, ts % W].cpu(), T["k"][b][:, ts].cpu())
        assert torch.equal(rv[b][:, ts % W].cpu(), T["v"][b][:, ts].cpu())
    assert pos.cpu().tolist() == [p + L for p in prefix]


@pytest.mark.parametrize("dtname,D,L,W,M", [("bf16", 128, 300, 128, 4), ("fp32", 64, 77, 64, 3),
                                            ("bf16", 64, 64, 1, 0)])
def test_continue_from_empty_carry_equals_forward(dtname, D, L, W, M):
    """pos = 0 and a zero state: the output is the one-shot forward's, bit for bit, and
    the carry is its final state and the last W keys / values."""
    x = make_small(2, 3, L, D, M, seed=L + W, bf16=(dtname == "bf16"), with_grad=False, with_meta_v=False)
    dt = tdtype(dtname)
    T = {n: dev(x[n], dt) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], dt) if M > 0 else None
    ref = lizard_attn_fwd(T["q"], T["k"], T["v"], T["g"], mk, None, window=W, want_state=True)
    state, rk, rv, pos = empty_carry(2, 3, W, D, dt)
    o = lizard_attn_fwd_continue(T["q"], T["k"], T["v"], T["g"], mk, None, state, rk, rv, pos, window=W)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"])
    assert torch.equal(state, ref["state"])
    ts = torch.arange(max(0, L - W), L, device="cuda")
    assert torch.equal(rk[:, :, ts % W], T["k"][:, :, ts]) and torch.equal(rv[:, :, ts % W], T["v"][:, :, ts])
    assert pos.cpu().tolist() == [L, L]


def test_continue_then_decode():
    """Continued segments, then decode steps on the same carry: the full sequence."""
    D, W, M, B, H = 128, 128, 4, 2, 2
    N = 260
    x = make_small(B, H, N, D, M, seed=5, bf16=True, with_grad=False, with_meta_v=False)
    T = {n: dev(x[n], torch.bfloat16) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], torch.bfloat16)
    carry = empty_carry(B, H, W, D, torch.bfloat16)
    outs = []
    for a, e in ((0, 100), (100, 101), (101, 230)):
        outs.append(lizard_attn_fwd_continue(*(T[n][:, :, a:e].contiguous() for n in "qkvg"), mk, None, *carry,
                                             window=W))
    for t in range(230, N):
        outs.append(lizard_attn_decode_step(*(T[n][:, :, t].contiguous() for n in "qkvg"), mk, None, *carry,
                                            window=W).unsqueeze(2))
    torch.cuda.synchronize()
    ref = orc.hybrid_forward(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=W,
                             scale=1.0 / math.sqrt(D))
    e_o = rel_l2(host(torch.cat(outs, 2)), ref["o"])
    e_s = rel_l2(host(carry[0]), ref["state"])
    print(f"o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]
    assert carry[3].cpu().tolist() == [N, N]


def test_continue_zero_length_is_noop():
    state, rk, rv, pos = empty_carry(1, 2, 8, 64, torch.bfloat16)
    state.fill_(0.5)
    pos.fill_(3)
    e = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o = lizard_attn_fwd_continue(e, e, e, e.float(), None, None, state, rk, rv, pos, window=8)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 64)
    assert bool((state == 0.5).all()) and pos.cpu().tolist() == [3]


def test_prefill_64k_in_segments_equals_one_shot():
    """The 65 536-token prefill (B=1, H=32, d=128, W=128, M=4) as eight continued
    8192-token segments against the one-shot forward (which the forward tests pin to the
    oracle on sampled heads): the same outputs and final state up to the rounding order
    of the state sums (both sweep the sequence in segments, cut differently)."""
    w = WORKLOADS["prefill_64k"]
    x = make_inputs_device(w, "cuda", with_grad=False)
    ref = lizard_attn_fwd(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=w.W, scale=w.scale,
                          want_state=True)
    S = 8192
    carry = empty_carry(w.B, w.H, w.W, w.D, torch.bfloat16)
    ws = continue_workspace(w.B, w.H, S, w.D, torch.bfloat16, "cuda")
    o = torch.empty_like(x["q"])
    for a in range(0, w.L, S):
        seg = {n: x[n][:, :, a:a + S].contiguous() for n in "qkvg"}
        o[:, :, a:a + S] = lizard_attn_fwd_continue(seg["q"], seg["k"], seg["v"], seg["g"], x["meta_k"], None,
                                                    *carry, window=w.W, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    e_o = rel_l2(host(o), host(ref["o"]))
    e_s = rel_l2(host(carry[0]), host(ref["state"]))
    print(f"chunked vs one-shot: o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= 1e-3 and e_s <= 1e-5
    assert carry[3].cpu().tolist() == [w.L]


@pytest.mark.parametrize("dtname,D,W", [("bf16", 128, 128), ("fp32", 64, 16)])
def test_variable_length_batched_decode(dtname, D, W):
    """Sequences of one batch at different positions (prefixes of 0, 5, 130 and 64
    tokens) decode together: each step's output per sequence is the oracle's output of
    that sequence at its own position."""
    prefix, steps, M = (0, 5, 130, 64), 12, 4
    B, H = len(prefix), 2
    N = max(prefix) + steps
    x = make_small(B, H, N, D, M, seed=11 * D + W, bf16=(dtname == "bf16"), with_grad=False, with_meta_v=True)
    dt = tdtype(dtname)
    scale, mix = 1.0 / math.sqrt(D), 0.5
    T = {n: dev(x[n], dt) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk, mv = dev(x["meta_k"], dt), dev(x["meta_v"], dt)
    parts = [carry_after(T, b, prefix[b], mk, mv, W, scale, mix, 64) for b in range(B)]
    state, rk, rv, pos = (torch.cat([p[i] for p in parts]).contiguous() for i in range(4))
    outs = []
    for j in range(steps):
        tok = {n: torch.stack([T[n][b, :, prefix[b] + j] for b in range(B)]).contiguous() for n in "qkvg"}
        outs.append(lizard_attn_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], mk, mv, state, rk, rv, pos,
                                            window=W, scale=scale, mix=mix))
    torch.cuda.synchronize()
    got = torch.stack(outs, 2)
    for b in range(B):
        n = prefix[b] + steps
        ref = orc.hybrid_forward(*(x[k][b:b + 1, :, :n] for k in ("q", "k", "v", "g")), x["meta_k"], x["meta_v"],
                                 window=W, scale=scale, mix=mix)
        e_o = rel_l2(host(got[b:b + 1]), ref["o"][:, :, prefix[b]:])
        e_s = rel_l2(host(state[b:b + 1]), ref["state"])
        print(dtname, D, W, prefix[b], f"o {e_o:.2e} state {e_s:.2e}", flush=True)
        assert e_o <= TOL[dtname] and e_s <= TOL[dtname]
    assert pos.cpu().tolist() == [p + steps for p in prefix]

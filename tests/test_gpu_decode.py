"""GPU parity of lizard_attn_decode_step: prefill (GPU forward) then decode
steps, checked against the oracle's full-sequence forward at the same
positions (decode after prefill must equal the full-sequence output)."""
import math

import numpy as np
import pytest
import torch

from oracle import lizard_oracle as orc
from gated_linear_attention_chunkwise_amd import lizard_attn_decode_step, lizard_attn_fwd
from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs_device, make_small
from helpers import TOL, dev, host, rel_l2, tdtype

pytestmark = pytest.mark.gpu


def prefill_handoff(q, k, v, g, mk, mv, W, scale, mix):
    """GPU forward over the prefix, then the decode state: final GLA state,
    ring slots t mod W for the last min(L, W) tokens, pos = L."""
    B, H, L, D = q.shape
    ring_k = torch.zeros(B, H, W, D, device=q.device, dtype=q.dtype)
    ring_v = torch.zeros_like(ring_k)
    if L > 0:
        out = lizard_attn_fwd(q, k, v, g, mk, mv, window=W, scale=scale, mix=mix, want_state=True)
        state = out["state"]
        ts = torch.arange(max(0, L - W), L, device=q.device)
        ring_k[:, :, ts % W] = k[:, :, ts]
        ring_v[:, :, ts % W] = v[:, :, ts]
    else:
        state = torch.zeros(B, H, D, D, device=q.device, dtype=torch.float32)
    pos = torch.full((B,), L, device=q.device, dtype=torch.int32)
    return state, ring_k, ring_v, pos


@pytest.mark.parametrize("dtname,D", [("fp32", 64), ("bf16", 64), ("bf16", 128), ("fp32", 128)])
@pytest.mark.parametrize("L0,steps,W,M,with_mv", [(20, 12, 8, 2, False), (3, 10, 8, 4, True),
                                                  (0, 9, 4, 0, False), (70, 20, 128, 4, False),
                                                  (130, 5, 129, 16, True)])
def test_decode_after_prefill(dtname, D, L0, steps, W, M, with_mv):
    x = make_small(3, 2, L0 + steps, D, M, seed=L0 + 31 * steps + W, bf16=(dtname == "bf16"),
                   with_grad=False, with_meta_v=with_mv)
    dt = tdtype(dtname)
    scale, mix = 1.0 / math.sqrt(D), 0.75
    T = {n: dev(x[n], dt) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], dt) if M > 0 else None
    mv = dev(x["meta_v"], dt) if with_mv else None
    pre = L0 if not (dtname == "fp32" and D == 128) else 0   # fp32 forward supports d=64 only
    state, rk, rv, pos = prefill_handoff(*(T[n][:, :, :pre].contiguous() for n in "qkvg"),
                                         mk, mv, W, scale, mix)
    outs = []
    for t in range(pre, L0 + steps):
        o = lizard_attn_decode_step(*(T[n][:, :, t].contiguous() for n in "qkvg"), mk, mv,
                                    state, rk, rv, pos, window=W, scale=scale, mix=mix)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.stack(outs, 2)
    ref = orc.hybrid_forward(x["q"], x["k"], x["v"], x["g"], x["meta_k"], x.get("meta_v"),
                             window=W, scale=scale, mix=mix)
    e_o = rel_l2(host(got), ref["o"][:, :, pre:])
    e_s = rel_l2(host(state), ref["state"])
    print(dtname, D, L0, steps, W, M, f"o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL[dtname] and e_s <= TOL[dtname]
    assert (pos.cpu().numpy() == L0 + steps).all()


@pytest.mark.parametrize("dtname,D,B,H,L0,steps,W,M", [
    ("bf16", 128, 5, 2, 1100, 6, 1000, 3),    # window of 1000 slots, ring wrapped; 10 heads: both head maps
    ("bf16", 64, 3, 3, 300, 4, 8192, 16),     # the largest ring, mostly empty
    ("fp32", 64, 1, 9, 40, 5, 33, 1),         # 9 heads: one group of 8 and a remainder
])
def test_decode_long_ring_and_head_maps(dtname, D, B, H, L0, steps, W, M):
    """Windows of many key blocks (the logits walk the ring in groups of blocks, the value sum
    beyond the rows loaded ahead), and head counts on either side of the workgroup map's groups
    of eight heads."""
    x = make_small(B, H, L0 + steps, D, M, seed=W + 7 * L0 + B * H, bf16=(dtname == "bf16"),
                   with_grad=False, with_meta_v=True)
    dt = tdtype(dtname)
    scale, mix = 1.0 / math.sqrt(D), 1.25
    T = {n: dev(x[n], dt) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk, mv = dev(x["meta_k"], dt), dev(x["meta_v"], dt)
    state, rk, rv, pos = prefill_handoff(*(T[n][:, :, :L0].contiguous() for n in "qkvg"), mk, mv, W, scale, mix)
    outs = [lizard_attn_decode_step(*(T[n][:, :, t].contiguous() for n in "qkvg"), mk, mv, state, rk, rv, pos,
                                    window=W, scale=scale, mix=mix) for t in range(L0, L0 + steps)]
    torch.cuda.synchronize()
    ref = orc.hybrid_forward(x["q"], x["k"], x["v"], x["g"], x["meta_k"], x["meta_v"], window=W, scale=scale,
                             mix=mix)
    e_o = rel_l2(host(torch.stack(outs, 2)), ref["o"][:, :, L0:])
    e_s = rel_l2(host(state), ref["state"])
    print(dtname, D, B, H, W, f"o {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL[dtname] and e_s <= TOL[dtname]
    assert (pos.cpu().numpy() == L0 + steps).all()


def test_decode_b64_full_size_sampled():
    """4096-token prefill + 1024 decode steps at B=64, H=32, d=128, W=128, M=4."""
    w = WORKLOADS["decode_b64"]
    x = make_inputs_device(w, "cuda")
    P, L = w.prefill, w.L
    state, rk, rv, pos = prefill_handoff(*(x[n][:, :, :P].contiguous() for n in "qkvg"),
                                         x["meta_k"], None, w.W, w.scale, 1.0)
    outs = torch.empty(L - P, w.B, w.H, w.D, device="cuda", dtype=torch.bfloat16)
    for t in range(P, L):
        lizard_attn_decode_step(*(x[n][:, :, t].contiguous() for n in "qkvg"), x["meta_k"], None,
                                state, rk, rv, pos, window=w.W, scale=w.scale, mix=1.0,
                                out=outs[t - P])
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (63, 31), (17, 5)]:
        sl = lambda n: x[n][b:b + 1, h:h + 1].float().cpu().numpy()
        ref = orc.hybrid_forward(sl("q"), sl("k"), sl("v"), sl("g"),
                                 x["meta_k"][h:h + 1].float().cpu().numpy(), None,
                                 window=w.W, scale=w.scale)
        e_o = rel_l2(host(outs[:, b, h]), ref["o"][0, 0, P:])
        e_s = rel_l2(host(state[b:b + 1, h:h + 1]), ref["state"])
        print("decode_b64", (b, h), f"o {e_o:.2e} state {e_s:.2e}", flush=True)
        assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]
    assert (pos.cpu().numpy() == L).all()


def test_decode_caller_workspace_matches_default():
    """A caller-owned workspace passed to every step gives bit-identical results to none (the
    step needs no workspace; one that is passed is left alone)."""
    from gated_linear_attention_chunkwise_amd import decode_workspace
    x = make_small(3, 4, 40, 128, 4, seed=77, bf16=True)
    T = {n: dev(x[n], torch.bfloat16) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], torch.bfloat16)
    runs = []
    for use_ws in (False, True):
        state, rk, rv, pos = prefill_handoff(*(T[n][:, :, :30].contiguous() for n in ("q", "k", "v", "g")),
                                             mk, None, 16, 1 / math.sqrt(128), 1.0)
        ws = decode_workspace(3, 4, 128, "cuda") if use_ws else None
        outs = [lizard_attn_decode_step(*(T[n][:, :, t].contiguous() for n in ("q", "k", "v", "g")), mk, None,
                                        state, rk, rv, pos, window=16, workspace=ws) for t in range(30, 40)]
        torch.cuda.synchronize()
        runs.append((torch.stack(outs), state.clone(), rk.clone(), rv.clone(), pos.clone()))
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtname,D", [("fp32", 64), ("bf16", 128)])
def test_decode_checkpoint_restore(dtname, D):
    """The decode carry (state, ring, pos) is the whole of a sequence's memory: copied out after
    some steps (a checkpoint, here through host memory) and copied into fresh buffers, it continues
    bit for bit like the uninterrupted run, for sequences at different positions."""
    B, H, W, M, pre, n1, n2 = 3, 2, 16, 4, 37, 9, 14
    x = make_small(B, H, pre + n1 + n2, D, M, seed=91, bf16=(dtname == "bf16"), with_grad=False)
    dt = tdtype(dtname)
    scale = 1.0 / math.sqrt(D)
    T = {n: dev(x[n], dt) for n in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], dt)
    state = torch.zeros(B, H, D, D, device="cuda", dtype=torch.float32)
    rk = torch.zeros(B, H, W, D, device="cuda", dtype=dt)
    rv = torch.zeros_like(rk)
    pos = torch.zeros(B, device="cuda", dtype=torch.int32)
    step = lambda t, st, a, b, p: lizard_attn_decode_step(*(T[n][:, :, t].contiguous() for n in "qkvg"), mk, None,
                                                          st, a, b, p, window=W, scale=scale)
    for t in range(pre + n1):
        step(t, state, rk, rv, pos)
    torch.cuda.synchronize()
    ckpt = [a.cpu() for a in (state, rk, rv, pos)]            # the checkpoint
    ref = [step(t, state, rk, rv, pos) for t in range(pre + n1, pre + n1 + n2)]
    torch.cuda.synchronize()
    s2, rk2, rv2, pos2 = (a.to("cuda") for a in ckpt)          # restored into fresh buffers
    got = [step(t, s2, rk2, rv2, pos2) for t in range(pre + n1, pre + n1 + n2)]
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    for a, b in zip((s2, rk2, rv2, pos2), (state, rk, rv, pos)):
        assert torch.equal(a, b)
    # and the continued run still matches the oracle's whole-sequence forward
    o = host(torch.stack(got, 2))
    r = orc.hybrid_forward(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=W, scale=scale)
    assert rel_l2(o, r["o"][:, :, pre + n1:]) <= TOL[dtname]


def test_decode_steps_captured_in_a_graph():
    """Decode steps captured once in a HIP graph (kernel nodes only) and replayed: every replay,
    from a restored carry and with host work and synchronisations between the replays, equals
    the eager steps bit for bit."""
    B, H, D, W, pre, n = 4, 4, 128, 32, 40, 6
    x = make_small(B, H, pre + n, D, 4, seed=123, bf16=True, with_grad=False)
    T = {k_: dev(x[k_], torch.bfloat16) for k_ in ("q", "k", "v")}
    T["g"] = dev(x["g"], torch.float32)
    mk = dev(x["meta_k"], torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    carry0 = prefill_handoff(*(T[c][:, :, :pre].contiguous() for c in "qkvg"), mk, None, W, scale, 1.0)
    tok = {c: T[c][:, :, pre:].permute(2, 0, 1, 3).contiguous() for c in "qkvg"}
    from gated_linear_attention_chunkwise_amd import decode_workspace
    ws = decode_workspace(B, H, D, "cuda")

    def run(carry, outs):
        st, a, b, p = carry
        for t in range(n):
            lizard_attn_decode_step(tok["q"][t], tok["k"][t], tok["v"][t], tok["g"][t], mk, None, st, a, b, p,
                                    window=W, scale=scale, out=outs[t], workspace=ws)

    eager = [torch.empty(B, H, D, device="cuda", dtype=torch.bfloat16) for _ in range(n)]
    c_e = tuple(a.clone() for a in carry0)
    run(c_e, eager)
    torch.cuda.synchronize()
    c_g = tuple(a.clone() for a in carry0)
    gout = [torch.empty_like(eager[0]) for _ in range(n)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run(c_g, gout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for a, b in zip(c_g, carry0):
            a.copy_(b)                       # restore the carry the graph starts from
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(n):
            assert torch.equal(gout[t], eager[t]), (rep, t)
        for a, b in zip(c_g, c_e):
            assert torch.equal(a, b), rep
        _ = float(gout[0].float().sum())     # eager work between the replays

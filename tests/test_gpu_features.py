"""GPU parity of the layer with GLA log features (lizard_attn_fwd_feat /
lizard_attn_bwd_feat) against the CPU oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import feature_map as fm
from gated_linear_attention_chunkwise_amd import lizard_attn_bwd_feat, lizard_attn_fwd_feat
from gated_linear_attention_chunkwise_amd.inputs import (WORKLOADS, make_inputs_device, make_log_features,
                                                          make_log_features_device, make_small)
from helpers import TOL, dev, host, rel_l2, tdtype

pytestmark = pytest.mark.gpu


def run_case(dtname, B, H, L, D, W, M, with_mv, seed):
    x = make_small(B, H, L, D, M, seed=seed, bf16=(dtname == "bf16"), with_meta_v=with_mv)
    x.update(make_log_features((B, H, L, D), seed=seed + 7))
    dt = tdtype(dtname)
    T = {n: dev(x[n], dt) for n in ("q", "k", "v", "dO")}
    for n in ("g", "lq", "lk"):
        T[n] = dev(x[n], torch.float32)
    mk = dev(x["meta_k"], dt) if M > 0 else None
    mv = dev(x["meta_v"], dt) if (with_mv and M > 0) else None
    scale, mix = 1.0 / math.sqrt(D), 0.7
    f = lizard_attn_fwd_feat(T["q"], T["k"], T["v"], T["lq"], T["lk"], T["g"], mk, mv, window=W, scale=scale,
                             mix=mix, want_lse=True, want_o_swa=True, want_chunk_states=True, want_state=True)
    b = lizard_attn_bwd_feat(T["q"], T["k"], T["v"], T["lq"], T["lk"], T["g"], mk, mv, T["dO"], f["lse"],
                             f["o_swa"], f["chunk_states"], window=W, scale=scale, mix=mix)
    torch.cuda.synchronize()
    mvr = x.get("meta_v") if (with_mv and M > 0) else None
    ref = fm.hybrid_forward_features(x["q"], x["k"], x["v"], x["lq"], x["lk"], x["g"], x["meta_k"], mvr, window=W,
                                     scale=scale, mix=mix)
    gr = fm.hybrid_backward_features(x["q"], x["k"], x["v"], x["lq"], x["lk"], x["g"], x["meta_k"], mvr, x["dO"],
                                     window=W, scale=scale, mix=mix)
    errs = {n: rel_l2(host(f[n]), ref[n]) for n in ("o", "o_swa", "state")}
    names = ["dq", "dk", "dv", "dlq", "dlk"] + (["dg"] if L > 1 else [])
    errs.update({n: rel_l2(host(b[n]), gr[n]) for n in names})
    if L == 1:   # the first token's gate multiplies the zero initial state
        assert float(b["dg"].abs().max()) == 0.0
    if M > 0:
        errs["dmeta_k"] = rel_l2(host(b["dmeta_k"]), gr["dmeta_k"])
    if mvr is not None:
        errs["dmeta_v"] = rel_l2(host(b["dmeta_v"]), gr["dmeta_v"])
    print(dtname, B, H, L, D, W, M, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtname], (n, e)


CASES = [("fp32", 1, 2, 256, 64, 64, 4, True), ("fp32", 2, 1, 130, 64, 5, 0, False),
         ("bf16", 2, 2, 200, 128, 128, 4, False), ("bf16", 1, 2, 65, 64, 129, 16, True),
         ("bf16", 1, 1, 1, 128, 1, 0, False), ("bf16", 1, 3, 1000, 128, 100, 2, False),
         ("bf16", 1, 1, 2100, 128, 128, 4, False)]   # long, one head: the sweeps run in segments


@pytest.mark.parametrize("dtname,B,H,L,D,W,M,with_mv", CASES)
def test_features_parity(dtname, B, H, L, D, W, M, with_mv):
    run_case(dtname, B, H, L, D, W, M, with_mv, seed=L + D + W)


def test_features_train_shape_sampled_head():
    """B=4, H=32, L=8192, d=128 with log features: every output of one sampled head."""
    w = WORKLOADS["train_8k"]
    x = make_inputs_device(w, "cuda", with_grad=True)
    x.update(make_log_features_device((w.B, w.H, w.L, w.D), seed=99, device="cuda"))
    f = lizard_attn_fwd_feat(x["q"], x["k"], x["v"], x["lq"], x["lk"], x["g"], x["meta_k"], None, window=w.W,
                             scale=w.scale, want_lse=True, want_o_swa=True, want_chunk_states=True)
    b = lizard_attn_bwd_feat(x["q"], x["k"], x["v"], x["lq"], x["lk"], x["g"], x["meta_k"], None, x["dO"],
                             f["lse"], f["o_swa"], f["chunk_states"], window=w.W, scale=w.scale)
    torch.cuda.synchronize()
    bb, h = 1, 21
    hs = {n: x[n][bb:bb + 1, h:h + 1].float().cpu().numpy() for n in ("q", "k", "v", "g", "lq", "lk", "dO")}
    mk = x["meta_k"][h:h + 1].float().cpu().numpy()
    ref = fm.hybrid_forward_features(hs["q"], hs["k"], hs["v"], hs["lq"], hs["lk"], hs["g"], mk, None, window=w.W,
                                     scale=w.scale)
    gr = fm.hybrid_backward_features(hs["q"], hs["k"], hs["v"], hs["lq"], hs["lk"], hs["g"], mk, None, hs["dO"],
                                     window=w.W, scale=w.scale)
    errs = {"o": rel_l2(host(f["o"][bb:bb + 1, h:h + 1]), ref["o"])}
    errs.update({n: rel_l2(host(b[n][bb:bb + 1, h:h + 1]), gr[n]) for n in ("dq", "dk", "dv", "dlq", "dlk", "dg")})
    print("train shape features head", h, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


def test_features_prefill_continue_decode():
    """Log-feature prefill (state hand-off) -> two continued segments -> decode steps, against
    the oracle's whole-sequence log-feature forward."""
    from gated_linear_attention_chunkwise_amd import lizard_attn_decode_step_feat, lizard_attn_fwd_continue_feat
    B, H, N, D, W, M, P = 2, 2, 300, 128, 128, 4, 100
    x = make_small(B, H, N, D, M, seed=41, bf16=True)
    x.update(make_log_features((B, H, N, D), seed=42))
    bf = torch.bfloat16
    T = {n: dev(x[n], bf) for n in ("q", "k", "v", "meta_k")}
    for n in ("g", "lq", "lk"):
        T[n] = dev(x[n], torch.float32)
    scale = 1.0 / math.sqrt(D)
    seg = lambda n, a, e: T[n][:, :, a:e].contiguous()
    f = lizard_attn_fwd_feat(*(seg(n, 0, P) for n in ("q", "k", "v", "lq", "lk", "g")), T["meta_k"], None, window=W,
                             scale=scale, want_state=True)
    outs = [f["o"]]
    state = f["state"]
    ring_k = torch.zeros(B, H, W, D, device="cuda", dtype=bf)
    ring_v = torch.zeros_like(ring_k)
    ts = torch.arange(max(0, P - W), P, device="cuda")
    ring_k[:, :, ts % W] = T["k"][:, :, ts]
    ring_v[:, :, ts % W] = T["v"][:, :, ts]
    pos = torch.full((B,), P, device="cuda", dtype=torch.int32)
    for a, e in ((P, 180), (180, 250)):
        outs.append(lizard_attn_fwd_continue_feat(*(seg(n, a, e) for n in ("q", "k", "v", "lq", "lk", "g")),
                                                  T["meta_k"], None, state, ring_k, ring_v, pos, window=W,
                                                  scale=scale))
    for t in range(250, N):
        outs.append(lizard_attn_decode_step_feat(*(T[n][:, :, t].contiguous() for n in ("q", "k", "v", "lq", "lk", "g")),
                                                 T["meta_k"], None, state, ring_k, ring_v, pos, window=W,
                                                 scale=scale).unsqueeze(2))
    torch.cuda.synchronize()
    ref = fm.hybrid_forward_features(x["q"], x["k"], x["v"], x["lq"], x["lk"], x["g"], x["meta_k"], None, window=W,
                                     scale=scale)
    e_o = rel_l2(host(torch.cat(outs, 2)), ref["o"])
    e_s = rel_l2(host(state), ref["state"])
    print(f"feature carry: o {e_o:.2e} state {e_s:.2e}; pos {pos.tolist()}", flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"] and pos.tolist() == [N] * B

"""GPU parity of the Hedgehog log-feature map (lizard_hedgehog_fwd / _bwd)
against the CPU oracle, alone and chained into the layer's log-feature calls."""
import math

import numpy as np
import pytest
import torch

from oracle import feature_map as fm
from gated_linear_attention_chunkwise_amd import (lizard_attn_bwd_feat, lizard_attn_fwd_feat, lizard_hedgehog_bwd,
                                                  lizard_hedgehog_fwd)
from gated_linear_attention_chunkwise_amd.inputs import make_small, round_to_bf16
from helpers import TOL, dev, host, rel_l2, tdtype

pytestmark = pytest.mark.gpu


def weights(H, D, seed, bf16):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((H, D, D // 2)) * 8.0 / math.sqrt(D)).astype(np.float32)   # q, k ~ N(0,1)/8
    return round_to_bf16(w) if bf16 else w


CASES = [("fp32", 1, 2, 256, 64), ("fp32", 2, 1, 77, 64), ("bf16", 2, 2, 300, 128), ("bf16", 1, 3, 1, 128),
         ("bf16", 3, 2, 129, 64), ("bf16", 1, 2, 2000, 128)]


@pytest.mark.parametrize("dtname,B,H,L,D", CASES)
def test_hedgehog_parity(dtname, B, H, L, D):
    bf = dtname == "bf16"
    x = make_small(B, H, L, D, 0, seed=L + D, bf16=bf)
    w = weights(H, D, L, bf)
    dl = np.random.default_rng(L).standard_normal((B, H, L, D)).astype(np.float32)
    dt = tdtype(dtname)
    X, Wt = dev(x["q"], dt), dev(w, dt)
    lphi = lizard_hedgehog_fwd(X, Wt)
    dx, dw = lizard_hedgehog_bwd(X, Wt, dev(dl, torch.float32))
    torch.cuda.synchronize()
    ref = fm.hedgehog_log_features(x["q"], w)
    rdx, rdw = fm.hedgehog_log_features_backward(x["q"], w, dl)
    errs = {"lphi": rel_l2(host(lphi), ref), "dx": rel_l2(host(dx), rdx), "dw": rel_l2(host(dw), rdw)}
    print(dtname, B, H, L, D, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtname], (n, e)


def test_hedgehog_then_layer():
    """q, k -> log features -> layer (GLA on the features, window on q, k) -> backward -> feature
    map backward: gradients of q, k and of both maps' weights against the oracle's chain."""
    B, H, L, D, W, M = 2, 2, 200, 128, 128, 4
    x = make_small(B, H, L, D, M, seed=5, bf16=True)
    wq, wk = weights(H, D, 1, True), weights(H, D, 2, True)
    bf = torch.bfloat16
    T = {n: dev(x[n], bf) for n in ("q", "k", "v", "meta_k", "dO")}
    T["g"] = dev(x["g"], torch.float32)
    Wq, Wk = dev(wq, bf), dev(wk, bf)
    scale = 1.0 / math.sqrt(D)
    lq, lk = lizard_hedgehog_fwd(T["q"], Wq), lizard_hedgehog_fwd(T["k"], Wk)
    f = lizard_attn_fwd_feat(T["q"], T["k"], T["v"], lq, lk, T["g"], T["meta_k"], None, window=W, scale=scale,
                             want_lse=True, want_o_swa=True, want_chunk_states=True)
    b = lizard_attn_bwd_feat(T["q"], T["k"], T["v"], lq, lk, T["g"], T["meta_k"], None, T["dO"], f["lse"],
                             f["o_swa"], f["chunk_states"], window=W, scale=scale)
    dxq, dwq = lizard_hedgehog_bwd(T["q"], Wq, b["dlq"])
    dxk, dwk = lizard_hedgehog_bwd(T["k"], Wk, b["dlk"])
    torch.cuda.synchronize()
    rlq, rlk = fm.hedgehog_log_features(x["q"], wq), fm.hedgehog_log_features(x["k"], wk)
    ref = fm.hybrid_forward_features(x["q"], x["k"], x["v"], rlq, rlk, x["g"], x["meta_k"], None, window=W,
                                     scale=scale)
    gr = fm.hybrid_backward_features(x["q"], x["k"], x["v"], rlq, rlk, x["g"], x["meta_k"], None, x["dO"],
                                     window=W, scale=scale)
    rdxq, rdwq = fm.hedgehog_log_features_backward(x["q"], wq, gr["dlq"])
    rdxk, rdwk = fm.hedgehog_log_features_backward(x["k"], wk, gr["dlk"])
    errs = {"o": rel_l2(host(f["o"]), ref["o"]),
            "dq": rel_l2(host(b["dq"]) + host(dxq), gr["dq"] + rdxq),
            "dk": rel_l2(host(b["dk"]) + host(dxk), gr["dk"] + rdxk),
            "dWq": rel_l2(host(dwq), rdwq), "dWk": rel_l2(host(dwk), rdwk),
            "dv": rel_l2(host(b["dv"]), gr["dv"]), "dg": rel_l2(host(b["dg"]), gr["dg"])}
    print("chain", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)

"""GPU parity of the gate projection g = log sigmoid(x W^T)/tau (forward and
backward) against the CPU oracle, on its own and chained into the layer."""
import math

import numpy as np
import pytest
import torch

from oracle import gate_projection as gpo
from oracle import lizard_oracle as orc
from gated_linear_attention_chunkwise_amd import (lizard_attn_bwd, lizard_attn_fwd, lizard_gate_proj_bwd,
                                                  lizard_gate_proj_fwd)
from gated_linear_attention_chunkwise_amd.inputs import make_gate_device, make_gate_small, make_small
from helpers import TOL, dev, host, rel_l2, tdtype

pytestmark = pytest.mark.gpu


def run_case(dtname, B, L, H, dk, Dm, tau, scalar, seed):
    ng = H if scalar else H * dk
    gshape = (B, H, L) if scalar else (B, H, L, dk)
    x = make_gate_small(B, L, Dm, ng, gshape, seed=seed, bf16=(dtname == "bf16"))
    dt = tdtype(dtname)
    X, Wt, dG = dev(x["x"], dt), dev(x["w"], dt), dev(x["dg"], torch.float32)
    g = lizard_gate_proj_fwd(X, Wt, heads=H, d_k=dk, tau=tau, scalar=scalar)
    dx, dw = lizard_gate_proj_bwd(X, Wt, g, dG, heads=H, d_k=dk, tau=tau, scalar=scalar)
    torch.cuda.synchronize()
    ref_g = gpo.gate_projection(x["x"], x["w"], H, tau=tau, scalar=scalar)
    ref_dx, ref_dw = gpo.gate_projection_backward(x["x"], x["w"], H, x["dg"], tau=tau, scalar=scalar)
    assert g.shape == ref_g.shape and dx.shape == ref_dx.shape and dw.shape == ref_dw.shape
    errs = {"g": rel_l2(host(g), ref_g), "dx": rel_l2(host(dx), ref_dx), "dw": rel_l2(host(dw), ref_dw)}
    print(dtname, B, L, H, dk, Dm, tau, "scalar" if scalar else "per-dim",
          {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtname], (n, e)


# (dtype, B, L, H, d_k, d_model, tau): several tiles in every direction with ragged tails
CASES = [("fp32", 1, 256, 2, 64, 128, 16.0), ("fp32", 2, 77, 3, 64, 96, 1.0),
         ("bf16", 2, 300, 4, 64, 320, 16.0), ("bf16", 1, 130, 2, 128, 256, 1.0),
         ("bf16", 3, 1, 2, 64, 32, 4.0), ("bf16", 1, 1000, 1, 128, 544, 16.0)]


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("dtname,B,L,H,dk,Dm,tau", CASES)
def test_gate_projection_parity(dtname, B, L, H, dk, Dm, tau, scalar):
    run_case(dtname, B, L, H, dk, Dm, tau, scalar, seed=B * 1000 + L + Dm)


def test_gate_projection_empty_sequence():
    x = torch.zeros(2, 0, 64, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(2 * 64, 64, device="cuda").to(torch.bfloat16)
    g = lizard_gate_proj_fwd(x, w, heads=2, d_k=64, tau=16.0)
    assert g.shape == (2, 2, 0, 64)
    dx, dw = lizard_gate_proj_bwd(x, w, g, torch.zeros_like(g), heads=2, d_k=64, tau=16.0)
    torch.cuda.synchronize()
    assert dx.shape == x.shape and float(dw.abs().max()) == 0.0


def test_gate_projection_repeated_calls_reuse_workspace():
    """dw partial sums live in the workspace: a second call on a smaller input must not see the first."""
    from gated_linear_attention_chunkwise_amd import gate_proj_workspace
    H, dk, Dm = 2, 64, 128
    ws = gate_proj_workspace((2, 512, Dm), H, dk, torch.bfloat16, "cuda")
    for L in (512, 200):
        x = make_gate_small(2, L, Dm, H * dk, (2, H, L, dk), seed=L, bf16=True)
        X, Wt, dG = dev(x["x"], torch.bfloat16), dev(x["w"], torch.bfloat16), dev(x["dg"], torch.float32)
        g = lizard_gate_proj_fwd(X, Wt, heads=H, d_k=dk, tau=16.0)
        dx, dw = lizard_gate_proj_bwd(X, Wt, g, dG, heads=H, d_k=dk, tau=16.0, workspace=ws)
        torch.cuda.synchronize()
        _, ref_dw = gpo.gate_projection_backward(x["x"], x["w"], H, x["dg"], tau=16.0)
        assert rel_l2(host(dw), ref_dw) <= TOL["bf16"], L


@pytest.mark.parametrize("scalar", [False, True])
def test_gate_projection_into_the_layer(scalar):
    """x -> gate projection -> hybrid layer forward/backward -> gradients of x and W through
    the gate, against the oracle's same chain."""
    B, H, L, D, Dm, M, W, tau = 2, 2, 200, 64, 128, 4, 64, 16.0
    ng = H if scalar else H * D
    gshape = (B, H, L) if scalar else (B, H, L, D)
    gx = make_gate_small(B, L, Dm, ng, gshape, seed=31, bf16=True)
    lx = make_small(B, H, L, D, M, seed=32, bf16=True)
    bf = torch.bfloat16
    X, Wt = dev(gx["x"], bf), dev(gx["w"], bf)
    T = {n: dev(lx[n], bf) for n in ("q", "k", "v", "meta_k", "dO")}
    scale = 1.0 / math.sqrt(D)
    g = lizard_gate_proj_fwd(X, Wt, heads=H, d_k=D, tau=tau, scalar=scalar)
    f = lizard_attn_fwd(T["q"], T["k"], T["v"], g, T["meta_k"], None, window=W, scale=scale, want_lse=True,
                        want_o_swa=True, want_chunk_states=True)
    b = lizard_attn_bwd(T["q"], T["k"], T["v"], g, T["meta_k"], None, T["dO"], f["lse"], f["o_swa"],
                        f["chunk_states"], window=W, scale=scale)
    dx, dw = lizard_gate_proj_bwd(X, Wt, g, b["dg"], heads=H, d_k=D, tau=tau, scalar=scalar)
    torch.cuda.synchronize()

    ref_g = gpo.gate_projection(gx["x"], gx["w"], H, tau=tau, scalar=scalar)
    ref = orc.hybrid_forward(lx["q"], lx["k"], lx["v"], ref_g, lx["meta_k"], None, window=W, scale=scale)
    gr = orc.hybrid_backward(lx["q"], lx["k"], lx["v"], ref_g, lx["meta_k"], None, lx["dO"], window=W,
                             scale=scale)
    ref_dx, ref_dw = gpo.gate_projection_backward(gx["x"], gx["w"], H, gr["dg"], tau=tau, scalar=scalar)
    errs = {"o": rel_l2(host(f["o"]), ref["o"]), "dg": rel_l2(host(b["dg"]), gr["dg"]),
            "dx": rel_l2(host(dx), ref_dx), "dw": rel_l2(host(dw), ref_dw)}
    print("chain", "scalar" if scalar else "per-dim", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)


@pytest.mark.parametrize("scalar", [False, True])
def test_gate_projection_train_shape_sampled(scalar):
    """B=4, L=8192, d_model=4096, H=32, d_k=128 (Ng = 4096 or 32), tau = 16: g and dx on
    sampled tokens and dw on sampled rows, each computed by the oracle from the inputs alone."""
    B, L, Dm, H, dk, tau = 4, 8192, 4096, 32, 128, 16.0
    ng = H if scalar else H * dk
    gshape = (B, H, L) if scalar else (B, H, L, dk)
    t = make_gate_device(B, L, Dm, ng, gshape, seed=2024, device="cuda", dtype=torch.bfloat16)
    g = lizard_gate_proj_fwd(t["x"], t["w"], heads=H, d_k=dk, tau=tau, scalar=scalar)
    dx, dw = lizard_gate_proj_bwd(t["x"], t["w"], g, t["dg"], heads=H, d_k=dk, tau=tau, scalar=scalar)
    torch.cuda.synchronize()
    xs = host(t["x"])                          # [B, L, Dm] as float64
    ws = host(t["w"])
    dgs = t["dg"].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    toks = [(int(b), int(s)) for b, s in zip(rng.integers(0, B, 12), rng.integers(0, L, 12))] + [(B - 1, L - 1)]
    gh = host(g)
    dxh = host(dx)
    eg, edx = [], []
    for b, s in toks:
        xb = xs[b:b + 1, s:s + 1]              # one token, [1, 1, Dm]
        dgt = dgs[b:b + 1, :, s:s + 1]
        rg = gpo.gate_projection(xb, ws, H, tau=tau, scalar=scalar)
        rdx, _ = gpo.gate_projection_backward(xb, ws, H, dgt, tau=tau, scalar=scalar)
        eg.append(rel_l2(gh[b:b + 1, :, s:s + 1], rg))
        edx.append(rel_l2(dxh[b, s], rdx[0, 0]))
    # rows of dw: the full contraction over all B*L tokens for a few gate rows
    dwh = host(dw)
    edw = []
    for n in rng.choice(ng, 3, replace=False):
        # gate row n alone is a one-head scalar gate: the oracle's backward gives its dw row
        dgn = dgs[:, n] if scalar else dgs[:, n // dk, :, n % dk]
        _, ref_row = gpo.gate_projection_backward(xs, ws[n:n + 1], 1, dgn[:, None, :], tau=tau, scalar=True)
        edw.append(rel_l2(dwh[n], ref_row[0]))
    print("train shape", "scalar" if scalar else "per-dim", f"g {max(eg):.2e} dx {max(edx):.2e} dw {max(edw):.2e}",
          flush=True)
    assert max(eg) <= TOL["bf16"] and max(edx) <= TOL["bf16"] and max(edw) <= TOL["bf16"]

"""lizard_attn_decode_step_noalloc (no workspace argument; the step needs no device memory beyond
its arguments) against lizard_attn_decode_step, through the C ABI: two runs in a row on one
device, the second on a smaller batch, each bit for bit equal to the plain step and within the
bf16 bound of the oracle's whole-sequence forward."""
import ctypes
import math

import numpy as np
import pytest
import torch

from oracle import lizard_oracle as orc
from gated_linear_attention_chunkwise_amd import _lib, lizard_attn_fwd
from gated_linear_attention_chunkwise_amd.inputs import make_small
from helpers import TOL, dev, host, rel_l2

pytestmark = pytest.mark.gpu


def carry(x, pre, W, scale):
    """Prefill hand-off: final state of a forward over the prefix, its last W keys/values in
    ring slots t mod W, pos = pre."""
    T = {n: dev(x[n][:, :, :pre], torch.bfloat16) for n in ("q", "k", "v")}
    g = dev(x["g"][:, :, :pre], torch.float32)
    mk = dev(x["meta_k"], torch.bfloat16)
    f = lizard_attn_fwd(T["q"], T["k"], T["v"], g, mk, None, window=W, scale=scale, want_state=True)
    B, H, _, D = x["q"].shape
    rk = torch.zeros(B, H, W, D, device="cuda", dtype=torch.bfloat16)
    rv = torch.zeros_like(rk)
    ts = torch.arange(max(0, pre - W), pre, device="cuda")
    rk[:, :, ts % W] = T["k"][:, :, ts]
    rv[:, :, ts % W] = T["v"][:, :, ts]
    return f["state"], rk, rv, torch.full((B,), pre, device="cuda", dtype=torch.int32)


def run_case(B, H, D, W, pre, steps, seed):
    lib = _lib.load()
    x = make_small(B, H, pre + steps, D, 4, seed=seed, bf16=True, with_grad=False)
    scale = 1.0 / math.sqrt(D)
    mk = dev(x["meta_k"], torch.bfloat16)
    s = _lib.make_shape(B, H, 0, D, W, 4, scale, 1.0, torch.bfloat16)
    ws = _lib.decode_workspace(B, H, D, "cuda")
    c_plain = carry(x, pre, W, scale)
    c_noalloc = tuple(a.clone() for a in c_plain)
    outs = {}
    for name, (state, rk, rv, pos) in (("plain", c_plain), ("noalloc", c_noalloc)):
        o_all = torch.empty(steps, B, H, D, device="cuda", dtype=torch.bfloat16)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i, t in enumerate(range(pre, pre + steps)):
            q, k, v = (dev(np.ascontiguousarray(x[n][:, :, t]), torch.bfloat16) for n in ("q", "k", "v"))
            g = dev(np.ascontiguousarray(x["g"][:, :, t]), torch.float32)
            P = lambda a: ctypes.c_void_p(a.data_ptr())
            if name == "plain":
                rc = lib.lizard_attn_decode_step(ctypes.byref(s), P(q), P(k), P(v), P(g), P(mk), None, P(state),
                                                 P(rk), P(rv), P(pos), P(o_all[i]), P(ws), ws.numel(), stream)
            else:
                rc = lib.lizard_attn_decode_step_noalloc(ctypes.byref(s), P(q), P(k), P(v), P(g), P(mk), None,
                                                         P(state), P(rk), P(rv), P(pos), P(o_all[i]), stream)
            assert rc == 0, (name, rc)
        torch.cuda.synchronize()
        outs[name] = (o_all, state, rk, rv, pos)
    for a, b in zip(outs["plain"], outs["noalloc"]):
        assert torch.equal(a, b)
    ref = orc.hybrid_forward(x["q"], x["k"], x["v"], x["g"], x["meta_k"], None, window=W, scale=scale)
    o = host(outs["noalloc"][0]).transpose(1, 2, 0, 3)
    e = rel_l2(o, ref["o"][:, :, pre:])
    print(B, H, D, f"noalloc vs oracle {e:.2e}", flush=True)
    assert e <= TOL["bf16"]


def test_noalloc_decode_two_calls_second_smaller():
    run_case(B=8, H=8, D=128, W=32, pre=70, steps=12, seed=3)
    run_case(B=2, H=3, D=128, W=32, pre=45, steps=9, seed=4)

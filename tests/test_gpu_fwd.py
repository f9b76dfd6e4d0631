"""GPU parity of lizard_attn_fwd against the CPU oracle (relative L2 per tensor)."""
import math

import numpy as np
import pytest
import torch

from oracle import lizard_oracle as orc
from gated_linear_attention_chunkwise_amd import lizard_attn_fwd
from gated_linear_attention_chunkwise_amd.inputs import WORKLOADS, make_inputs, make_small
from helpers import TOL, dev, host, rel_l2, tdtype

pytestmark = pytest.mark.gpu


def run_fwd(x, dtname, W, mix=1.0, scale=None):
    dt = tdtype(dtname)
    D = x["q"].shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    mv = x.get("meta_v")
    out = lizard_attn_fwd(dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt),
                          dev(x["g"], torch.float32),
                          dev(x["meta_k"], dt) if x["meta_k"].shape[1] > 0 else None,
                          None if mv is None else dev(mv, dt),
                          window=W, scale=scale, mix=mix, want_lse=True, want_o_swa=True,
                          want_chunk_states=True, want_state=True)
    torch.cuda.synchronize()
    ref = orc.hybrid_forward(x["q"], x["k"], x["v"], x["g"], x["meta_k"], mv, window=W,
                             scale=scale, mix=mix)
    return out, ref


def check(out, ref, dtname, what=("o", "o_swa", "lse", "state")):
    tol = TOL[dtname]
    errs = {}
    for n in what:
        errs[n] = rel_l2(host(out[n]), ref[n])
    print("rel_l2", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return errs


def test_tiny_fp32_workload():
    w = WORKLOADS["tiny_fp32"]
    x = make_inputs(w)
    out, ref = run_fwd(x, "fp32", w.W)
    check(out, ref, "fp32")
    # states entering each chunk (row-major [d_k][d_v]), saved for the backward pass
    _, _, states = orc.gla_forward(x["q"], x["k"], x["v"], x["g"], return_states=True)
    cs = host(out["chunk_states"])
    assert np.abs(cs[:, :, 0]).max() == 0.0
    for c in range(1, cs.shape[2]):
        assert rel_l2(cs[:, :, c], states[64 * c - 1]) <= 1e-5, c


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
def test_bf16_d128_ragged(L):
    x = make_small(2, 3, L, 128, 4, seed=100 + L, bf16=True, with_grad=False)
    out, ref = run_fwd(x, "bf16", 128)
    check(out, ref, "bf16")


@pytest.mark.parametrize("W,M,with_mv,mix", [(1, 0, False, 1.0), (5, 1, False, 0.5), (64, 16, True, 1.0),
                                             (65, 4, True, 2.0), (129, 3, False, 1.0), (100, 0, False, 1.0),
                                             # windows beyond three chunks, and past the sequence's end
                                             (130, 2, False, 1.0), (190, 4, True, 1.0), (1000, 1, False, 0.5)])
@pytest.mark.parametrize("dtname", ["fp32", "bf16"])
def test_window_and_meta_edge_cases(W, M, with_mv, mix, dtname):
    x = make_small(1, 2, 190, 64, M, seed=7 * W + M, bf16=(dtname == "bf16"), with_grad=False,
                   with_meta_v=with_mv)
    out, ref = run_fwd(x, dtname, W, mix=mix)
    check(out, ref, dtname)


@pytest.mark.parametrize("dtname,D", [("fp32", 64), ("bf16", 128)])
def test_long_window(dtname, D):
    """A window of up to six chunks of keys (W = 300 over L = 700)."""
    x = make_small(2, 2, 700, D, 4, seed=300 + D, bf16=(dtname == "bf16"), with_grad=False, with_meta_v=True)
    out, ref = run_fwd(x, dtname, 300)
    check(out, ref, dtname)


def test_strong_gates_stay_in_range():
    # gates 8x stronger than the workloads (chunk-local sums near -36): still exact in fp32
    x = make_small(1, 2, 256, 64, 4, seed=5, bf16=False, with_grad=False, gate_div=2.0)
    out, ref = run_fwd(x, "fp32", 64)
    check(out, ref, "fp32")


def test_empty_sequence_is_noop():
    x = make_small(1, 2, 0, 64, 4, seed=1, bf16=False, with_grad=False)
    out, _ = run_fwd(x, "fp32", 64)
    assert out["o"].numel() == 0
    assert float(out["state"].abs().max()) == 0.0


@pytest.mark.parametrize("dtname,D,L", [("fp32", 64, 2085), ("bf16", 64, 4101), ("bf16", 128, 2048)])
def test_segmented_state_sweep(dtname, D, L):
    """Few heads and a long sequence: the state sweep runs in sequence segments (a
    reduce pass per segment, a scan over segments, then the sweep of every segment from
    its entering state).  Outputs, the final state and every chunk state match the oracle."""
    x = make_small(1, 2, L, D, 4, seed=L + D, bf16=(dtname == "bf16"), with_grad=False)
    out, ref = run_fwd(x, dtname, 128 if D == 128 else 64)
    check(out, ref, dtname)
    _, _, states = orc.gla_forward(x["q"], x["k"], x["v"], x["g"], return_states=True)
    cs = host(out["chunk_states"])
    assert np.abs(cs[:, :, 0]).max() == 0.0
    for c in range(1, cs.shape[2]):
        assert rel_l2(cs[:, :, c], states[64 * c - 1]) <= TOL[dtname], c


def _sampled(name, heads):
    w = WORKLOADS[name]
    x = make_inputs(w)
    out = lizard_attn_fwd(dev(x["q"], torch.bfloat16), dev(x["k"], torch.bfloat16),
                          dev(x["v"], torch.bfloat16), dev(x["g"], torch.float32),
                          dev(x["meta_k"], torch.bfloat16), None, window=w.W, scale=w.scale,
                          want_lse=True, want_state=True)
    torch.cuda.synchronize()
    for (b, h) in heads:
        sl = lambda a: a[b:b + 1, h:h + 1]
        ref = orc.hybrid_forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]),
                                 x["meta_k"][h:h + 1], None, window=w.W, scale=w.scale)
        errs = {n: rel_l2(host(out[n][b:b + 1, h:h + 1]), ref[n]) for n in ("o", "lse", "state")}
        print(name, (b, h), {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        for n, e in errs.items():
            assert e <= TOL["bf16"], (name, b, h, n, e)


def test_fwd_4k_full_size_sampled_heads():
    _sampled("fwd_4k", [(0, 0), (0, 31)])


def test_prefill_64k_full_size_sampled_heads():
    _sampled("prefill_64k", [(0, 0), (0, 31)])

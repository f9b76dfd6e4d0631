"""The library keeps no mutable global state: calls from two host threads, each on its own stream,
overlap and still give, bit for bit, what the same calls give one after another (the kernels are
deterministic, so any shared scratch, flag or attribute race would show as a difference)."""
import math
import threading

import pytest
import torch

from gated_linear_attention_chunkwise_amd import lizard_attn_bwd, lizard_attn_fwd
from gated_linear_attention_chunkwise_amd.inputs import make_small

pytestmark = pytest.mark.gpu

REPS = 4


def _inputs(seed, D, L):
    x = make_small(2, 4, L, D, 4, seed=seed, bf16=True, with_meta_v=True)
    T = {n: torch.from_numpy(x[n]).cuda().to(torch.bfloat16) for n in ("q", "k", "v", "dO", "meta_k", "meta_v")}
    T["g"] = torch.from_numpy(x["g"]).cuda()
    return T


def _step(T, chunk):
    D = T["q"].shape[-1]
    kw = dict(window=96, scale=1.0 / math.sqrt(D), chunk=chunk)
    f = lizard_attn_fwd(T["q"], T["k"], T["v"], T["g"], T["meta_k"], T["meta_v"], want_lse=True, want_o_swa=True,
                        want_chunk_states=True, want_state=True, **kw)
    b = lizard_attn_bwd(T["q"], T["k"], T["v"], T["g"], T["meta_k"], T["meta_v"], T["dO"], f["lse"], f["o_swa"],
                        f["chunk_states"], **kw)
    return {**{n: f[n] for n in ("o", "lse", "state")}, **b}


@pytest.mark.parametrize("chunk", [64, 32])   # the fast kernels; the general path
def test_two_threads_two_streams_match_serial(chunk):
    xs = [_inputs(11, 128, 300), _inputs(12, 64, 257)]
    ref = [_step(x, chunk) for x in xs]
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [_step(xs[i], chunk) for _ in range(REPS)]
            s.synchronize()
            got[i] = outs
        except Exception as e:   # reported from the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i in range(2):
        assert got[i] is not None
        for rep, out in enumerate(got[i]):
            for n, r in ref[i].items():
                if r is None:
                    continue
                assert torch.equal(out[n], r), (i, rep, n)

"""Seeded synthetic inputs for the Lizard hybrid attention layer.

This module draws random tensors and nothing else: it holds none of the
layer's arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it without sharing any of the method's code.

Workloads (all synthetic; the explainer pages measure speed on no named
workload and print no shapes):

* ``tiny_fp32``   B=1  H=2  L=256   d=64  W=64  M=4, everything fp32
* ``fwd_4k``      B=1  H=32 L=4096  d=128 W=128 M=4, bf16 activations
* ``train_8k``    B=4  H=32 L=8192  d=128 W=128 M=4, bf16, with dO ~ N(0,1)
* ``prefill_64k`` B=1  H=32 L=65536 d=128 W=128 M=4, bf16, gate input x ~ N(2,1)
* ``decode_b64``  B=64 H=32 d=128 W=128 M=4, a 4096-token prefill followed by
  1024 single-token decode steps, drawn up front as one 5120-token sequence

Recipe (numpy ``default_rng(seed)``, draw order q, k, v, x, meta_k, dO):

* q, k, v ~ N(0, 1) / 8
* x ~ N(mu, 1) with mu = 0 (mu = 2 for ``prefill_64k``); the log-gate is
  g = logsigmoid(x) / 16, evaluated in fp64 and stored as fp32, per key dim
* meta_k ~ N(0, 1) / 8, shape [H, M, d_k]; meta values are absent (zero)
* dO ~ N(0, 1)

For bf16 workloads q, k, v, meta_k and dO are rounded to bf16 (round to
nearest even) and handed out as float32 arrays that hold exactly those bf16
values, so the oracle sees the very numbers the GPU sees; g stays fp32.

Gate-projection inputs (``make_gate_small`` / ``make_gate_device``, draw order
x, w, dg): the layer input x ~ N(0, 1) [B, L, d_model]; the gate weight
w ~ N(0, 1) / sqrt(d_model) [Ng, d_model], so that every pre-activation is
about N(0, 1) like the gate input of the recipe above; dg ~ N(0, 1) in the
gate layout.  The train-shaped case is d_model = 4096 (the 8B-shaped layer
with H = 32 heads of d = 128): Ng = 4096 per key dimension, 32 scalar.

Log features for the GLA branch (``make_log_features``): lq, lk ~
N(-log(d/2), 0.5^2) fp32, the spread of a softmax over d/2 features.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    D: int
    W: int
    M: int
    chunk: int
    dtype: str          # "fp32" or "bf16": dtype of q, k, v, o, meta, dO and grads
    x_mean: float
    seed: int
    prefill: int = 0    # decode workloads: tokens consumed by the prefill

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 256, 64, 64, 4, 64, "fp32", 0.0, 1000),
    "fwd_4k": Workload("fwd_4k", 1, 32, 4096, 128, 128, 4, 64, "bf16", 0.0, 1001),
    "train_8k": Workload("train_8k", 4, 32, 8192, 128, 128, 4, 64, "bf16", 0.0, 1002),
    "prefill_64k": Workload("prefill_64k", 1, 32, 65536, 128, 128, 4, 64, "bf16", 2.0, 1003),
    "decode_b64": Workload("decode_b64", 64, 32, 5120, 128, 128, 4, 64, "bf16", 0.0, 1004,
                           prefill=4096),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    # log(1 / (1 + e^-x)), evaluated without overflow for either sign of x
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def make_inputs(w: Workload, *, with_grad: bool = False, L: int | None = None) -> dict:
    """Draw the seeded inputs of workload ``w`` (optionally a shorter ``L``).

    Returns a dict of float32 numpy arrays: q, k, v [B,H,L,D], g [B,H,L,D],
    meta_k [H,M,D] and, with ``with_grad``, dO [B,H,L,D].
    """
    L = w.L if L is None else L
    rng = np.random.default_rng(w.seed)
    shp = (w.B, w.H, L, w.D)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = (rng.standard_normal(shp, dtype=np.float64) / 8.0).astype(np.float32)
    x = rng.standard_normal(shp, dtype=np.float64) + w.x_mean
    out["g"] = (_logsigmoid(x) / 16.0).astype(np.float32)
    del x
    out["meta_k"] = (rng.standard_normal((w.H, w.M, w.D), dtype=np.float64) / 8.0).astype(np.float32)
    if with_grad:
        out["dO"] = rng.standard_normal(shp, dtype=np.float64).astype(np.float32)
    if w.dtype == "bf16":
        for name in ("q", "k", "v", "meta_k", "dO"):
            if name in out:
                out[name] = round_to_bf16(out[name])
    return out


def make_small(B: int, H: int, L: int, D: int, M: int, *, seed: int, bf16: bool,
               x_mean: float = 0.0, gate_div: float = 16.0, with_grad: bool = True,
               Dv: int | None = None, with_meta_v: bool = False) -> dict:
    """Same recipe at arbitrary small sizes (parity and edge-case tests)."""
    Dv = D if Dv is None else Dv
    rng = np.random.default_rng(seed)
    out = {
        "q": (rng.standard_normal((B, H, L, D)) / 8.0).astype(np.float32),
        "k": (rng.standard_normal((B, H, L, D)) / 8.0).astype(np.float32),
        "v": (rng.standard_normal((B, H, L, Dv)) / 8.0).astype(np.float32),
    }
    x = rng.standard_normal((B, H, L, D)) + x_mean
    out["g"] = (_logsigmoid(x) / gate_div).astype(np.float32)
    out["meta_k"] = (rng.standard_normal((H, M, D)) / 8.0).astype(np.float32)
    if with_grad:
        out["dO"] = rng.standard_normal((B, H, L, Dv)).astype(np.float32)
    if with_meta_v:
        out["meta_v"] = (rng.standard_normal((H, M, Dv)) / 8.0).astype(np.float32)
    if bf16:
        for name in ("q", "k", "v", "meta_k", "meta_v", "dO"):
            if name in out:
                out[name] = round_to_bf16(out[name])
    return out


def make_gate_small(B: int, L: int, d_model: int, ng: int, dg_shape, *, seed: int, bf16: bool) -> dict:
    """Gate-projection inputs at small sizes (x and w bf16-rounded when bf16)."""
    rng = np.random.default_rng(seed)
    out = {"x": rng.standard_normal((B, L, d_model)).astype(np.float32),
           "w": (rng.standard_normal((ng, d_model)) / np.sqrt(d_model)).astype(np.float32),
           "dg": rng.standard_normal(tuple(dg_shape)).astype(np.float32)}
    if bf16:
        out["x"] = round_to_bf16(out["x"])
        out["w"] = round_to_bf16(out["w"])
    return out


def make_gate_device(B: int, L: int, d_model: int, ng: int, dg_shape, *, seed: int, device, dtype) -> dict:
    """The same recipe drawn on the device with a seeded torch generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn((B, L, d_model), generator=gen, device=device, dtype=torch.float32).to(dtype)
    w = (torch.randn((ng, d_model), generator=gen, device=device, dtype=torch.float32) /
         float(np.sqrt(d_model))).to(dtype)
    dg = torch.randn(tuple(dg_shape), generator=gen, device=device, dtype=torch.float32)
    return {"x": x, "w": w, "dg": dg}


def make_log_features(shape, *, seed: int) -> dict:
    """Log features lq, lk for the GLA branch's feature-map inputs: ~ N(-log(d/2), 0.5^2) each
    (the spread of a softmax over d/2 features), fp32."""
    rng = np.random.default_rng(seed)
    mu = -np.log(shape[-1] / 2.0)
    return {"lq": (rng.standard_normal(shape) * 0.5 + mu).astype(np.float32),
            "lk": (rng.standard_normal(shape) * 0.5 + mu).astype(np.float32)}


def make_log_features_device(shape, *, seed: int, device) -> dict:
    """The same law drawn on the device with a seeded torch generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    mu = -float(np.log(shape[-1] / 2.0))
    return {n: torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32) * 0.5 + mu
            for n in ("lq", "lk")}


def make_inputs_device(w: Workload, device, *, with_grad: bool = False, L: int | None = None,
                       B: int | None = None) -> dict:
    """Same recipe drawn on the device with a seeded torch generator (for the
    full-size workloads, whose host-side generation would take minutes).

    Returns torch tensors on ``device``: q, k, v (and dO) in the workload's
    dtype, g fp32 (logsigmoid evaluated in fp64), meta_k [H,M,D].
    """
    import torch
    L = w.L if L is None else L
    B = w.B if B is None else B
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shp = (B, w.H, L, w.D)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = (torch.randn(shp, generator=gen, device=device, dtype=torch.float32) / 8.0).to(dt)
    x = torch.randn(shp, generator=gen, device=device, dtype=torch.float64) + w.x_mean
    out["g"] = (torch.nn.functional.logsigmoid(x) / 16.0).to(torch.float32)
    del x
    out["meta_k"] = (torch.randn((w.H, w.M, w.D), generator=gen, device=device,
                                 dtype=torch.float32) / 8.0).to(dt)
    if with_grad:
        out["dO"] = torch.randn(shp, generator=gen, device=device, dtype=torch.float32).to(dt)
    return out

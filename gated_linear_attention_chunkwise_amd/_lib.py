"""ctypes binding of liblizard_attn.so (argument marshalling only).

Every function here allocates its outputs with torch on the inputs' device,
passes raw device pointers and the current torch stream to the C ABI and
raises if the library reports an error.  All arithmetic runs in the HIP
kernels; there is no fallback of any kind: without the built library on a
ROCm device these functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblizard_attn.so")

LIZARD_FP32, LIZARD_BF16 = 0, 1
OP_FWD, OP_BWD, OP_DECODE, OP_FWD_CONTINUE, OP_DISTILL, OP_FEATURE_BWD, OP_BWD_RECOMPUTE = 0, 1, 2, 3, 4, 5, 6
GATE_PER_DIM, GATE_SCALAR = 0, 1
SYMBOLS = ("lizard_attn_fwd", "lizard_attn_bwd", "lizard_attn_decode_step", "lizard_attn_fwd_continue",
           "lizard_attn_workspace_bytes", "lizard_attn_status_string", "lizard_gate_proj_fwd",
           "lizard_gate_proj_bwd", "lizard_gate_proj_workspace_bytes", "lizard_distill_mse",
           "lizard_attn_fwd_feat", "lizard_attn_bwd_feat", "lizard_hedgehog_fwd", "lizard_hedgehog_bwd",
           "lizard_attn_fwd_continue_feat", "lizard_attn_decode_step_feat", "lizard_attn_decode_step_noalloc")


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("W", ctypes.c_int32), ("M", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("mix", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32)]


class LizardError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lizard_attn error {code}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m "
                           "gated_linear_attention_chunkwise_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    SP = ctypes.POINTER(Shape)
    lib.lizard_attn_fwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_attn_fwd.restype = I32
    lib.lizard_attn_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P, P]
    lib.lizard_attn_bwd.restype = I32
    lib.lizard_attn_decode_step.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_attn_decode_step.restype = I32
    lib.lizard_attn_fwd_continue.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_attn_fwd_continue.restype = I32
    lib.lizard_attn_workspace_bytes.argtypes = [SP, ctypes.c_int]
    lib.lizard_attn_workspace_bytes.restype = SZ
    lib.lizard_attn_fwd_feat.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_attn_fwd_feat.restype = I32
    lib.lizard_attn_bwd_feat.argtypes = [SP] + [P] * 21 + [SZ, P, P]
    lib.lizard_attn_bwd_feat.restype = I32
    lib.lizard_attn_fwd_continue_feat.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_attn_fwd_continue_feat.restype = I32
    lib.lizard_attn_decode_step_feat.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_attn_decode_step_feat.restype = I32
    lib.lizard_attn_decode_step_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.lizard_attn_decode_step_noalloc.restype = I32
    lib.lizard_hedgehog_fwd.argtypes = [SP, P, P, P, P]
    lib.lizard_hedgehog_fwd.restype = I32
    lib.lizard_hedgehog_bwd.argtypes = [SP, P, P, P, P, P, P, SZ, P]
    lib.lizard_hedgehog_bwd.restype = I32
    lib.lizard_distill_mse.argtypes = [SP, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_distill_mse.restype = I32
    lib.lizard_gate_proj_fwd.argtypes = [SP, I32, F, P, P, P, P]
    lib.lizard_gate_proj_fwd.restype = I32
    lib.lizard_gate_proj_bwd.argtypes = [SP, I32, F, P, P, P, P, P, P, P, SZ, P]
    lib.lizard_gate_proj_bwd.restype = I32
    lib.lizard_gate_proj_workspace_bytes.argtypes = [SP, I32]
    lib.lizard_gate_proj_workspace_bytes.restype = SZ
    lib.lizard_attn_status_string.argtypes = [I32]
    lib.lizard_attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code: int):
    if code != 0:
        raise LizardError(code, load().lizard_attn_status_string(code).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return LIZARD_BF16
    if dt == torch.float32:
        return LIZARD_FP32
    raise TypeError(f"unsupported dtype {dt}: use torch.bfloat16 or torch.float32")


def _need(t, name, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _opt(t, name, dtype, device):
    if t is not None:
        _need(t, name, dtype, device)


def make_shape(B, H, L, d, W, M, scale, mix, dtype, chunk=64, gate=GATE_PER_DIM) -> Shape:
    return Shape(B, H, L, d, d, W, M, chunk, float(scale), float(mix), _dtype_code(dtype), gate)


def _gate_mode(g, q) -> int:
    """Per key dimension when g has q's shape; scalar per head and token when g drops
    q's last axis."""
    if tuple(g.shape) == tuple(q.shape):
        return GATE_PER_DIM
    if tuple(g.shape) == tuple(q.shape[:-1]):
        return GATE_SCALAR
    raise ValueError(f"g must have shape {tuple(q.shape)} (per key dimension) or {tuple(q.shape[:-1])} "
                     f"(one per head and token), got {tuple(g.shape)}")


def _events(evs, n):
    if evs is None:
        return None
    if len(evs) != n:
        raise ValueError(f"need {n} events, got {len(evs)}")
    arr = (ctypes.c_void_p * n)(*[int(e) for e in evs])
    return ctypes.cast(arr, ctypes.c_void_p)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def lizard_attn_fwd(q, k, v, g, meta_k, meta_v=None, *, window: int, scale: float | None = None,
                    mix: float = 1.0, chunk: int = 64, want_lse: bool = False,
                    want_o_swa: bool = False, want_chunk_states: bool = False,
                    want_state: bool = False) -> dict:
    """Forward pass; q, k, v [B,H,L,d] (bf16 or fp32), g [B,H,L,d] fp32, meta_k [H,M,d]."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, n, dt, dev)
    _need(g, "g", torch.float32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, L, d = q.shape
    M = 0 if meta_k is None else meta_k.shape[1]
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,L,d] shape")
    gate = _gate_mode(g, q)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, window, M, scale, mix, dt, chunk, gate)
    C = chunk if chunk else 64
    NC = (L + C - 1) // C
    out = {"o": torch.empty_like(q)}
    out["lse"] = torch.empty(B, H, L, device=dev, dtype=torch.float32) if want_lse else None
    out["o_swa"] = torch.empty_like(q) if want_o_swa else None
    out["chunk_states"] = (torch.empty(B, H, NC, d, d, device=dev, dtype=dt)
                           if want_chunk_states else None)
    out["state"] = torch.empty(B, H, d, d, device=dev, dtype=torch.float32) if want_state else None
    ws, ws_bytes = None, 0
    if L > 0:
        # segment buffers of the state sweep, plus the chunk states unless they are an output
        ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_FWD)
        if want_chunk_states:
            ws_bytes -= out["chunk_states"].numel() * out["chunk_states"].element_size()
        if ws_bytes > 0:
            ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    _check(lib.lizard_attn_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(meta_k),
                               _ptr(meta_v), _ptr(out["o"]), _ptr(out["lse"]), _ptr(out["o_swa"]),
                               _ptr(out["chunk_states"]), _ptr(out["state"]), _ptr(ws), ws_bytes,
                               _stream(dev)))
    return out


BWD_STAGES = 3


def lizard_attn_bwd(q, k, v, g, meta_k, meta_v, dO, lse=None, o_swa=None, chunk_states=None, *, window: int,
                    scale: float | None = None, mix: float = 1.0, chunk: int = 64,
                    stage_events=None) -> dict:
    """Backward pass; returns dq, dk, dv, dg, dmeta_k, dmeta_v.  ``lse``, ``o_swa`` and
    ``chunk_states`` are the forward's saved tensors; when any is None the library
    recomputes them (a forward's time, a larger workspace).

    ``stage_events``: optional sequence of BWD_STAGES + 1 raw hipEvent_t handles
    (ints) recorded around the backward's kernels (profiling hook)."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _need(t, n, dt, dev)
    _opt(o_swa, "o_swa", dt, dev)
    _opt(chunk_states, "chunk_states", dt, dev)
    _need(g, "g", torch.float32, dev)
    _opt(lse, "lse", torch.float32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, L, d = q.shape
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, window, M, scale, mix, dt, chunk, _gate_mode(g, q))
    recompute = lse is None or o_swa is None or chunk_states is None
    ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_BWD_RECOMPUTE if recompute else OP_BWD)
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dg": torch.empty_like(g)}
    out["dmeta_k"] = torch.empty(H, M, d, device=dev, dtype=torch.float32) if M > 0 else None
    out["dmeta_v"] = (torch.empty(H, M, d, device=dev, dtype=torch.float32)
                      if (meta_v is not None and M > 0) else None)
    if M == 0:
        meta_v = None
    _check(lib.lizard_attn_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(meta_k),
                               _ptr(meta_v), _ptr(dO), _ptr(lse), _ptr(o_swa), _ptr(chunk_states),
                               _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                               _ptr(out["dmeta_k"]), _ptr(out["dmeta_v"]), _ptr(ws), ws_bytes,
                               _stream(dev), _events(stage_events, BWD_STAGES + 1)))
    return out


def decode_workspace(B: int, H: int, d: int, device) -> torch.Tensor:
    """Workspace for lizard_attn_decode_step at this shape (the step needs none: a one-byte
    placeholder, kept so that callers written for a workspace still work)."""
    s = make_shape(B, H, 0, d, 1, 0, 1.0, 1.0, torch.bfloat16)
    n = int(load().lizard_attn_workspace_bytes(ctypes.byref(s), OP_DECODE))
    return torch.empty(max(n, 1), device=device, dtype=torch.uint8)


def lizard_attn_decode_step(q, k, v, g, meta_k, meta_v, state, ring_k, ring_v, pos, *,
                            window: int, scale: float | None = None, mix: float = 1.0, out=None,
                            workspace=None):
    """One decode step, in place on (state, ring_k, ring_v, pos); returns o [B,H,d].
    ``workspace``: optional uint8 device tensor from decode_workspace() (allocated per call
    when omitted)."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("ring_k", ring_k), ("ring_v", ring_v)):
        _need(t, n, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    _need(pos, "pos", torch.int32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, d = q.shape
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, 0, d, window, M, scale, mix, dt, gate=_gate_mode(g, q))
    o = torch.empty_like(q) if out is None else out
    ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_DECODE)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    if workspace.numel() < ws_bytes:
        raise ValueError(f"decode workspace needs {ws_bytes} bytes, got {workspace.numel()}")
    _check(lib.lizard_attn_decode_step(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(meta_k), _ptr(meta_v), _ptr(state), _ptr(ring_k),
                                       _ptr(ring_v), _ptr(pos), _ptr(o), _ptr(workspace),
                                       ws_bytes, _stream(dev)))
    return o


def lizard_attn_decode_step_noalloc(q, k, v, g, meta_k, meta_v, state, ring_k, ring_v, pos, *,
                                    window: int, scale: float | None = None, mix: float = 1.0, out):
    """lizard_attn_decode_step with no workspace argument (the step needs none).  ``out`` [B,H,d]
    must be given (this call allocates nothing); returns it."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("ring_k", ring_k), ("ring_v", ring_v), ("out", out)):
        _need(t, n, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    _need(pos, "pos", torch.int32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, d = q.shape
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, 0, d, window, M, scale, mix, dt, gate=_gate_mode(g, q))
    _check(lib.lizard_attn_decode_step_noalloc(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                               _ptr(meta_k), _ptr(meta_v), _ptr(state), _ptr(ring_k),
                                               _ptr(ring_v), _ptr(pos), _ptr(out), _stream(dev)))
    return out


def continue_workspace(B: int, H: int, L: int, d: int, dtype, device) -> torch.Tensor:
    """Workspace for lizard_attn_fwd_continue at this shape (reusable across segments of length <= L)."""
    s = make_shape(B, H, L, d, 1, 0, 1.0, 1.0, dtype)
    n = int(load().lizard_attn_workspace_bytes(ctypes.byref(s), OP_FWD_CONTINUE))
    return torch.empty(max(n, 1), device=device, dtype=torch.uint8)


def lizard_attn_fwd_continue(q, k, v, g, meta_k, meta_v, state, ring_k, ring_v, pos, *,
                             window: int, scale: float | None = None, mix: float = 1.0,
                             out=None, workspace=None):
    """Forward of the next L tokens of every sequence, resuming from the carry
    (state [B,H,d,d] fp32, ring_k / ring_v [B,H,W,d], pos [B] int32), all updated in
    place for the next segment or decode step; returns o [B,H,L,d].  ``workspace``:
    optional uint8 device tensor from continue_workspace() (allocated per call when omitted)."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("ring_k", ring_k), ("ring_v", ring_v)):
        _need(t, n, dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(state, "state", torch.float32, dev)
    _need(pos, "pos", torch.int32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, L, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,L,d] shape")
    gate = _gate_mode(g, q)
    if state.shape != (B, H, d, d) or ring_k.shape != (B, H, window, d) or ring_v.shape != ring_k.shape \
            or pos.shape != (B,):
        raise ValueError("carry shapes must be state [B,H,d,d], ring [B,H,W,d], pos [B]")
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, window, M, scale, mix, dt, gate=gate)
    o = torch.empty_like(q) if out is None else out
    ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_FWD_CONTINUE)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    if workspace.numel() < ws_bytes:
        raise ValueError(f"continuation workspace needs {ws_bytes} bytes, got {workspace.numel()}")
    _check(lib.lizard_attn_fwd_continue(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                        _ptr(meta_k), _ptr(meta_v), _ptr(state), _ptr(ring_k),
                                        _ptr(ring_v), _ptr(pos), _ptr(o), _ptr(workspace),
                                        workspace.numel(), _stream(dev)))
    return o


def lizard_attn_fwd_feat(q, k, v, lq, lk, g, meta_k, meta_v=None, *, window: int, scale: float | None = None,
                         mix: float = 1.0, chunk: int = 64, want_lse: bool = False, want_o_swa: bool = False,
                         want_chunk_states: bool = False, want_state: bool = False) -> dict:
    """Forward with GLA log features: the GLA branch runs on exp(lq), exp(lk) (fp32 [B,H,L,d],
    gate absorbed in log space), the window on q, k; otherwise as lizard_attn_fwd."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need(t, n, dt, dev)
    for n, t in (("lq", lq), ("lk", lk), ("g", g)):
        _need(t, n, torch.float32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, L, d = q.shape
    if not (k.shape == v.shape == lq.shape == lk.shape == g.shape == q.shape):
        raise ValueError("q, k, v, lq, lk and g must share one [B,H,L,d] shape")
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, window, M, scale, mix, dt, chunk, GATE_PER_DIM)
    NC = (L + 63) // 64
    out = {"o": torch.empty_like(q)}
    out["lse"] = torch.empty(B, H, L, device=dev, dtype=torch.float32) if want_lse else None
    out["o_swa"] = torch.empty_like(q) if want_o_swa else None
    out["chunk_states"] = (torch.empty(B, H, NC, d, d, device=dev, dtype=dt) if want_chunk_states else None)
    out["state"] = torch.empty(B, H, d, d, device=dev, dtype=torch.float32) if want_state else None
    ws, ws_bytes = None, 0
    if L > 0:
        ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_FWD)
        if want_chunk_states:
            ws_bytes -= out["chunk_states"].numel() * out["chunk_states"].element_size()
        if ws_bytes > 0:
            ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    _check(lib.lizard_attn_fwd_feat(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(lq), _ptr(lk), _ptr(g),
                                    _ptr(meta_k), _ptr(meta_v), _ptr(out["o"]), _ptr(out["lse"]),
                                    _ptr(out["o_swa"]), _ptr(out["chunk_states"]), _ptr(out["state"]), _ptr(ws),
                                    ws_bytes, _stream(dev)))
    return out


def lizard_attn_bwd_feat(q, k, v, lq, lk, g, meta_k, meta_v, dO, lse=None, o_swa=None, chunk_states=None, *,
                         window: int, scale: float | None = None, mix: float = 1.0, chunk: int = 64,
                         stage_events=None) -> dict:
    """Backward of lizard_attn_fwd_feat: dq, dk (window branch), dv, dlq, dlk (GLA log features),
    dg, dmeta_k, dmeta_v; the saved forward tensors may be None (recomputed)."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _need(t, n, dt, dev)
    _opt(o_swa, "o_swa", dt, dev)
    _opt(chunk_states, "chunk_states", dt, dev)
    for n, t in (("lq", lq), ("lk", lk), ("g", g)):
        _need(t, n, torch.float32, dev)
    _opt(lse, "lse", torch.float32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, L, d = q.shape
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, window, M, scale, mix, dt, chunk, GATE_PER_DIM)
    recompute = lse is None or o_swa is None or chunk_states is None
    ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_BWD_RECOMPUTE if recompute else OP_BWD)
    ws = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dlq": torch.empty_like(lq), "dlk": torch.empty_like(lk), "dg": torch.empty_like(g)}
    out["dmeta_k"] = torch.empty(H, M, d, device=dev, dtype=torch.float32) if M > 0 else None
    out["dmeta_v"] = (torch.empty(H, M, d, device=dev, dtype=torch.float32)
                      if (meta_v is not None and M > 0) else None)
    if M == 0:
        meta_v = None
    _check(lib.lizard_attn_bwd_feat(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(lq), _ptr(lk), _ptr(g),
                                    _ptr(meta_k), _ptr(meta_v), _ptr(dO), _ptr(lse), _ptr(o_swa),
                                    _ptr(chunk_states), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                    _ptr(out["dlq"]), _ptr(out["dlk"]), _ptr(out["dg"]), _ptr(out["dmeta_k"]),
                                    _ptr(out["dmeta_v"]), _ptr(ws), ws_bytes, _stream(dev),
                                    _events(stage_events, BWD_STAGES + 1)))
    return out


def lizard_attn_fwd_continue_feat(q, k, v, lq, lk, g, meta_k, meta_v, state, ring_k, ring_v, pos, *,
                                  window: int, scale: float | None = None, mix: float = 1.0, out=None,
                                  workspace=None):
    """lizard_attn_fwd_continue with GLA log features lq, lk (fp32 [B,H,L,d]); returns o."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("ring_k", ring_k), ("ring_v", ring_v)):
        _need(t, n, dt, dev)
    for n, t in (("lq", lq), ("lk", lk), ("g", g), ("state", state)):
        _need(t, n, torch.float32, dev)
    _need(pos, "pos", torch.int32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, L, d = q.shape
    if not (k.shape == v.shape == lq.shape == lk.shape == g.shape == q.shape):
        raise ValueError("q, k, v, lq, lk and g must share one [B,H,L,d] shape")
    if state.shape != (B, H, d, d) or ring_k.shape != (B, H, window, d) or ring_v.shape != ring_k.shape \
            or pos.shape != (B,):
        raise ValueError("carry shapes must be state [B,H,d,d], ring [B,H,W,d], pos [B]")
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, window, M, scale, mix, dt, gate=GATE_PER_DIM)
    o = torch.empty_like(q) if out is None else out
    ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_FWD_CONTINUE)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    _check(lib.lizard_attn_fwd_continue_feat(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(lq), _ptr(lk),
                                             _ptr(g), _ptr(meta_k), _ptr(meta_v), _ptr(state), _ptr(ring_k),
                                             _ptr(ring_v), _ptr(pos), _ptr(o), _ptr(workspace), workspace.numel(),
                                             _stream(dev)))
    return o


def lizard_attn_decode_step_feat(q, k, v, lq, lk, g, meta_k, meta_v, state, ring_k, ring_v, pos, *,
                                 window: int, scale: float | None = None, mix: float = 1.0, out=None,
                                 workspace=None):
    """lizard_attn_decode_step with GLA log features lq, lk (fp32 [B,H,d]); returns o [B,H,d]."""
    lib = load()
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("ring_k", ring_k), ("ring_v", ring_v)):
        _need(t, n, dt, dev)
    for n, t in (("lq", lq), ("lk", lk), ("g", g), ("state", state)):
        _need(t, n, torch.float32, dev)
    _need(pos, "pos", torch.int32, dev)
    _opt(meta_k, "meta_k", dt, dev)
    _opt(meta_v, "meta_v", dt, dev)
    B, H, d = q.shape
    M = 0 if meta_k is None else meta_k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, 0, d, window, M, scale, mix, dt, gate=GATE_PER_DIM)
    o = torch.empty_like(q) if out is None else out
    ws_bytes = lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_DECODE)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    _check(lib.lizard_attn_decode_step_feat(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(lq), _ptr(lk), _ptr(g),
                                            _ptr(meta_k), _ptr(meta_v), _ptr(state), _ptr(ring_k), _ptr(ring_v),
                                            _ptr(pos), _ptr(o), _ptr(workspace), workspace.numel(), _stream(dev)))
    return o


def _feat_shape(x, w):
    B, H, L, d = x.shape
    if tuple(w.shape) != (H, d, d // 2):
        raise ValueError(f"w must have shape ({H}, {d}, {d // 2}), got {tuple(w.shape)}")
    return make_shape(B, H, L, d, 1, 0, 1.0, 1.0, x.dtype)


def lizard_hedgehog_fwd(x, w):
    """log phi(x) = [z - lse(z), -z - lse(-z)], z = x w_h: x [B,H,L,d] (bf16 or fp32), w [H,d,d/2]
    in x's dtype; returns fp32 [B,H,L,d]."""
    lib = load()
    dt, dev = x.dtype, x.device
    _need(x, "x", dt, dev)
    _need(w, "w", dt, dev)
    s = _feat_shape(x, w)
    out = torch.empty(x.shape, device=dev, dtype=torch.float32)
    _check(lib.lizard_hedgehog_fwd(ctypes.byref(s), _ptr(x), _ptr(w), _ptr(out), _stream(dev)))
    return out


def lizard_hedgehog_bwd(x, w, dl, workspace=None):
    """Gradients (dx in x's dtype, dw fp32 [H,d,d/2]) of sum(dl * log phi(x))."""
    lib = load()
    dt, dev = x.dtype, x.device
    _need(x, "x", dt, dev)
    _need(w, "w", dt, dev)
    _need(dl, "dl", torch.float32, dev)
    s = _feat_shape(x, w)
    n = int(lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_FEATURE_BWD))
    if workspace is None:
        workspace = torch.empty(max(n, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    dx = torch.empty_like(x)
    dw = torch.empty(w.shape, device=dev, dtype=torch.float32)
    _check(lib.lizard_hedgehog_bwd(ctypes.byref(s), _ptr(x), _ptr(w), _ptr(dl), _ptr(dx), _ptr(dw),
                                   _ptr(workspace), workspace.numel(), _stream(dev)))
    return dx, dw


def lizard_distill_mse(q_t, k_t, v_t, o_s, *, scale: float | None = None, out=None, workspace=None) -> dict:
    """Stage-1 loss: the teacher's causal softmax attention of (q_t, k_t, v_t) against the layer
    output o_s; returns {"loss": fp32 device scalar (mean squared error over every element),
    "dO": 2 (o_s - o_T) / N in o_s's dtype, the gradient for lizard_attn_bwd}."""
    lib = load()
    dt, dev = q_t.dtype, q_t.device
    for n, t in (("q_t", q_t), ("k_t", k_t), ("v_t", v_t), ("o_s", o_s)):
        _need(t, n, dt, dev)
    if not (q_t.shape == k_t.shape == v_t.shape == o_s.shape):
        raise ValueError("q_t, k_t, v_t and o_s must share one [B,H,L,d] shape")
    B, H, L, d = q_t.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = make_shape(B, H, L, d, 1, 0, scale, 1.0, dt)
    n = int(lib.lizard_attn_workspace_bytes(ctypes.byref(s), OP_DISTILL))
    if workspace is None:
        workspace = torch.empty(max(n, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    dO = torch.empty_like(o_s) if out is None else out
    loss = torch.empty((), device=dev, dtype=torch.float32)
    _check(lib.lizard_distill_mse(ctypes.byref(s), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(o_s), _ptr(dO),
                                  _ptr(loss), _ptr(workspace), workspace.numel(), _stream(dev)))
    return {"loss": loss, "dO": dO}


def _gate_shape(x, w, heads, d_k, scalar):
    B, L, Dm = x.shape
    ng = heads if scalar else heads * d_k
    if tuple(w.shape) != (ng, Dm):
        raise ValueError(f"w must have shape ({ng}, {Dm}), got {tuple(w.shape)}")
    return make_shape(B, heads, L, d_k, 1, 0, 1.0, 1.0, x.dtype,
                      gate=GATE_SCALAR if scalar else GATE_PER_DIM), Dm


def lizard_gate_proj_fwd(x, w, *, heads: int, d_k: int, tau: float = 1.0, scalar: bool = False):
    """g = log sigmoid(x w^T) / tau in the layer's gate layout: x [B,L,d_model], w [Ng,d_model]
    (Ng = heads*d_k, or heads for the scalar gate), both bf16 or fp32; returns g fp32
    [B,heads,L,d_k] or [B,heads,L]."""
    lib = load()
    dt, dev = x.dtype, x.device
    _need(x, "x", dt, dev)
    _need(w, "w", dt, dev)
    s, Dm = _gate_shape(x, w, heads, d_k, scalar)
    B, L = x.shape[0], x.shape[1]
    g = torch.empty((B, heads, L) if scalar else (B, heads, L, d_k), device=dev, dtype=torch.float32)
    _check(lib.lizard_gate_proj_fwd(ctypes.byref(s), Dm, float(tau), _ptr(x), _ptr(w), _ptr(g), _stream(dev)))
    return g


def lizard_gate_proj_bwd(x, w, g, dg, *, heads: int, d_k: int, tau: float = 1.0, scalar: bool = False,
                         workspace=None):
    """Gradients (dx [B,L,d_model] in x's dtype, dw [Ng,d_model] fp32) of sum(dg * g) for
    g = lizard_gate_proj_fwd(x, w, ...); g is that forward's output."""
    lib = load()
    dt, dev = x.dtype, x.device
    _need(x, "x", dt, dev)
    _need(w, "w", dt, dev)
    _need(g, "g", torch.float32, dev)
    _need(dg, "dg", torch.float32, dev)
    s, Dm = _gate_shape(x, w, heads, d_k, scalar)
    if tuple(g.shape) != tuple(dg.shape):
        raise ValueError("g and dg must share one shape")
    n = int(lib.lizard_gate_proj_workspace_bytes(ctypes.byref(s), Dm))
    if workspace is None:
        workspace = torch.empty(max(n, 1), device=dev, dtype=torch.uint8)
    _need(workspace, "workspace", torch.uint8, dev)
    dx = torch.empty_like(x)
    dw = torch.empty(w.shape, device=dev, dtype=torch.float32)
    _check(lib.lizard_gate_proj_bwd(ctypes.byref(s), Dm, float(tau), _ptr(x), _ptr(w), _ptr(g), _ptr(dg),
                                    _ptr(dx), _ptr(dw), _ptr(workspace), workspace.numel(), _stream(dev)))
    return dx, dw


def gate_proj_workspace(x_shape, heads: int, d_k: int, dtype, device, scalar: bool = False) -> torch.Tensor:
    """Workspace for lizard_gate_proj_bwd at this shape (reusable across calls)."""
    B, L, Dm = x_shape
    s = make_shape(B, heads, L, d_k, 1, 0, 1.0, 1.0, dtype, gate=GATE_SCALAR if scalar else GATE_PER_DIM)
    n = int(load().lizard_gate_proj_workspace_bytes(ctypes.byref(s), Dm))
    return torch.empty(max(n, 1), device=device, dtype=torch.uint8)


def workspace_bytes(shape: Shape, op: int) -> int:
    return int(load().lizard_attn_workspace_bytes(ctypes.byref(shape), op))


# short aliases
fwd = lizard_attn_fwd
bwd = lizard_attn_bwd
decode_step = lizard_attn_decode_step
fwd_continue = lizard_attn_fwd_continue
distill_mse = lizard_distill_mse
fwd_feat = lizard_attn_fwd_feat
hedgehog_fwd = lizard_hedgehog_fwd
hedgehog_bwd = lizard_hedgehog_bwd
bwd_feat = lizard_attn_bwd_feat
gate_proj_fwd = lizard_gate_proj_fwd
gate_proj_bwd = lizard_gate_proj_bwd

"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid calls on the host before any launch."""
import ctypes
import os
import re

import pytest

import gated_linear_attention_chunkwise_amd as pkg
from gated_linear_attention_chunkwise_amd._lib import Shape, load

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lizard_attn.h")

OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, EHIP = range(6)


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_][a-z_0-9 ]*[\s\*]+(lizard_(?:attn|gate|distill|hedgehog)_[a-z_]+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def lib():
    # LIZARD_ATTN_LIB: another build of the same library (the host-sanitized variant)
    path = os.environ.get("LIZARD_ATTN_LIB", pkg._lib.LIB_PATH)
    if not os.path.exists(path):
        pytest.skip("library not built")
    return load(path)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == {"lizard_attn_fwd", "lizard_attn_bwd", "lizard_attn_decode_step",
                          "lizard_attn_fwd_continue", "lizard_attn_workspace_bytes",
                          "lizard_attn_status_string", "lizard_gate_proj_fwd", "lizard_gate_proj_bwd",
                          "lizard_gate_proj_workspace_bytes", "lizard_distill_mse", "lizard_attn_fwd_feat",
                          "lizard_attn_bwd_feat", "lizard_hedgehog_fwd", "lizard_hedgehog_bwd",
                          "lizard_attn_fwd_continue_feat", "lizard_attn_decode_step_feat",
                          "lizard_attn_decode_step_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(pkg.SYMBOLS) == set(names)


def test_status_strings(lib):
    for code in range(6):
        assert lib.lizard_attn_status_string(code)
    assert b"unknown" in lib.lizard_attn_status_string(99)


def shape(**kw):
    base = dict(B=1, H=2, L=128, d_k=128, d_v=128, W=128, M=4, chunk=64, scale=0.088, mix=1.0,
                dtype=1, gate=0)
    base.update(kw)
    return Shape(*(base[f] for f, _ in Shape._fields_))


P = ctypes.c_void_p
GOOD = P(0x10000)          # aligned, never dereferenced (validation fails first)
BAD = P(0x10008)           # 8-byte aligned only


def fwd(lib, s, q=GOOD, meta_k=GOOD, meta_v=None, o=GOOD, lse=None):
    return lib.lizard_attn_fwd(ctypes.byref(s), q, GOOD, GOOD, GOOD, meta_k, meta_v, o, lse, None,
                               None, None, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d_k=96, d_v=96), EUNSUPPORTED), (dict(d_k=64, d_v=128), EUNSUPPORTED),
    (dict(dtype=7), EUNSUPPORTED), (dict(gate=2), EUNSUPPORTED),
    (dict(M=17), EUNSUPPORTED), (dict(chunk=24), EUNSUPPORTED), (dict(chunk=256), EUNSUPPORTED),
    (dict(chunk=-64), EUNSUPPORTED), (dict(L=(1 << 30) + 1), EUNSUPPORTED),
    (dict(B=0), EINVAL), (dict(L=-1), EINVAL), (dict(W=0), EINVAL), (dict(M=-1), EINVAL),
    (dict(scale=float("nan")), EINVAL),
])
def test_fwd_rejects_bad_shapes(lib, kw, code):
    assert fwd(lib, shape(**kw)) == code


def test_fwd_rejects_bad_pointers(lib):
    assert lib.lizard_attn_fwd(None, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None, None, None,
                               None, None, 0, None) == EINVAL
    assert fwd(lib, shape(), q=None) == EINVAL
    assert fwd(lib, shape(), o=None) == EINVAL
    assert fwd(lib, shape(), meta_k=None) == EINVAL          # M > 0 needs meta keys
    assert fwd(lib, shape(), q=BAD) == EALIGN
    assert fwd(lib, shape(), lse=BAD) == EALIGN


def test_bwd_validation(lib):
    s = shape()
    def call(meta_v=None, dmeta_v=None, ws=GOOD, ws_bytes=1 << 40, dq=GOOD, dmeta_k=GOOD):
        return lib.lizard_attn_bwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, meta_v, GOOD,
                                   GOOD, GOOD, GOOD, dq, GOOD, GOOD, GOOD, dmeta_k, dmeta_v, ws,
                                   ws_bytes, None, None)
    assert call(meta_v=GOOD, dmeta_v=None) == EINVAL
    assert call(meta_v=None, dmeta_v=GOOD) == EINVAL
    assert call(dq=None) == EINVAL
    assert call(dmeta_k=None) == EINVAL
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 1)
    if need > 0:
        assert call(ws=None) == EWORKSPACE
        assert call(ws_bytes=need - 1) == EWORKSPACE


def test_bwd_saved_tensors_optional(lib):
    """lse, o_swa and chunk_states may be NULL: the backward then recomputes them, in a larger
    workspace (the forward's workspace with its chunk states, lse and o_swa on top)."""
    s = shape()
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 1)
    rc = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 6)
    up = lambda x: (x + 255) // 256 * 256
    fwd = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 0)
    B, H, L, d = 1, 2, 128, 128
    assert rc == need + up(fwd) + up(4 * B * H * L) + up(2 * B * H * L * d)
    def call(lse=GOOD, o_swa=GOOD, cs=GOOD, ws=GOOD, ws_bytes=need):
        return lib.lizard_attn_bwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD,
                                   lse, o_swa, cs, GOOD, GOOD, GOOD, GOOD, GOOD, None, ws,
                                   ws_bytes, None, None)
    for kw in (dict(lse=None), dict(o_swa=None), dict(cs=None), dict(lse=None, o_swa=None, cs=None)):
        assert call(**kw) == EWORKSPACE, kw                  # the plain backward's workspace is too small
        assert call(ws=BAD, ws_bytes=rc, **kw) == EALIGN, kw
    assert call(lse=BAD) == EALIGN
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(shape(L=0)), 6) == 0


def test_decode_validation(lib):
    s = shape(L=0)
    def call(state=GOOD, pos=GOOD, s_=s, ws=GOOD, ws_bytes=1 << 40):
        return lib.lizard_attn_decode_step(ctypes.byref(s_), GOOD, GOOD, GOOD, GOOD, GOOD, None,
                                           state, GOOD, GOOD, pos, GOOD, ws, ws_bytes, None)
    assert call(state=None) == EINVAL
    assert call(pos=None) == EINVAL
    assert call(pos=BAD) == EALIGN
    assert call(s_=shape(W=9000)) == EUNSUPPORTED
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(s), 2) == 0   # the step needs no workspace
    assert call(ws=BAD, ws_bytes=0) == EALIGN                          # one that is given is still checked


def test_long_windows_accepted(lib):
    """Forward and backward take any window length: W beyond three chunks, and W far beyond L
    (the whole causal prefix), pass validation up to the workspace check."""
    for W in (130, 1000, 2 ** 31 - 1):
        s = shape(W=W)
        assert lib.lizard_attn_fwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None,
                                   None, None, None, None, 0, None) == EWORKSPACE
        assert lib.lizard_attn_bwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD,
                                   GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 0, None, None) == EWORKSPACE


def test_fwd_needs_workspace_without_chunk_states(lib):
    s = shape()
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 0)
    n = 1 * 2 * 2                                     # B*H*chunks
    up = lambda x: (x + 255) // 256 * 256
    dispatch = 256 + up(4 * n) + up(2 * n * (128 // 16))   # strong-gate counter, list, column masks
    assert need == n * 128 * 128 * 2 + dispatch       # + the bf16 chunk states
    def call(ws, ws_bytes):
        return lib.lizard_attn_fwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None,
                                   None, None, None, ws, ws_bytes, None)
    assert call(None, 0) == EWORKSPACE
    assert call(GOOD, need - 1) == EWORKSPACE
    assert call(BAD, need) == EALIGN


def test_fwd_continue_validation(lib):
    s = shape()
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 3)
    assert need == lib.lizard_attn_workspace_bytes(ctypes.byref(s), 0)   # the chunk states
    def call(s_=s, state=GOOD, ring_k=GOOD, pos=GOOD, meta_k=GOOD, ws=GOOD, ws_bytes=1 << 40, q=GOOD):
        return lib.lizard_attn_fwd_continue(ctypes.byref(s_), q, GOOD, GOOD, GOOD, meta_k, None,
                                            state, ring_k, GOOD, pos, GOOD, ws, ws_bytes, None)
    assert call(state=None) == EINVAL
    assert call(ring_k=None) == EINVAL
    assert call(pos=None) == EINVAL
    assert call(meta_k=None) == EINVAL
    assert call(pos=BAD) == EALIGN
    assert call(s_=shape(W=9000)) == EUNSUPPORTED           # the ring holds at most 8192 keys
    assert call(s_=shape(W=8192), ws=None) == EWORKSPACE    # (a valid shape: the workspace check is next)
    assert call(s_=shape(dtype=0)) == EUNSUPPORTED          # fp32 runs d = 64 only
    assert call(ws=None) == EWORKSPACE
    assert call(ws_bytes=need - 1) == EWORKSPACE
    assert call(ws=BAD, ws_bytes=need) == EALIGN
    # no new tokens: nothing is touched, NULL tensors allowed
    z = shape(L=0)
    assert lib.lizard_attn_fwd_continue(ctypes.byref(z), None, None, None, None, GOOD, None, None, None,
                                        None, None, None, None, 0, None) == OK


def test_workspace_query(lib):
    assert lib.lizard_attn_workspace_bytes(None, 1) == 0
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(shape(d_k=96, d_v=96)), 1) == 0
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(shape(L=0)), 0) == 0
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(shape()), 7) == 0       # unknown op


def test_gate_proj_validation(lib):
    F = ctypes.c_float
    def fwdc(s, d_model=256, tau=1.0, x=GOOD, w=GOOD, g=GOOD):
        return lib.lizard_gate_proj_fwd(ctypes.byref(s), d_model, F(tau), x, w, g, None)
    def bwdc(s, d_model=256, tau=1.0, dx=GOOD, dw=GOOD, ws=GOOD, ws_bytes=1 << 40):
        return lib.lizard_gate_proj_bwd(ctypes.byref(s), d_model, F(tau), GOOD, GOOD, GOOD, GOOD, dx, dw, ws,
                                        ws_bytes, None)
    s = shape()
    assert lib.lizard_gate_proj_fwd(None, 256, F(1.0), GOOD, GOOD, GOOD, None) == EINVAL
    assert fwdc(s, tau=0.0) == EINVAL
    assert fwdc(s, tau=float("inf")) == EINVAL
    assert fwdc(s, d_model=0) == EINVAL
    assert fwdc(s, d_model=100) == EUNSUPPORTED
    assert fwdc(s, d_model=65568) == EUNSUPPORTED
    assert fwdc(shape(d_k=96, d_v=96)) == EUNSUPPORTED
    assert fwdc(shape(gate=2)) == EUNSUPPORTED
    assert fwdc(shape(dtype=5)) == EUNSUPPORTED
    assert fwdc(shape(B=4, H=32, L=1 << 20)) == EUNSUPPORTED      # 2^22 tokens x 4096 gate rows
    assert fwdc(s, x=None) == EINVAL
    assert fwdc(s, g=BAD) == EALIGN
    assert bwdc(s, dx=None) == EINVAL
    assert bwdc(s, dw=BAD) == EALIGN
    need = lib.lizard_gate_proj_workspace_bytes(ctypes.byref(s), 256)
    assert need > 0
    assert bwdc(s, ws=None) == EWORKSPACE
    assert bwdc(s, ws_bytes=need - 1) == EWORKSPACE
    # L = 0: the forward writes nothing and accepts absent token tensors
    assert lib.lizard_gate_proj_fwd(ctypes.byref(shape(L=0)), 256, F(1.0), None, GOOD, None, None) == OK


def test_gate_proj_workspace_sizes(lib):
    # dz [tokens][Ng rounded up to 16 bytes] in the operand dtype (256-byte aligned), then fp32
    # partials of dw when its contraction over tokens is split
    s = shape(B=1, H=2, L=128, d_k=128, d_v=128, dtype=1, gate=0)      # Ng = 256, 4 output tiles
    assert lib.lizard_gate_proj_workspace_bytes(ctypes.byref(s), 256) == 128 * 256 * 2 + 4 * 256 * 256 * 4
    s = shape(B=1, H=2, L=128, d_k=128, d_v=128, dtype=1, gate=1)      # Ng = 2 (padded to 8), one split
    assert lib.lizard_gate_proj_workspace_bytes(ctypes.byref(s), 256) == 128 * 8 * 2
    assert lib.lizard_gate_proj_workspace_bytes(ctypes.byref(shape(L=0)), 256) == 0
    assert lib.lizard_gate_proj_workspace_bytes(ctypes.byref(s), 100) == 0


def test_distill_validation(lib):
    s = shape()
    def call(s=s, q=GOOD, dO=GOOD, loss=GOOD, ws=GOOD, ws_bytes=1 << 30):
        return lib.lizard_distill_mse(ctypes.byref(s), q, GOOD, GOOD, GOOD, dO, loss, ws, ws_bytes, None)
    assert lib.lizard_distill_mse(None, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 30, None) == EINVAL
    assert call(q=None) == EINVAL
    assert call(loss=None) == EINVAL
    assert call(dO=BAD) == EALIGN
    assert call(s=shape(d_k=96, d_v=96)) == EUNSUPPORTED
    assert call(s=shape(dtype=0)) == EUNSUPPORTED           # fp32 only at d = 64
    # one fp32 partial per (batch, head, block of 128 queries)
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(shape(B=2, H=3, L=300)), 4) == 2 * 3 * 3 * 4
    assert call(ws_bytes=4 * 2 - 1) == EWORKSPACE             # B=1 H=2 L=128: two partials
    assert call(ws=None) == EINVAL


def test_feature_entry_points_validation(lib):
    s = shape()
    def fwdf(s=s, lq=GOOD, lk=GOOD):
        return lib.lizard_attn_fwd_feat(ctypes.byref(s), GOOD, GOOD, GOOD, lq, lk, GOOD, GOOD, None, GOOD, None,
                                        None, GOOD, None, None, 0, None)
    assert fwdf(lq=None) == EINVAL
    assert fwdf(lk=None) == EINVAL
    assert fwdf(lq=BAD) == EALIGN
    assert fwdf(s=shape(gate=1)) == EUNSUPPORTED
    assert fwdf(s=shape(d_k=96, d_v=96)) == EUNSUPPORTED
    def bwdf(dlq=GOOD, dlk=GOOD, s=s):
        return lib.lizard_attn_bwd_feat(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD,
                                        GOOD, GOOD, GOOD, GOOD, GOOD, dlq, dlk, GOOD, GOOD, None, GOOD, 1 << 40,
                                        None, None)
    assert bwdf(dlq=None) == EINVAL
    assert bwdf(dlk=BAD) == EALIGN
    assert bwdf(s=shape(gate=1)) == EUNSUPPORTED


def test_hedgehog_validation(lib):
    s = shape()
    assert lib.lizard_hedgehog_fwd(ctypes.byref(s), None, GOOD, GOOD, None) == EINVAL
    assert lib.lizard_hedgehog_fwd(ctypes.byref(s), GOOD, GOOD, BAD, None) == EALIGN
    assert lib.lizard_hedgehog_fwd(ctypes.byref(shape(d_k=96, d_v=96)), GOOD, GOOD, GOOD, None) == EUNSUPPORTED
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 5)
    assert need > 0
    def bw(ws=GOOD, nb=need, dx=GOOD):
        return lib.lizard_hedgehog_bwd(ctypes.byref(s), GOOD, GOOD, GOOD, dx, GOOD, ws, nb, None)
    assert bw(dx=None) == EINVAL
    assert bw(ws=None) == EINVAL
    assert bw(nb=need - 1) == EWORKSPACE
    assert lib.lizard_attn_workspace_bytes(ctypes.byref(shape(L=0)), 5) == 0


def test_feature_carry_entry_points_validation(lib):
    s = shape()
    def cont(s=s, lq=GOOD):
        return lib.lizard_attn_fwd_continue_feat(ctypes.byref(s), GOOD, GOOD, GOOD, lq, GOOD, GOOD, GOOD, None,
                                                 GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 40, None)
    assert cont(lq=None) == EINVAL
    assert cont(lq=BAD) == EALIGN
    assert cont(s=shape(gate=1)) == EUNSUPPORTED
    d = shape(L=0)
    def dec(s=d, lk=GOOD):
        return lib.lizard_attn_decode_step_feat(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, lk, GOOD, GOOD, None,
                                                GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 40, None)
    assert dec(lk=None) == EINVAL
    assert dec(lk=BAD) == EALIGN
    assert dec(s=shape(L=0, gate=1)) == EUNSUPPORTED


def _device_visible():
    # (counting devices through torch does not initialise the GPU on this image)
    import torch
    return os.path.exists("/dev/kfd") or torch.cuda.device_count() > 0


@pytest.mark.skipif(_device_visible(), reason="needs a machine without a GPU: the call below passes "
                    "validation with placeholder pointers and must fail at its launch")
def test_launch_failure_returns_ehip(lib):
    """A call that passes validation but whose launch fails (here: no device at all) returns
    LIZARD_EHIP instead of succeeding or crashing, for the forward, backward and decode step."""
    s = shape()
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 0)
    assert lib.lizard_attn_fwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None, None, None,
                               None, GOOD, need, None) == EHIP
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 1)
    assert lib.lizard_attn_bwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD, GOOD,
                               GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, need, None, None) == EHIP
    d = shape(L=0)
    need = lib.lizard_attn_workspace_bytes(ctypes.byref(d), 2)
    assert lib.lizard_attn_decode_step(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD,
                                       GOOD, GOOD, GOOD, need, None) == EHIP
    assert lib.lizard_attn_decode_step_noalloc(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD,
                                               GOOD, GOOD, GOOD, None) == EHIP


def test_decode_noalloc_validation(lib):
    """The allocation-free decode step validates like the plain one."""
    def call(s_, state=GOOD, pos=GOOD, o=GOOD):
        return lib.lizard_attn_decode_step_noalloc(ctypes.byref(s_), GOOD, GOOD, GOOD, GOOD, GOOD, None,
                                                   state, GOOD, GOOD, pos, o, None)
    assert call(shape(L=0), state=None) == EINVAL
    assert call(shape(L=0), o=None) == EINVAL
    assert call(shape(L=0), pos=BAD) == EALIGN
    assert call(shape(L=0, W=9000)) == EUNSUPPORTED
    assert call(shape(L=0, d_k=96, d_v=96)) == EUNSUPPORTED


def test_general_path_validation(lib):
    """Chunks of 16, 32 and 128 tokens and fp32 at d = 128 run on the general path (forward and
    backward of the plain layer): accepted up to the workspace check, with their own workspace
    layout (the gates' 16-token block sums, then the chunk states); the entry points that run on
    the fast kernels only (log features, continuation, Hedgehog map) refuse them."""
    up = lambda x: (x + 255) // 256 * 256
    B, H, L, D = 1, 2, 128, 128
    for kw in (dict(chunk=16), dict(chunk=32), dict(chunk=128), dict(dtype=0), dict(dtype=0, chunk=16)):
        s = shape(**kw)
        C = kw.get("chunk", 64)
        esz = 4 if kw.get("dtype", 1) == 0 else 2
        nc, nb = (L + C - 1) // C, (L + 15) // 16
        need = lib.lizard_attn_workspace_bytes(ctypes.byref(s), 0)
        assert need == up(4 * B * H * L * D) + up(4 * B * H * nb * D) + up(esz * B * H * nc * D * D), kw
        assert lib.lizard_attn_workspace_bytes(ctypes.byref(s), 1) > 0
        assert lib.lizard_attn_workspace_bytes(ctypes.byref(s), 6) > lib.lizard_attn_workspace_bytes(ctypes.byref(s), 1)
        fwd_call = lambda ws, nbytes: lib.lizard_attn_fwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD,
                                                          None, None, None, None, ws, nbytes, None)
        assert fwd_call(None, 0) == EWORKSPACE, kw
        assert fwd_call(GOOD, need - 1) == EWORKSPACE, kw
        assert fwd_call(BAD, need) == EALIGN, kw
        assert lib.lizard_attn_bwd(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD, GOOD, GOOD,
                                   GOOD, GOOD, GOOD, GOOD, None, None, 0, None, None) == EWORKSPACE, kw
        # fast kernels only
        assert lib.lizard_attn_fwd_feat(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None,
                                        None, GOOD, None, GOOD, 1 << 40, None) == EUNSUPPORTED, kw
        assert lib.lizard_attn_bwd_feat(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD,
                                        GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, 1 << 40,
                                        None, None) == EUNSUPPORTED, kw
        assert lib.lizard_attn_fwd_continue(ctypes.byref(s), GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD,
                                            GOOD, GOOD, GOOD, 1 << 40, None) == EUNSUPPORTED, kw
        assert lib.lizard_attn_workspace_bytes(ctypes.byref(s), 3) == 0, kw
    f128 = shape(dtype=0)
    assert lib.lizard_hedgehog_fwd(ctypes.byref(f128), GOOD, GOOD, GOOD, None) == EUNSUPPORTED
    assert lib.lizard_hedgehog_bwd(ctypes.byref(f128), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 40, None) == EUNSUPPORTED

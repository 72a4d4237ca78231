"""The C ABI on the CPU: the library loads, exports what include/kda.h
declares, sizes the state independently of context length, and rejects bad
arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_83_amd as kda
from gated_delta_rule_83_amd import kda as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # an aligned address that is never dereferenced on these paths


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[A-Za-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = kda.lib()
    names = header_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(K.EXPORTED) == names


def test_state_size_independent_of_context():
    # 69 layers x 96 heads x 128 x 128 x 4 bytes = 414 MiB ("414MB 的 KDA 状态从哪来")
    d = kda.make_dims(69, 96, 128, 128, kda.KDA_F32)
    s, r = kda.kda_state_bytes(d)
    assert s == 69 * 96 * 128 * 128 * 4 == 434_110_464
    assert abs(s / 2**20 - 414) < 0.01
    # ring: 3 projections x 3 taps x 96*128 channels x 4 bytes x 69 layers ~ 30 MiB
    assert r == 69 * 3 * 96 * (3 * 128) * 4
    assert 29 < r / 2**20 < 30
    # the size query takes no token count; bf16 rings are half as large
    s2, r2 = kda.kda_state_bytes(kda.make_dims(69, 96, 128, 128, kda.KDA_BF16))
    assert s2 == s and r2 * 2 == r


@pytest.mark.parametrize("dims,code", [
    ((1, 2, 96, 16, 0, 4), kda.KDAError),
    ((0, 2, 16, 16, 0, 4), kda.KDAError),
    ((1, 2, 16, 16, 0, 3), kda.KDAError),
    ((1, 2, 16, 16, 7, 4), kda.KDAError),
])
def test_bad_dims_rejected(dims, code):
    B, H, dk, dv, io, w = dims
    d = kda.make_dims(B, H, dk, dv, io, conv_width=w)
    assert kda.kda_state_bytes(d) == (0, 0)
    with pytest.raises(code):
        kda.kda_state_alloc(d, FAKE, FAKE)


def test_unsupported_width_code():
    d = kda.make_dims(1, 2, 96, 16, kda.KDA_F32)
    h = ctypes.c_void_p()
    st = kda.lib().kda_state_alloc(ctypes.byref(d), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                   ctypes.byref(h))
    assert st == K.KDA_ERR_UNSUPPORTED
    assert "d_k=96" in kda.last_error()


@pytest.fixture
def fake_state():
    d = kda.make_dims(2, 3, 16, 32, kda.KDA_F32)
    h = ctypes.c_void_p()
    assert kda.lib().kda_state_alloc(ctypes.byref(d), ctypes.c_void_p(FAKE),
                                     ctypes.c_void_p(2 * FAKE), ctypes.byref(h)) == 0
    yield h
    kda.kda_state_free(h)  # caller-owned buffers: nothing is freed on the device


def test_views_and_dims(fake_state):
    assert kda.kda_state_S(fake_state) == FAKE
    assert kda.kda_state_ring(fake_state) == 2 * FAKE
    d = kda.kda_state_get_dims(fake_state)
    assert (d.batch, d.heads, d.d_k, d.d_v, d.conv_width) == (2, 3, 16, 32, 4)


def _vp(x):
    return ctypes.c_void_p(x) if x is not None else None


def call_decode(h, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, w=FAKE, o=FAKE, flags=0):
    return kda.lib().kda_decode_step(h, _vp(q), _vp(k), _vp(v), _vp(g), _vp(beta), _vp(w),
                                     _vp(o), flags, None)


def call_prefill(h, T=8, chunk=64, ws=None, ws_bytes=0, flags=0, q=FAKE, w=FAKE):
    return kda.lib().kda_chunk_prefill(h, T, _vp(q), _vp(FAKE), _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                       _vp(w), _vp(FAKE), chunk, _vp(ws), ws_bytes, flags, None)


def test_decode_validation(fake_state):
    assert call_decode(None) == K.KDA_ERR_INVALID
    assert call_decode(fake_state, q=None) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert call_decode(fake_state, beta=FAKE + 2) == K.KDA_ERR_INVALID
    assert "4-byte aligned" in kda.last_error()
    assert call_decode(fake_state, w=FAKE + 4) == K.KDA_ERR_INVALID
    assert "conv_w is not 16-byte aligned" in kda.last_error()
    assert call_decode(fake_state, flags=16) == K.KDA_ERR_INVALID
    assert call_decode(fake_state, w=None) == K.KDA_ERR_INVALID
    assert "conv_w" in kda.last_error()


def test_prefill_validation(fake_state):
    assert call_prefill(fake_state, chunk=48) == K.KDA_ERR_UNSUPPORTED
    assert call_prefill(fake_state, T=-1) == K.KDA_ERR_INVALID
    assert call_prefill(fake_state, T=0) == K.KDA_OK          # nothing to do
    assert call_prefill(fake_state, q=None) == K.KDA_ERR_INVALID
    assert call_prefill(fake_state, ws=FAKE, ws_bytes=16) == K.KDA_ERR_INVALID
    assert "below" in kda.last_error()


def test_prefill_null_workspace_validates_before_allocating(fake_state):
    """With workspace = NULL the call may allocate the handle's buffer (and so
    synchronise); every argument is checked before that, so a bad call fails
    with its own error and allocates nothing (include/kda.h)."""
    assert call_prefill(fake_state, ws=None, q=None) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert call_prefill(fake_state, ws=None, chunk=8) == K.KDA_ERR_UNSUPPORTED
    assert call_prefill(fake_state, ws=None, T=0) == K.KDA_OK
    assert call_prefill(fake_state, ws=FAKE + 8, ws_bytes=1 << 30) == K.KDA_ERR_INVALID
    assert "16-byte aligned" in kda.last_error()


def call_prefill_noalloc(h, T=8, chunk=64, flags=0, q=FAKE, w=FAKE):
    return kda.lib().kda_chunk_prefill_noalloc(h, T, _vp(q), _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                               _vp(FAKE), _vp(w), _vp(FAKE), chunk, flags, None)


def test_prefill_noalloc_validation(fake_state):
    """The allocation-free prefill validates like kda_chunk_prefill and rejects
    a state whose single chunk does not fit its fixed scratch, all before any
    device call."""
    assert call_prefill_noalloc(None) == K.KDA_ERR_INVALID
    assert call_prefill_noalloc(fake_state, q=None) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert call_prefill_noalloc(fake_state, chunk=48) == K.KDA_ERR_UNSUPPORTED
    assert call_prefill_noalloc(fake_state, T=0) == K.KDA_OK
    assert call_prefill_noalloc(fake_state, flags=16) == K.KDA_ERR_INVALID
    d = kda.make_dims(12, 96, 128, 128, kda.KDA_BF16)  # 85.5 MB per chunk > 64 MiB
    assert kda.kda_prefill_workspace_bytes(d, 64, 64) > kda.KDA_NOALLOC_SCRATCH_BYTES
    h = ctypes.c_void_p()
    assert kda.lib().kda_state_alloc(ctypes.byref(d), ctypes.c_void_p(FAKE),
                                     ctypes.c_void_p(2 * FAKE), ctypes.byref(h)) == 0
    try:
        assert call_prefill_noalloc(h, T=64) == K.KDA_ERR_UNSUPPORTED
        assert "static scratch" in kda.last_error()
    finally:
        kda.kda_state_free(h)


def test_stream_probe_validation():
    L = kda.lib()
    assert L.kda_stream_rmw(None, 16, ctypes.c_float(1.0), None) == K.KDA_ERR_INVALID
    assert L.kda_stream_rmw(_vp(FAKE + 4), 16, ctypes.c_float(1.0), None) == K.KDA_ERR_INVALID
    assert L.kda_stream_rmw(_vp(FAKE), 20, ctypes.c_float(1.0), None) == K.KDA_ERR_INVALID


def test_scalar_decay_flag_validation(fake_state):
    """KDA_F_SCALAR_G and KDA_F_RAW_GATES are flags of the decode step and the
    prefill only: there validation goes on past them (to the NULL q here); the
    prologue rejects them."""
    sg = kda.KDA_F_SCALAR_G
    assert call_decode(fake_state, q=None, flags=sg) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert call_decode(fake_state, flags=sg | 16) == K.KDA_ERR_INVALID
    assert call_prefill(fake_state, q=None, flags=sg | kda.KDA_F_SKIP_CONV) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert call_prefill(fake_state, T=0, flags=sg) == K.KDA_OK
    d = kda.make_dims(1, 2, 16, 16, kda.KDA_F32)
    assert kda.lib().kda_conv_prologue(ctypes.byref(d), 4, *([_vp(FAKE)] * 8), sg,
                                       None) == K.KDA_ERR_INVALID
    assert "0x4" in kda.last_error()
    raw = kda.KDA_F_RAW_GATES
    assert call_decode(fake_state, q=None, flags=raw | sg) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert call_prefill(fake_state, q=None, flags=raw) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert kda.lib().kda_conv_prologue(ctypes.byref(d), 4, *([_vp(FAKE)] * 8), raw,
                                       None) == K.KDA_ERR_INVALID
    assert "0x8" in kda.last_error()


def test_output_gate_validation(fake_state):
    """Argument checks of the output gate entry points (every case fails before
    anything is enqueued)."""
    L = kda.lib()
    d = kda.make_dims(1, 2, 16, 16, kda.KDA_F32)
    f = ctypes.c_float

    def gate(T=4, x=FAKE, z=2 * FAKE, w=3 * FAKE, eps=1e-5, out=FAKE):
        return L.kda_gated_rmsnorm(ctypes.byref(d), T, _vp(x), _vp(z), _vp(w), f(eps), _vp(out),
                                   None)

    assert gate(T=0) == K.KDA_OK
    assert gate(T=-1) == K.KDA_ERR_INVALID
    for bad in (0.0, -1e-5, float("inf"), float("nan")):
        assert gate(eps=bad) == K.KDA_ERR_INVALID
        assert "eps" in kda.last_error()
    assert gate(x=None) == K.KDA_ERR_INVALID
    assert gate(w=3 * FAKE + 4) == K.KDA_ERR_INVALID
    assert "norm_w is not 16-byte aligned" in kda.last_error()
    assert gate(out=FAKE + 64) == K.KDA_ERR_INVALID          # partly overlaps x
    assert "overlaps x" in kda.last_error()
    assert gate(out=2 * FAKE) == K.KDA_ERR_INVALID           # is the gate
    assert "overlaps gate" in kda.last_error()

    def dec(gate_p=4 * FAKE, w=3 * FAKE, eps=1e-5, q=FAKE, flags=0):
        return L.kda_decode_step_gated(fake_state, _vp(q), _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                       _vp(FAKE), _vp(FAKE), _vp(gate_p), _vp(w), f(eps),
                                       _vp(FAKE), flags, None)

    assert dec(gate_p=None) == K.KDA_ERR_INVALID
    assert "gate is NULL" in kda.last_error()
    assert dec(w=None) == K.KDA_ERR_INVALID
    assert dec(eps=0.0) == K.KDA_ERR_INVALID
    assert dec(q=None) == K.KDA_ERR_INVALID
    assert "q is NULL" in kda.last_error()
    assert dec(flags=16) == K.KDA_ERR_INVALID
    assert L.kda_decode_step_gated(None, *([_vp(FAKE)] * 8), f(1e-5), _vp(FAKE), 0,
                                   None) == K.KDA_ERR_INVALID


def test_reset_validation(fake_state):
    arr = (ctypes.c_int32 * 2)(0, 5)
    assert kda.lib().kda_state_reset(fake_state, arr, 2, None) == K.KDA_ERR_INVALID
    assert "outside" in kda.last_error()
    assert kda.lib().kda_state_reset(None, None, 0, None) == K.KDA_ERR_INVALID
    arr = (ctypes.c_int32 * 1)(0)
    assert kda.lib().kda_state_reset(fake_state, arr, -1, None) == K.KDA_ERR_INVALID


def test_prologue_validation():
    d = kda.make_dims(1, 2, 16, 16, kda.KDA_F32)
    L = kda.lib()
    assert L.kda_conv_prologue(ctypes.byref(d), -1, *([_vp(FAKE)] * 8), 0, None) == K.KDA_ERR_INVALID
    assert L.kda_conv_prologue(ctypes.byref(d), 0, *([None] * 8), 0, None) == K.KDA_OK
    assert L.kda_conv_prologue(ctypes.byref(d), 4, None, *([_vp(FAKE)] * 7), 0, None) == \
        K.KDA_ERR_INVALID


def test_workspace_size():
    d = kda.make_dims(1, 96, 128, 128, kda.KDA_BF16)
    one = kda.kda_prefill_workspace_bytes(d, 64, 64)
    # per chunk-head: -W, Q~ [64x128], K^T [128x64], P [64x64], U' [64x128] bf16 + 128 fp32
    assert one == 96 * ((3 * 64 * 128 + 64 * 64 + 64 * 128) * 2 + 128 * 4)
    assert kda.kda_prefill_workspace_bytes(d, 4096, 64) == 64 * one
    assert kda.kda_prefill_workspace_bytes(d, 4097, 64) == 65 * one
    assert kda.kda_prefill_workspace_bytes(d, 64, 48) == 0


def call_backward(d, T=8, chunk=16, ws_bytes=None, flags=0, S0=None, dST=None, dS0=None,
                  **ptrs):
    names = ["q", "k", "v", "g", "beta", "dO", "dq", "dk", "dv", "dg", "dbeta", "ws"]
    p = {n: ptrs.get(n, FAKE) for n in names}
    if ws_bytes is None:
        ws_bytes = kda.kda_backward_workspace_bytes(d, max(T, 0), chunk)
    L = kda.lib()
    return L.kda_chunk_backward(
        ctypes.byref(d), T, _vp(p["q"]), _vp(p["k"]), _vp(p["v"]), _vp(p["g"]), _vp(p["beta"]),
        _vp(S0), _vp(p["dO"]), _vp(dST), _vp(p["dq"]), _vp(p["dk"]), _vp(p["dv"]),
        _vp(p["dg"]), _vp(p["dbeta"]), _vp(dS0), chunk, _vp(p["ws"]), ws_bytes, flags, None)


def test_backward_workspace_size():
    d = kda.make_dims(1, 96, 128, 128, kda.KDA_F32)
    one = kda.kda_backward_workspace_bytes(d, 64, 64)
    # per chunk-head: 9 [64 x 128] and 2 [64 x 128] token arrays, 5 [64 x 64],
    # e^{Gam_n} [128], plus the entering state and its gradient [128 x 128]
    assert one == 96 * 4 * (11 * 64 * 128 + 5 * 64 * 64 + 128 + 2 * 128 * 128)
    assert kda.kda_backward_workspace_bytes(d, 4096, 64) == 64 * one
    assert kda.kda_backward_workspace_bytes(d, 4097, 64) == 65 * one
    assert kda.kda_backward_workspace_bytes(d, 0, 64) == 0
    assert kda.kda_backward_workspace_bytes(d, 64, 48) == 0
    assert kda.kda_backward_workspace_bytes(d, -1, 64) == 0


def test_backward_validation():
    d = kda.make_dims(2, 3, 16, 32, kda.KDA_F32)
    assert call_backward(d, T=-1) == K.KDA_ERR_INVALID
    assert call_backward(d, chunk=48) == K.KDA_ERR_UNSUPPORTED
    assert call_backward(d, flags=kda.KDA_F_SKIP_CONV) == K.KDA_ERR_INVALID
    for name in ["q", "k", "v", "g", "beta", "dO", "dq", "dk", "dv", "dg", "dbeta", "ws"]:
        assert call_backward(d, **{name: None}) == K.KDA_ERR_INVALID, name
        assert {"ws": "workspace"}.get(name, name) in kda.last_error()
    assert call_backward(d, q=FAKE + 4) == K.KDA_ERR_INVALID       # 16-byte activations
    assert call_backward(d, g=FAKE + 4) == K.KDA_ERR_INVALID
    assert call_backward(d, dO=FAKE + 8) == K.KDA_ERR_INVALID
    assert call_backward(d, dq=FAKE + 2) == K.KDA_ERR_INVALID      # fp32 output: 4 bytes
    assert call_backward(d, ws=FAKE + 4) == K.KDA_ERR_INVALID      # 16-byte workspace
    assert call_backward(d, S0=FAKE + 4) == K.KDA_ERR_INVALID
    assert call_backward(d, dST=FAKE + 4) == K.KDA_ERR_INVALID
    assert call_backward(d, dS0=FAKE + 4) == K.KDA_ERR_INVALID
    need = kda.kda_backward_workspace_bytes(d, 8, 16)
    assert call_backward(d, ws_bytes=need - 1) == K.KDA_ERR_INVALID
    assert "workspace" in kda.last_error()
    # T = 0 with no dS0 asked for: nothing to do, nothing enqueued
    assert call_backward(d, T=0, ws_bytes=0, ws=None, q=None, dO=None) == K.KDA_OK
    bad = kda.make_dims(1, 1, 24, 32, kda.KDA_F32)
    assert call_backward(bad, ws_bytes=0) == K.KDA_ERR_UNSUPPORTED


def test_prologue_backward_validation():
    d = kda.make_dims(2, 3, 16, 32, kda.KDA_F32)
    L = kda.lib()
    ctot = 3 * (2 * 16 + 32)
    assert kda.kda_prologue_backward_workspace_bytes(d, 32) == 2 * 1 * ctot * 16
    assert kda.kda_prologue_backward_workspace_bytes(d, 33) == 2 * 2 * ctot * 16
    assert kda.kda_prologue_backward_workspace_bytes(d, -1) == 0
    need = kda.kda_prologue_backward_workspace_bytes(d, 8)
    names = ["q", "k", "v", "w", "ring", "dqh", "dkh", "dvh", "dq", "dk", "dv", "dw", "dring",
             "ws"]

    def call(T=8, ws_bytes=need, flags=0, **over):
        p = {n: over.get(n, FAKE) for n in names}
        return L.kda_prologue_backward(ctypes.byref(d), T, *[_vp(p[n]) for n in names],
                                       ws_bytes, flags, None)

    assert call(T=-1) == K.KDA_ERR_INVALID
    assert call(flags=1) == K.KDA_ERR_INVALID
    for name in ["q", "k", "v", "w", "dqh", "dkh", "dvh", "dq", "dk", "dv", "dw", "ws"]:
        assert call(**{name: None}) == K.KDA_ERR_INVALID, name
    assert call(w=FAKE + 4) == K.KDA_ERR_INVALID
    assert call(dw=FAKE + 4) == K.KDA_ERR_INVALID
    assert call(q=FAKE + 4) == K.KDA_ERR_INVALID
    assert call(ring=FAKE + 8) == K.KDA_ERR_INVALID
    assert call(dvh=FAKE + 8) == K.KDA_ERR_INVALID
    assert call(ws=FAKE + 4) == K.KDA_ERR_INVALID
    assert call(ws_bytes=need - 1) == K.KDA_ERR_INVALID
    assert "workspace" in kda.last_error()
    bad = kda.make_dims(1, 1, 24, 32, kda.KDA_F32)
    assert L.kda_prologue_backward(ctypes.byref(bad), 8, *[_vp(FAKE)] * 14, need, 0, None) == \
        K.KDA_ERR_UNSUPPORTED


def test_backward_workspace_sizes():
    """The one-pass size is per chunk and head; the least size the call
    accepts takes chunk ranges with kept states and is far smaller at a
    training layer's length (16 x 32768 tokens, 96 heads of 128 x 128)."""
    d = kda.make_dims(16, 96, 128, 128, kda.KDA_BF16)
    full = kda.kda_backward_workspace_bytes(d, 32768, 64)
    least = kda.kda_backward_workspace_min_bytes(d, 32768, 64)
    assert full > 400e9 and 10e9 < least < 16e9
    state = 16 * 96 * 128 * 128 * 4
    per_chunk = full // 512
    # the least is the best range length: L chunks' blocks + one state per range
    best = min(L * per_chunk + -(-512 // L) * state for L in range(1, 512))
    assert least == min(best, full)
    # small cases: one chunk needs no kept state, T = 0 nothing
    d1 = kda.make_dims(1, 2, 32, 32, kda.KDA_F32)
    assert kda.kda_backward_workspace_min_bytes(d1, 64, 64) == kda.kda_backward_workspace_bytes(d1, 64, 64)
    assert kda.kda_backward_workspace_min_bytes(d1, 0, 64) == 0
    # invalid arguments give 0
    assert kda.kda_backward_workspace_min_bytes(d1, -1, 64) == 0
    assert kda.kda_backward_workspace_min_bytes(d1, 64, 48) == 0
    assert kda.kda_backward_workspace_min_bytes(kda.make_dims(1, 2, 24, 32, kda.KDA_F32), 64, 64) == 0

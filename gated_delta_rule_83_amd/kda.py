"""ctypes binding of libkda.so (include/kda.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory (tensor data
pointers) and streams; nothing here computes on tensor values. If the
library is not built the import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_ERR_INVALID, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP, KDA_ERR_OOM = 0, -1, -2, -3, -4
KDA_F32, KDA_BF16 = 0, 1
KDA_F_SKIP_CONV, KDA_F_SKIP_L2, KDA_F_SCALAR_G, KDA_F_RAW_GATES = 1, 2, 4, 8
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20  # the fixed scratch of kda_chunk_prefill_noalloc

EXPORTED = [
    "kda_state_bytes", "kda_state_alloc", "kda_state_reset", "kda_state_free",
    "kda_state_S", "kda_state_ring", "kda_state_get_dims", "kda_conv_prologue",
    "kda_decode_step", "kda_prefill_workspace_bytes", "kda_chunk_prefill",
    "kda_chunk_prefill_noalloc",
    "kda_gated_rmsnorm", "kda_decode_step_gated", "kda_backward_workspace_bytes",
    "kda_backward_workspace_min_bytes",
    "kda_chunk_backward", "kda_prologue_backward_workspace_bytes", "kda_prologue_backward",
    "kda_stream_rmw", "kda_last_error", "kda_version",
]


class kda_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("io", ctypes.c_int)]


class KDAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"kda status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    f32 = ctypes.c_float
    dp = ctypes.POINTER(kda_dims)
    sig = {
        "kda_state_bytes": (sz, [dp, ctypes.POINTER(sz)]),
        "kda_state_alloc": (ctypes.c_int, [dp, vp, vp, ctypes.POINTER(vp)]),
        "kda_state_reset": (ctypes.c_int, [vp, ctypes.POINTER(i32), i32, vp]),
        "kda_state_free": (None, [vp]),
        "kda_state_S": (vp, [vp]),
        "kda_state_ring": (vp, [vp]),
        "kda_state_get_dims": (ctypes.c_int, [vp, dp]),
        "kda_conv_prologue": (ctypes.c_int, [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp]),
        "kda_decode_step": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, u32, vp]),
        "kda_prefill_workspace_bytes": (sz, [dp, i32, i32]),
        "kda_chunk_prefill": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz,
                                             u32, vp]),
        "kda_chunk_prefill_noalloc": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp, vp, vp, i32,
                                                     u32, vp]),
        "kda_gated_rmsnorm": (ctypes.c_int, [dp, i32, vp, vp, vp, f32, vp, vp]),
        "kda_decode_step_gated": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp,
                                                 u32, vp]),
        "kda_backward_workspace_bytes": (sz, [dp, i32, i32]),
        "kda_backward_workspace_min_bytes": (sz, [dp, i32, i32]),
        "kda_chunk_backward": (ctypes.c_int, [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, i32, vp, sz, u32, vp]),
        "kda_prologue_backward_workspace_bytes": (sz, [dp, i32]),
        "kda_prologue_backward": (ctypes.c_int, [dp, i32] + [vp] * 14 + [sz, u32, vp]),
        "kda_stream_rmw": (ctypes.c_int, [vp, sz, f32, vp]),
        "kda_last_error": (ctypes.c_char_p, []),
        "kda_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().kda_last_error().decode()


def _check(status):
    if status != KDA_OK:
        raise KDAError(status, last_error())


def make_dims(batch, heads, d_k, d_v, io=KDA_BF16, conv_width=4) -> kda_dims:
    if isinstance(io, torch.dtype):
        io = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}[io]
    return kda_dims(int(batch), int(heads), int(d_k), int(d_v), int(conv_width), int(io))


def io_dtype(dims: kda_dims) -> torch.dtype:
    return torch.bfloat16 if dims.io == KDA_BF16 else torch.float32


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or an int device pointer")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# ---- the C entry points, same names ---------------------------------------

def kda_state_bytes(dims: kda_dims):
    """(state bytes, ring bytes); (0, 0) for invalid or unsupported dims."""
    rb = ctypes.c_size_t(0)
    sb = lib().kda_state_bytes(ctypes.byref(dims), ctypes.byref(rb))
    return int(sb), int(rb.value)


def kda_state_alloc(dims: kda_dims, s_mem=None, ring_mem=None):
    h = ctypes.c_void_p()
    _check(lib().kda_state_alloc(ctypes.byref(dims), _ptr(s_mem, "s_mem", torch.float32),
                                 _ptr(ring_mem, "ring_mem", io_dtype(dims)), ctypes.byref(h)))
    return h


def kda_state_reset(handle, seq_ids=None, stream=None):
    if seq_ids is None:
        _check(lib().kda_state_reset(handle, None, 0, _stream(stream)))
        return
    ids = [int(i) for i in seq_ids]
    arr = (ctypes.c_int32 * max(1, len(ids)))(*ids)
    _check(lib().kda_state_reset(handle, arr, len(ids), _stream(stream)))


def kda_state_free(handle):
    lib().kda_state_free(handle)


def kda_state_S(handle) -> int:
    return lib().kda_state_S(handle) or 0


def kda_state_ring(handle) -> int:
    return lib().kda_state_ring(handle) or 0


def kda_state_get_dims(handle) -> kda_dims:
    d = kda_dims()
    _check(lib().kda_state_get_dims(handle, ctypes.byref(d)))
    return d


def kda_conv_prologue(dims, T, q, k, v, conv_w, ring, q_out, k_out, v_out, flags=0,
                      stream=None):
    io = io_dtype(dims)
    _check(lib().kda_conv_prologue(
        ctypes.byref(dims), int(T), _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(conv_w, "conv_w", torch.float32), _ptr(ring, "ring", io),
        _ptr(q_out, "q_out", torch.float32), _ptr(k_out, "k_out", torch.float32),
        _ptr(v_out, "v_out", torch.float32), int(flags), _stream(stream)))


def kda_decode_step(handle, q, k, v, g, beta, conv_w, o, flags=0, stream=None, io=None):
    io = io or io_dtype(kda_state_get_dims(handle))
    _check(lib().kda_decode_step(
        handle, _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(g, "g", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(conv_w, "conv_w", torch.float32), _ptr(o, "o", io), int(flags), _stream(stream)))


def kda_decode_step_gated(handle, q, k, v, g, beta, conv_w, gate, norm_w, eps, o, flags=0,
                          stream=None, io=None):
    io = io or io_dtype(kda_state_get_dims(handle))
    _check(lib().kda_decode_step_gated(
        handle, _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(g, "g", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(conv_w, "conv_w", torch.float32), _ptr(gate, "gate", io),
        _ptr(norm_w, "norm_w", torch.float32), ctypes.c_float(eps), _ptr(o, "o", io),
        int(flags), _stream(stream)))


def kda_gated_rmsnorm(dims, T, x, gate, norm_w, eps, out, stream=None):
    io = io_dtype(dims)
    _check(lib().kda_gated_rmsnorm(
        ctypes.byref(dims), int(T), _ptr(x, "x", io), _ptr(gate, "gate", io),
        _ptr(norm_w, "norm_w", torch.float32), ctypes.c_float(eps), _ptr(out, "out", io),
        _stream(stream)))


def kda_prefill_workspace_bytes(dims, T, chunk=64) -> int:
    return int(lib().kda_prefill_workspace_bytes(ctypes.byref(dims), int(T), int(chunk)))


def kda_chunk_prefill(handle, T, q, k, v, g, beta, conv_w, o, chunk=64, workspace=None,
                      flags=0, stream=None, io=None):
    io = io or io_dtype(kda_state_get_dims(handle))
    ws_bytes = 0
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().kda_chunk_prefill(
        handle, int(T), _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(g, "g", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(conv_w, "conv_w", torch.float32), _ptr(o, "o", io), int(chunk),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes), int(flags), _stream(stream)))


def kda_chunk_prefill_noalloc(handle, T, q, k, v, g, beta, conv_w, o, chunk=64, flags=0,
                              stream=None, io=None):
    """kda_chunk_prefill with the library's fixed device scratch as the
    workspace: the call allocates nothing (include/kda.h)."""
    io = io or io_dtype(kda_state_get_dims(handle))
    _check(lib().kda_chunk_prefill_noalloc(
        handle, int(T), _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(g, "g", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(conv_w, "conv_w", torch.float32), _ptr(o, "o", io), int(chunk), int(flags),
        _stream(stream)))


def kda_stream_rmw(buf, scale=1.0, stream=None):
    """In-place buf *= scale with the decode's state-stream memory pattern
    (a measurement helper; include/kda.h)."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().kda_stream_rmw(_ptr(buf, "buf"), ctypes.c_size_t(nbytes), ctypes.c_float(scale),
                                _stream(stream)))


def kda_backward_workspace_bytes(dims, T, chunk=64) -> int:
    return int(lib().kda_backward_workspace_bytes(ctypes.byref(dims), int(T), int(chunk)))


def kda_backward_workspace_min_bytes(dims, T, chunk=64) -> int:
    return int(lib().kda_backward_workspace_min_bytes(ctypes.byref(dims), int(T), int(chunk)))


def kda_chunk_backward(dims, T, q, k, v, g, beta, S0, dO, dST, dq, dk, dv, dg, dbeta, dS0,
                       chunk=64, workspace=None, flags=0, stream=None):
    """Gradients of the recurrence for T tokens (include/kda.h). S0, dST and
    dS0 may be None. `workspace` is a device tensor of at least
    kda_backward_workspace_min_bytes(dims, T, chunk) bytes (with less than
    kda_backward_workspace_bytes the chunks are taken in ranges); if None, one
    of kda_backward_workspace_bytes is taken from torch's allocator for this
    call."""
    io = io_dtype(dims)
    need = kda_backward_workspace_bytes(dims, T, chunk)
    if workspace is None and need > 0:
        dev = next(t.device for t in (q, dO, dS0) if isinstance(t, torch.Tensor))
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    f32 = torch.float32
    _check(lib().kda_chunk_backward(
        ctypes.byref(dims), int(T), _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(g, "g", f32), _ptr(beta, "beta", f32), _ptr(S0, "S0", f32), _ptr(dO, "dO", io),
        _ptr(dST, "dST", f32), _ptr(dq, "dq", io), _ptr(dk, "dk", io), _ptr(dv, "dv", io),
        _ptr(dg, "dg", f32), _ptr(dbeta, "dbeta", f32), _ptr(dS0, "dS0", f32), int(chunk),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes), int(flags), _stream(stream)))


def kda_prologue_backward_workspace_bytes(dims, T) -> int:
    return int(lib().kda_prologue_backward_workspace_bytes(ctypes.byref(dims), int(T)))


def kda_prologue_backward(dims, T, q, k, v, conv_w, ring, dq_hat, dk_hat, dv_hat, dq, dk, dv,
                          dconv_w, dring, workspace=None, flags=0, stream=None):
    """Gradients of the prologue (include/kda.h). ring and dring may be None;
    with workspace None one is taken from torch's allocator for this call."""
    io = io_dtype(dims)
    need = kda_prologue_backward_workspace_bytes(dims, T)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dconv_w.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    f32 = torch.float32
    _check(lib().kda_prologue_backward(
        ctypes.byref(dims), int(T), _ptr(q, "q", io), _ptr(k, "k", io), _ptr(v, "v", io),
        _ptr(conv_w, "conv_w", f32), _ptr(ring, "ring", io), _ptr(dq_hat, "dq_hat", io),
        _ptr(dk_hat, "dk_hat", io), _ptr(dv_hat, "dv_hat", io), _ptr(dq, "dq", io),
        _ptr(dk, "dk", io), _ptr(dv, "dv", io), _ptr(dconv_w, "dconv_w", f32),
        _ptr(dring, "dring", f32), _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        int(flags), _stream(stream)))


def kda_version() -> str:
    return lib().kda_version().decode()


# ---- a handle whose S and ring are torch-owned device tensors --------------

class KDAState:
    """Session state of one KDA layer for `batch` sequences. S [B,H,dk,dv]
    fp32 and ring [B,3,H*(2dk+dv)] (io dtype) are torch tensors; the library
    handle refers to them and never frees them."""

    def __init__(self, batch, heads, d_k, d_v, io=torch.bfloat16, device="cuda"):
        self.dims = make_dims(batch, heads, d_k, d_v, io)
        self.io = io_dtype(self.dims)
        ctot = heads * (2 * d_k + d_v)
        self.S = torch.empty((batch, heads, d_k, d_v), dtype=torch.float32, device=device)
        self.ring = torch.empty((batch, 3, ctot), dtype=self.io, device=device)
        self.handle = kda_state_alloc(self.dims, self.S, self.ring)

    def reset(self, seq_ids=None, stream=None):
        kda_state_reset(self.handle, seq_ids, stream)

    def decode_step(self, q, k, v, g, beta, conv_w, o, flags=0, stream=None):
        kda_decode_step(self.handle, q, k, v, g, beta, conv_w, o, flags, stream, io=self.io)

    def decode_step_gated(self, q, k, v, g, beta, conv_w, gate, norm_w, eps, o, flags=0,
                          stream=None):
        kda_decode_step_gated(self.handle, q, k, v, g, beta, conv_w, gate, norm_w, eps, o,
                              flags, stream, io=self.io)

    def gated_rmsnorm(self, T, x, gate, norm_w, eps, out, stream=None):
        """The output gate on T tokens of this state's dims ([B,T,H,dv] tensors)."""
        kda_gated_rmsnorm(self.dims, T, x, gate, norm_w, eps, out, stream)

    def prefill(self, T, q, k, v, g, beta, conv_w, o, chunk=64, workspace=None, flags=0,
                stream=None):
        kda_chunk_prefill(self.handle, T, q, k, v, g, beta, conv_w, o, chunk, workspace, flags,
                          stream, io=self.io)

    def close(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            kda_state_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

"""KDA oracle: plain fp64 CPU implementations of the recurrence.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. It shares no code
with the GPU library and imports nothing from it.

Two independent formulations live here:

* :class:`Oracle` (and the module-level :func:`forward`, :func:`core`,
  :func:`prologue`) call ``kda_oracle.c``, built into ``libkda_oracle.so``
  by :func:`oracle.build.build`: the sequential
  per-token recurrence (short conv + SiLU, L2 normalisation of q and k, decay
  along the key axis, delta read, rank-1 write, readout), as stated in
  "KV缓存从11.25GB缩到0.21GB：WARP中Kimi Delta Attention线性注意力原理剖析",
  section "KDA 递推公式先衰减再差分".
* :func:`chunked_core`, numpy: the chunkwise-parallel form of the same
  recurrence described in "为什么 Kimi K3 敢把 KV Cache 扔掉？一篇讲透 GPT-2 到 K3
  的架构进化", section 5 (attention-like work inside a chunk, the previous
  chunk's final state passed on, a WY-style triangular solve) and section 6
  (the cumulative in-chunk decay). It exists so that the chunked and
  sequential forms can be checked against each other.

Two more steps around the recurrence, each a reading stated in
``kda_oracle.c``: :meth:`Oracle.gated_rmsnorm`, the output gate that follows
the readout (a gated RMSNorm per token and head), and
:meth:`Oracle.gates_from_raw`, the decay and beta formed from raw projections
(log-sigmoid and sigmoid). :meth:`Oracle.core_backward` is the gradient of
the recurrence for training, by reverse-mode differentiation token by token.

The decay g is per key channel. The scalar-alpha Gated DeltaNet form (one
decay per token and head, same page, sections 6 and 7) is the case of g equal
on every key channel of a head, so it is checked by passing g repeated over
d_k; that the case reproduces the Gated DeltaNet update of section 7 is a
pin of its own in the tests.

Everything is float64. bf16 inputs are upcast exactly before they get here.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
from scipy.linalg import solve_triangular

SKIP_CONV = 1
SKIP_L2 = 2
L2_EPS = 1e-6

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """The C oracle behind a ctypes handle (``lib_path`` defaults to the
    library built from ``kda_oracle.c``)."""

    def __init__(self, lib_path=None):
        lib_path = lib_path or LIB_PATH
        if not os.path.exists(lib_path):
            from oracle.build import build

            build(out=lib_path)
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kdao_forward.argtypes = ([ctypes.c_int] * 5 + [dp] * 9
                                     + [ctypes.c_int, ctypes.c_double, ctypes.c_int])
        lib.kdao_forward.restype = ctypes.c_int
        lib.kdao_prologue.argtypes = ([ctypes.c_int] * 5 + [dp] * 8
                                      + [ctypes.c_int, ctypes.c_double, ctypes.c_int])
        lib.kdao_prologue.restype = ctypes.c_int
        lib.kdao_gated_rmsnorm.argtypes = [ctypes.c_long, ctypes.c_int, dp, dp, dp,
                                           ctypes.c_double, dp]
        lib.kdao_gated_rmsnorm.restype = ctypes.c_int
        lib.kdao_gates_from_raw.argtypes = [ctypes.c_long, dp, dp, ctypes.c_long, dp, dp]
        lib.kdao_gates_from_raw.restype = ctypes.c_int
        lib.kdao_core_backward.argtypes = [ctypes.c_int] * 5 + [dp] * 14
        lib.kdao_core_backward.restype = ctypes.c_int
        lib.kdao_prologue_backward.argtypes = ([ctypes.c_int] * 5 + [dp] * 8
                                               + [ctypes.c_double] + [dp] * 5)
        lib.kdao_prologue_backward.restype = ctypes.c_int
        lib.kdao_max_threads.argtypes = []
        lib.kdao_max_threads.restype = ctypes.c_int
        self.lib = lib

    def max_threads(self) -> int:
        """Threads the C oracle uses by default (OpenMP)."""
        return int(self.lib.kdao_max_threads())

    def forward(self, q, k, v, g, beta, conv_w=None, S0=None, ring0=None, flags=0,
                eps=L2_EPS, threads=0):
        """Sequential KDA over a batch of token blocks.

        q, k: [B,T,H,dk]; v: [B,T,H,dv]; g: [B,T,H,dk] (log decay);
        beta: [B,T,H]; conv_w: [H*(2dk+dv), 4]; S0: [B,H,dk,dv] (zeros if
        None); ring0: [B,3,H*(2dk+dv)] (zeros if None).
        Returns (o [B,T,H,dv], S [B,H,dk,dv], ring [B,3,Ctot]), float64.
        """
        q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and g.shape == q.shape
        assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
        ctot = H * (2 * dk + dv)
        S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
        assert S.shape == (B, H, dk, dv)
        ring = np.zeros((B, 3, ctot)) if ring0 is None else _f64(ring0).copy()
        assert ring.shape == (B, 3, ctot)
        w = np.zeros((ctot, 4)) if conv_w is None else _f64(conv_w)
        assert w.shape == (ctot, 4)
        o = np.zeros((B, T, H, dv))
        rc = self.lib.kdao_forward(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                   _ptr(beta), _ptr(w), _ptr(ring), _ptr(S), _ptr(o),
                                   int(flags), float(eps), int(threads))
        if rc != 0:
            raise RuntimeError("kdao_forward failed")
        return o, S, ring

    def core(self, qh, kh, vh, g, beta, S0=None, eps=L2_EPS, threads=0):
        """Decay, delta read, rank-1 write and readout only, on activations
        that are already convolved and normalised (shapes as in forward)."""
        o, S, _ = self.forward(qh, kh, vh, g, beta, None, S0, None,
                               flags=SKIP_CONV | SKIP_L2, eps=eps, threads=threads)
        return o, S

    def prologue(self, q, k, v, conv_w, ring0=None, flags=0, eps=L2_EPS, threads=0):
        """Short conv + SiLU on q, k, v and L2 normalisation of q, k.

        Returns (q_hat, k_hat, v_hat, ring) in float64."""
        q, k, v = map(_f64, (q, k, v))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        ctot = H * (2 * dk + dv)
        ring = np.zeros((B, 3, ctot)) if ring0 is None else _f64(ring0).copy()
        w = np.zeros((ctot, 4)) if conv_w is None else _f64(conv_w)
        assert w.shape == (ctot, 4) and ring.shape == (B, 3, ctot)
        qo = np.zeros_like(q)
        ko = np.zeros_like(k)
        vo = np.zeros_like(v)
        rc = self.lib.kdao_prologue(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(w),
                                    _ptr(ring), _ptr(qo), _ptr(ko), _ptr(vo),
                                    int(flags), float(eps), int(threads))
        if rc != 0:
            raise RuntimeError("kdao_prologue failed")
        return qo, ko, vo, ring

    def gated_rmsnorm(self, x, z, w, eps):
        """Output gate on readout vectors: x, z [..., n] (rows of n values: one
        token of one head), w [n]. Returns y [..., n] in float64,
        y = x / sqrt(mean(x^2) + eps) * w * sigmoid(z) per row."""
        x, z, w = map(_f64, (x, z, w))
        n = x.shape[-1]
        assert z.shape == x.shape and w.shape == (n,)
        y = np.empty_like(x)
        rc = self.lib.kdao_gated_rmsnorm(x.size // n, n, _ptr(x), _ptr(z), _ptr(w),
                                         float(eps), _ptr(y))
        if rc != 0:
            raise RuntimeError("kdao_gated_rmsnorm failed")
        return y

    def gates_from_raw(self, a, b):
        """Gates from raw projections: g = log(sigmoid(a)) (any shape) and
        beta = sigmoid(b). Returns (g, beta) in float64."""
        a, b = _f64(a), _f64(b)
        g, beta = np.empty_like(a), np.empty_like(b)
        rc = self.lib.kdao_gates_from_raw(a.size, _ptr(a), _ptr(g), b.size, _ptr(b), _ptr(beta))
        if rc != 0:
            raise RuntimeError("kdao_gates_from_raw failed")
        return g, beta

    def core_backward(self, qh, kh, vh, g, beta, S0, dO, dST):
        """Gradient of the recurrence (decay, delta read, rank-1 write,
        readout) for the linear functional sum(dO * o) + sum(dST * S_T):
        returns dq, dk, dv, dg, dbeta, dS0 (float64, shapes of the inputs).
        Keeps every state of a forward pass: small inputs only."""
        qh, kh, vh, g, beta, S0, dO, dST = map(_f64, (qh, kh, vh, g, beta, S0, dO, dST))
        B, T, H, dk = qh.shape
        dv = vh.shape[-1]
        assert kh.shape == qh.shape and g.shape == qh.shape and beta.shape == (B, T, H)
        assert vh.shape == dO.shape == (B, T, H, dv) and S0.shape == dST.shape == (B, H, dk, dv)
        out = [np.zeros_like(qh), np.zeros_like(kh), np.zeros_like(vh), np.zeros_like(g),
               np.zeros_like(beta), np.zeros_like(S0)]
        rc = self.lib.kdao_core_backward(B, T, H, dk, dv, _ptr(qh), _ptr(kh), _ptr(vh), _ptr(g),
                                         _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dST),
                                         *[_ptr(x) for x in out])
        if rc != 0:
            raise RuntimeError("kdao_core_backward failed")
        return tuple(out)

    def prologue_backward(self, q, k, v, conv_w, ring0, dqh, dkh, dvh, eps=L2_EPS):
        """Gradient of the prologue (conv, SiLU, L2 of q and k) for the linear
        functional sum(dqh * q^) + sum(dkh * k^) + sum(dvh * v^): returns
        dq, dk, dv (raw projections), dconv_w [Ctot, 4] and dring [B, 3, Ctot]
        (the history read from the ring), float64."""
        q, k, v, dqh, dkh, dvh = map(_f64, (q, k, v, dqh, dkh, dvh))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        ctot = H * (2 * dk + dv)
        w = _f64(conv_w)
        ring = np.zeros((B, 3, ctot)) if ring0 is None else _f64(ring0)
        assert k.shape == q.shape == dqh.shape == dkh.shape and v.shape == dvh.shape
        assert w.shape == (ctot, 4) and ring.shape == (B, 3, ctot)
        out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros((ctot, 4)),
               np.zeros((B, 3, ctot))]
        rc = self.lib.kdao_prologue_backward(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(w),
                                             _ptr(ring), _ptr(dqh), _ptr(dkh), _ptr(dvh),
                                             float(eps), *[_ptr(x) for x in out])
        if rc != 0:
            raise RuntimeError("kdao_prologue_backward failed")
        return tuple(out)

    def chunked_core(self, *args, **kwargs):
        return chunked_core(*args, **kwargs)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def max_threads() -> int:
    return default().max_threads()


def forward(*args, **kwargs):
    return default().forward(*args, **kwargs)


def core(*args, **kwargs):
    return default().core(*args, **kwargs)


def prologue(*args, **kwargs):
    return default().prologue(*args, **kwargs)


def gated_rmsnorm(*args, **kwargs):
    return default().gated_rmsnorm(*args, **kwargs)


def gates_from_raw(*args, **kwargs):
    return default().gates_from_raw(*args, **kwargs)


def chunked_core(qh, kh, vh, g, beta, S0, chunk):
    """Chunkwise-parallel KDA for ONE head, fp64 (activations already
    convolved and normalised).

    qh, kh, g: [T, dk]; vh: [T, dv]; beta: [T]; S0: [dk, dv].
    Returns (o [T, dv], S [dk, dv]).

    Per chunk of n <= chunk tokens entering with state S:
      Gam_r = sum_{i<=r} g_i                       (cumulative in-chunk decay)
      A_rj  = sum_c k_r[c] k_j[c] exp(Gam_r[c] - Gam_j[c]),  j < r
      P_rj  = sum_c q_r[c] k_j[c] exp(Gam_r[c] - Gam_j[c]),  j <= r
      (I + diag(beta) A) U = diag(beta) (V - (exp(Gam) * K) S)   (WY solve)
      O     = (exp(Gam) * Q) S + P U               (intra-chunk attention)
      S    <- Diag(exp(Gam_n)) S + (exp(Gam_n - Gam) * K)^T U    (state pass)
    Requires finite g <= 0 (exponents of the form Gam_r - Gam_j, j <= r, are
    then <= 0).
    """
    qh, kh, vh, g, beta, S = map(_f64, (qh, kh, vh, g, beta, S0))
    S = S.copy()
    T, dk = qh.shape
    dv = vh.shape[1]
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        Q, K, V = qh[c0:c0 + n], kh[c0:c0 + n], vh[c0:c0 + n]
        G, bt = g[c0:c0 + n], beta[c0:c0 + n]
        Gam = np.cumsum(G, axis=0)
        le = np.tril(np.ones((n, n), dtype=bool))          # j <= r
        lt = np.tril(np.ones((n, n), dtype=bool), -1)      # j < r
        diff = Gam[:, None, :] - Gam[None, :, :]          # [r, j, c]
        E = np.where(le[:, :, None], np.exp(np.where(le[:, :, None], diff, 0.0)), 0.0)
        A = np.einsum("rc,jc,rjc->rj", K, K, E) * lt
        P = np.einsum("rc,jc,rjc->rj", Q, K, E) * le
        Ktil = np.exp(Gam) * K
        Qtil = np.exp(Gam) * Q
        M = np.eye(n) + bt[:, None] * A
        rhs = bt[:, None] * (V - Ktil @ S)
        U = solve_triangular(M, rhs, lower=True, unit_diagonal=True)
        o[c0:c0 + n] = Qtil @ S + P @ U
        Khat = np.exp(Gam[-1][None, :] - Gam) * K
        S = np.exp(Gam[-1])[:, None] * S + Khat.T @ U
    return o, S

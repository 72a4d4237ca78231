"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an :class:`oracle.kda_oracle.Oracle` and raises
AssertionError when the oracle disagrees with the pinned fact. They are kept
as plain functions so the same checks can run against deliberately broken
builds of the oracle (tests/test_oracle_mutants.py).

Pages cited:
  [WARP] "KV缓存从11.25GB缩到0.21GB：WARP中Kimi Delta Attention线性注意力原理剖析"
  [K3]   "为什么 Kimi K3 敢把 KV Cache 扔掉？一篇讲透 GPT-2 到 K3 的架构进化"
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_case(seed, B=1, T=9, H=2, dk=4, dv=3, g_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = -np.log1p(np.exp(-rng.standard_normal((B, T, H, dk)))) * g_scale  # logsigmoid
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    ctot = H * (2 * dk + dv)
    w = 0.5 * rng.standard_normal((ctot, 4))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    ring = rng.standard_normal((B, 3, ctot))
    return q, k, v, g, beta, w, S0, ring


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# P-a: the pages' worked example ([K3] section 4).
def pin_worked_example(orc):
    fx = json.load(open(os.path.join(GOLDEN, "delta_rule_worked_example.json")))
    k = np.array(fx["k"])
    v = np.stack([fx["v1"], fx["v2"]])                      # [2, 2]
    ex = fx["expected"]
    kk = np.broadcast_to(k, (1, 2, 1, 2)).copy()             # same key twice
    vv = v.reshape(1, 2, 1, 2)
    g = np.zeros((1, 2, 1, 2))
    # L2 normalisation on (eps = 0 so |k_hat| = 1 exactly), beta = 1, q = k.
    o, S, _ = orc.forward(kk, kk, vv, g, np.ones((1, 2, 1)), flags=1, eps=0.0)
    np.testing.assert_allclose(o[0, 0, 0], ex["o1"], atol=1e-12)
    np.testing.assert_allclose(o[0, 1, 0], ex["o2"], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], ex["S2_normalised"], atol=1e-12)
    # plain addition would read v1 + v2; the delta rule must not.
    assert np.abs(o[0, 1, 0] - np.array(ex["plain_addition_read_normalised"])).max() > 1.0
    # raw key, L2 off, beta = 1/|k|^2 = 0.1
    o, S, _ = orc.forward(kk, kk, vv, g, np.full((1, 2, 1), 0.1), flags=3)
    np.testing.assert_allclose(o[0, 0, 0], ex["o1"], atol=1e-12)
    np.testing.assert_allclose(o[0, 1, 0], ex["o2"], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], ex["S2_raw_beta_0p1"], atol=1e-12)


# --------------------------------------------------------------------------
# P-b: g = 0 gives the plain delta rule. Independent forms printed in [K3]
# section 7, kept in the d_v x d_k orientation they are printed in:
#   DeltaNet:          S_t = S_{t-1} - v_old k^T + v_new k^T   (beta = 1)
#   Gated DeltaNet:    S_t = S_{t-1} alpha (I - beta k k^T) + beta v k^T
def pin_zero_decay_is_delta_rule(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(1, T=8)
    qh, kh = _unit_rows(q), _unit_rows(k)
    g0 = np.zeros_like(g)
    B, T, H, dk = qh.shape
    dv = v.shape[-1]
    # Gated DeltaNet form with alpha = 1, arbitrary beta
    o, S = orc.core(qh, kh, v, g0, beta, S0)
    for h in range(H):
        Sp = S0[0, h].T.copy()                                 # d_v x d_k
        for t in range(T):
            kt, vt, bt = kh[0, t, h], v[0, t, h], beta[0, t, h]
            Sp = Sp @ (np.eye(dk) - bt * np.outer(kt, kt)) + bt * np.outer(vt, kt)
            np.testing.assert_allclose(o[0, t, h], Sp @ qh[0, t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], Sp.T, atol=1e-12)
    # DeltaNet form at beta = 1
    ones = np.ones_like(beta)
    o, S = orc.core(qh, kh, v, g0, ones, S0)
    for h in range(H):
        Sp = S0[0, h].T.copy()
        for t in range(T):
            kt, vt = kh[0, t, h], v[0, t, h]
            v_old = Sp @ kt
            Sp = Sp - np.outer(v_old, kt) + np.outer(vt, kt)
            np.testing.assert_allclose(o[0, t, h], Sp @ qh[0, t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], Sp.T, atol=1e-12)


# P-b': the same decay on every key channel gives scalar-alpha Gated DeltaNet.
def pin_scalar_decay_is_gated_deltanet(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(2, T=8)
    qh, kh = _unit_rows(q), _unit_rows(k)
    B, T, H, dk = qh.shape
    gs = g[..., :1].repeat(dk, axis=-1)                         # same g per channel
    o, S = orc.core(qh, kh, v, gs, beta, S0)
    for h in range(H):
        Sp = S0[0, h].T.copy()
        for t in range(T):
            a = np.exp(gs[0, t, h, 0])
            kt, vt, bt = kh[0, t, h], v[0, t, h], beta[0, t, h]
            Sp = Sp * a @ (np.eye(dk) - bt * np.outer(kt, kt)) + bt * np.outer(vt, kt)
            np.testing.assert_allclose(o[0, t, h], Sp @ qh[0, t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], Sp.T, atol=1e-12)


# --------------------------------------------------------------------------
# P-c: alpha = 0 (g = -inf) clears memory ([K3] section 6): whatever the
# previous state, S_t = beta k v^T and o_t = beta (k.q) v.
def pin_minus_inf_clears_memory(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(3, T=1)
    qh, kh = _unit_rows(q), _unit_rows(k)
    gi = np.full_like(g, -np.inf)
    o, S = orc.core(qh, kh, v, gi, beta, S0)
    for h in range(qh.shape[2]):
        b = beta[0, 0, h]
        np.testing.assert_allclose(S[0, h], b * np.outer(kh[0, 0, h], v[0, 0, h]), atol=1e-14)
        np.testing.assert_allclose(o[0, 0, h], b * (kh[0, 0, h] @ qh[0, 0, h]) * v[0, 0, h],
                                   atol=1e-14)
    # mid-sequence: a cleared token cuts every dependence on the tokens before it
    q, k, v, g, beta, w, S0, ring = _rand_case(4, T=10)
    qh, kh = _unit_rows(q), _unit_rows(k)
    g[:, 4] = -np.inf
    o_full, S_full = orc.core(qh, kh, v, g, beta, S0)
    o_tail, S_tail = orc.core(qh[:, 4:], kh[:, 4:], v[:, 4:], g[:, 4:], beta[:, 4:], None)
    np.testing.assert_allclose(o_full[:, 4:], o_tail, atol=1e-13)
    np.testing.assert_allclose(S_full, S_tail, atol=1e-13)
    # clearing only some key channels zeroes only those rows before the write
    q, k, v, g, beta, w, S0, ring = _rand_case(5, T=1)
    g[0, 0, :, :2] = -np.inf
    kh = _unit_rows(k)
    kh[0, 0, :, :2] = 0.0                                      # write nothing there
    o, S = orc.core(_unit_rows(q), kh, v, g, beta, S0)
    np.testing.assert_allclose(S[0, :, :2, :], 0.0, atol=0)


# --------------------------------------------------------------------------
# P-e: the chunked form ([K3] section 5) and the sequential form agree; C = 1
# is the recurrence itself and C = T the single quadratic block.
def pin_chunked_equals_sequential(orc):
    from oracle.kda_oracle import chunked_core

    q, k, v, g, beta, w, S0, ring = _rand_case(6, T=37, H=1, dk=8, dv=5)
    qh, kh = _unit_rows(q), _unit_rows(k)
    o, S = orc.core(qh, kh, v, g, beta, S0)
    for C in (1, 2, 4, 16, 37, 64):
        oc, Sc = chunked_core(qh[0, :, 0], kh[0, :, 0], v[0, :, 0], g[0, :, 0],
                              beta[0, :, 0], S0[0, 0], C)
        np.testing.assert_allclose(oc, o[0, :, 0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(Sc, S[0, 0], atol=1e-12, rtol=0)


# P-form: the two-step statement in [WARP] (decay, then delta on the decayed
# state) equals the one-line Kimi Linear update in [K3] section 7:
#   S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,  o_t = S_t^T q_t.
def pin_kimi_linear_form(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(7, T=7, dk=5, dv=3)
    qh, kh = _unit_rows(q), _unit_rows(k)
    o, S = orc.core(qh, kh, v, g, beta, S0)
    dk = qh.shape[-1]
    for h in range(qh.shape[2]):
        St = S0[0, h].copy()
        for t in range(qh.shape[1]):
            kt, vt, bt = kh[0, t, h], v[0, t, h], beta[0, t, h]
            St = (np.eye(dk) - bt * np.outer(kt, kt)) @ np.diag(np.exp(g[0, t, h])) @ St \
                + bt * np.outer(kt, vt)
            np.testing.assert_allclose(o[0, t, h], St.T @ qh[0, t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


# P-f: exact recall. With |k| = 1, beta = 1 and q = k, the readout returns the
# value just written, whatever g and the previous state are.
def pin_exact_recall(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(8, T=12)
    kh = _unit_rows(k)
    o, S = orc.core(kh, kh, v, g, np.ones_like(beta), S0, eps=0.0)
    np.testing.assert_allclose(o, v, atol=1e-12)
    # and for beta < 1 the readout mixes old and new: o = (1-beta) S'^T k + beta v
    o1, _ = orc.core(kh[:, :1], kh[:, :1], v[:, :1], g[:, :1], beta[:, :1], S0)
    for h in range(kh.shape[2]):
        Sd = np.exp(g[0, 0, h])[:, None] * S0[0, h]
        b = beta[0, 0, h]
        exp_o = (1 - b) * Sd.T @ kh[0, 0, h] + b * v[0, 0, h]
        np.testing.assert_allclose(o1[0, 0, h], exp_o, atol=1e-12)


# --------------------------------------------------------------------------
# P-g: the prologue reduces to library routines: depthwise causal conv1d of
# width 4 (padding 3, first T outputs), SiLU, and a unit-norm rescaling.
def pin_prologue_library(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(9, B=2, T=11, H=2, dk=4, dv=3)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    qo, ko, vo, ring_out = orc.prologue(q, k, v, w, ring, flags=2)   # conv+SiLU only
    x = np.concatenate([q.reshape(B, T, H * dk), k.reshape(B, T, H * dk),
                        v.reshape(B, T, H * dv)], axis=-1)            # [B, T, Ctot]
    xt = torch.from_numpy(np.concatenate([ring, x], axis=1)).permute(0, 2, 1)  # [B, C, 3+T]
    wt = torch.from_numpy(w).unsqueeze(1)                                       # [C, 1, 4]
    y = torch.nn.functional.conv1d(xt, wt, groups=wt.shape[0])                  # valid conv
    ref = torch.nn.functional.silu(y).permute(0, 2, 1).numpy()                  # [B, T, C]
    got = np.concatenate([qo.reshape(B, T, -1), ko.reshape(B, T, -1),
                          vo.reshape(B, T, -1)], axis=-1)
    np.testing.assert_allclose(got, ref, atol=1e-12)
    # the ring now holds the last three raw tokens
    np.testing.assert_array_equal(ring_out, np.concatenate([ring, x], axis=1)[:, -3:])
    # weights (0,0,0,1) make the conv the identity: output is SiLU(x)
    w_id = np.zeros_like(w)
    w_id[:, 3] = 1.0
    qo2, ko2, vo2, _ = orc.prologue(q, k, v, w_id, ring, flags=2)
    np.testing.assert_allclose(vo2, torch.nn.functional.silu(torch.from_numpy(v)).numpy(),
                               atol=1e-14)
    # L2 on: q_hat and k_hat have unit norm and point along the conv output
    qn, kn, vn, _ = orc.prologue(q, k, v, w, ring, eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(qn, axis=-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(kn, axis=-1), 1.0, atol=1e-12)
    cos = np.sum(qn * qo, axis=-1) / np.linalg.norm(qo, axis=-1)
    np.testing.assert_allclose(cos, 1.0, atol=1e-12)
    np.testing.assert_allclose(vn, vo, atol=0)                          # v is not normalised
    # causality: changing token 6 leaves outputs before token 6 unchanged
    q2 = q.copy()
    q2[:, 6] += 1.0
    qa, _, _, _ = orc.prologue(q2, k, v, w, ring)
    qb, _, _, _ = orc.prologue(q, k, v, w, ring)
    np.testing.assert_array_equal(qa[:, :6], qb[:, :6])
    assert np.abs(qa[:, 6:10] - qb[:, 6:10]).max() > 1e-6


# P-h: session state hand-off. Running T1 then T2 tokens (S and ring carried
# over) equals one run of T1 + T2 tokens, including splits shorter than the
# ring.
def pin_split_calls(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(10, B=2, T=13)
    o, S, r = orc.forward(q, k, v, g, beta, w, S0, ring)
    for T1 in (1, 2, 3, 7):
        o1, S1, r1 = orc.forward(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1],
                                 w, S0, ring)
        o2, S2, r2 = orc.forward(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:],
                                 w, S1, r1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-13)
        np.testing.assert_allclose(S2, S, atol=1e-13)
        np.testing.assert_array_equal(r2, r)
    # a chain of one-token calls (decode) gives the same too
    St, rt, outs = S0, ring, []
    for t in range(q.shape[1]):
        sl = slice(t, t + 1)
        ot, St, rt = orc.forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], w, St, rt)
        outs.append(ot)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), o, atol=1e-13)
    np.testing.assert_allclose(St, S, atol=1e-13)


# P-i: with |k| = 1, 0 <= beta <= 1 and g <= 0 each step grows the state by at
# most beta |v| in Frobenius norm: (I - beta k k^T) and Diag(exp g) are
# contractions.
def pin_stability_bound(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(11, T=20)
    qh, kh = _unit_rows(q), _unit_rows(k)
    S = S0
    for t in range(q.shape[1]):
        sl = slice(t, t + 1)
        _, Sn = orc.core(qh[:, sl], kh[:, sl], v[:, sl], g[:, sl], beta[:, sl], S, eps=0.0)
        for h in range(q.shape[2]):
            lhs = np.linalg.norm(Sn[0, h])
            rhs = np.linalg.norm(S[0, h]) + beta[0, t, h] * np.linalg.norm(v[0, t, h])
            assert lhs <= rhs + 1e-12
        S = Sn


# P-j: value columns never mix; with S0 = 0 the outputs are linear in v.
def pin_columns_and_linearity(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(12, T=9, dk=4, dv=6)
    qh, kh = _unit_rows(q), _unit_rows(k)
    perm = np.array([3, 0, 5, 1, 4, 2])
    o, S = orc.core(qh, kh, v, g, beta, S0)
    op, Sp = orc.core(qh, kh, v[..., perm], g, beta, S0[..., perm])
    np.testing.assert_allclose(op, o[..., perm], atol=1e-13)
    np.testing.assert_allclose(Sp, S[..., perm], atol=1e-13)
    v2 = np.random.default_rng(13).standard_normal(v.shape)
    oa, Sa = orc.core(qh, kh, v, g, beta, None)
    ob, Sb = orc.core(qh, kh, v2, g, beta, None)
    oc, Sc = orc.core(qh, kh, v + 2.0 * v2, g, beta, None)
    np.testing.assert_allclose(oc, oa + 2.0 * ob, atol=1e-12)
    np.testing.assert_allclose(Sc, Sa + 2.0 * Sb, atol=1e-12)


# P-k: brute force on a tiny case: the state after T tokens is the explicit
# product of per-token transition matrices M_t = (I - beta k k^T) Diag(alpha)
# applied to S0, plus each token's write carried forward.
def pin_transition_product(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(14, T=6, H=1, dk=3, dv=2)
    qh, kh = _unit_rows(q), _unit_rows(k)
    o, S = orc.core(qh, kh, v, g, beta, S0)
    T, dk = qh.shape[1], qh.shape[-1]
    M = [(np.eye(dk) - beta[0, t, 0] * np.outer(kh[0, t, 0], kh[0, t, 0]))
         @ np.diag(np.exp(g[0, t, 0])) for t in range(T)]
    for t in range(T):
        acc = np.eye(dk)
        for s in range(t + 1):
            acc = M[s] @ acc
        St = acc @ S0[0, 0]
        for s in range(t + 1):
            carry = np.eye(dk)
            for u in range(s + 1, t + 1):
                carry = M[u] @ carry
            St = St + carry @ (beta[0, s, 0] * np.outer(kh[0, s, 0], v[0, s, 0]))
        np.testing.assert_allclose(o[0, t, 0], St.T @ qh[0, t, 0], atol=1e-12)
    np.testing.assert_allclose(S[0, 0], St, atol=1e-12)


# --------------------------------------------------------------------------
# Output gate (gated RMSNorm after the readout; [WARP] "相关源码与文档导航"
# names it, [K3] section 6 gates the output; the formula is a reading):
# y = x / sqrt(mean x^2 + eps) * w * sigmoid(z) per (token, head) row.
def pin_gated_rmsnorm_library(orc):
    """Against torch's own RMSNorm and sigmoid (float64), several eps values."""
    rng = np.random.default_rng(71)
    for n, eps in ((16, 1e-6), (128, 1e-5), (32, 0.5)):
        x = rng.standard_normal((3, 5, 2, n)) * rng.uniform(0.1, 3.0, (3, 5, 2, 1))
        z = 2.0 * rng.standard_normal((3, 5, 2, n))
        w = 1.0 + 0.3 * rng.standard_normal(n)
        y = orc.gated_rmsnorm(x, z, w, eps)
        xt, zt, wt = (torch.from_numpy(a) for a in (x, z, w))
        want = torch.nn.functional.rms_norm(xt, (n,), wt, eps) * torch.sigmoid(zt)
        np.testing.assert_allclose(y, want.numpy(), rtol=1e-13, atol=1e-14)


def pin_gated_rmsnorm_closed_forms(orc):
    rng = np.random.default_rng(72)
    n = 24
    x = rng.standard_normal((6, n)) * np.array([0.01, 0.1, 1, 3, 10, 100])[:, None]
    ones = np.ones(n)
    big = np.full_like(x, 60.0)               # sigmoid(60) = 1 - 9e-27
    # open gate, unit weights, eps = 0: every row has mean square exactly 1
    y = orc.gated_rmsnorm(x, big, ones, 0.0)
    np.testing.assert_allclose((y * y).mean(-1), 1.0, rtol=1e-14)
    # with eps > 0 the mean square is m / (m + eps), m the row's mean square
    m = (x * x).mean(-1)
    y = orc.gated_rmsnorm(x, big, ones, 0.25)
    np.testing.assert_allclose((y * y).mean(-1), m / (m + 0.25), rtol=1e-13)
    # scale invariance at eps = 0, and the row direction is kept
    y1 = orc.gated_rmsnorm(x, big, ones, 0.0)
    y2 = orc.gated_rmsnorm(7.5 * x, big, ones, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    np.testing.assert_allclose(y1 * np.sqrt(m)[:, None], x, rtol=1e-13)
    # a closed gate (z = 0) halves everything; the weight scales per channel
    w = np.linspace(0.5, 2.0, n)
    z0 = np.zeros_like(x)
    np.testing.assert_allclose(orc.gated_rmsnorm(x, z0, w, 0.0), 0.5 * w * y1, rtol=1e-13)
    # gate values per channel: z -> -inf shuts a channel, the others are unchanged
    z = big.copy()
    z[:, 3] = -800.0
    y = orc.gated_rmsnorm(x, z, ones, 0.0)
    assert np.all(y[:, 3] == 0.0)
    np.testing.assert_allclose(np.delete(y, 3, -1), np.delete(y1, 3, -1), rtol=1e-13)
    # rows are independent: changing one row changes no other row
    x2 = x.copy()
    x2[2] *= -4.0
    x2[2, 0] += 1.0
    y = orc.gated_rmsnorm(x2, big, ones, 0.0)
    np.testing.assert_array_equal(np.delete(y, 2, 0), np.delete(y1, 2, 0))


# --------------------------------------------------------------------------
# Gates from raw projections ([K3] section 6: the Alpha/Beta projection sets
# the forgetting and update strengths; the sigmoid squashing is a reading):
# g = log(sigmoid(a)), beta = sigmoid(b).
def pin_gates_from_raw(orc):
    rng = np.random.default_rng(81)
    a = np.concatenate([4.0 * rng.standard_normal(200), [0.0, -700.0, 700.0, -40.0, 40.0]])
    b = 3.0 * rng.standard_normal(50)
    g, beta = orc.gates_from_raw(a, b)
    # torch's own log-sigmoid and sigmoid in float64
    at, bt = torch.from_numpy(a), torch.from_numpy(b)
    np.testing.assert_allclose(g, torch.nn.functional.logsigmoid(at).numpy(), rtol=1e-14,
                               atol=1e-300)
    np.testing.assert_allclose(beta, torch.sigmoid(bt).numpy(), rtol=1e-14)
    # closed forms: alpha = e^g = sigmoid(a) in (0, 1], g(0) = -ln 2, and
    # log sigmoid(a) - log sigmoid(-a) = a; sigmoid(b) + sigmoid(-b) = 1
    assert np.all(g <= 0.0)
    np.testing.assert_allclose(np.exp(g[:200]), 1.0 / (1.0 + np.exp(-a[:200])), rtol=1e-14)
    assert g[200] == -np.log(2.0)
    assert g[201] == -700.0                                   # a -> -inf: g ~ a
    np.testing.assert_allclose(g[202], -np.exp(-700.0), rtol=1e-14)  # a -> inf: g ~ -e^-a
    g_neg, beta_neg = orc.gates_from_raw(-a[:200], -b)
    np.testing.assert_allclose(g[:200] - g_neg, a[:200], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(beta + beta_neg, 1.0, rtol=1e-15)


# --------------------------------------------------------------------------
# Gradient of the recurrence (for training): the hand-derived reverse pass
# against central finite differences of the forward oracle itself, for every
# element of every input, on a linear functional of o and the final state.
def pin_core_backward_finite_differences(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(91, T=6, dk=3, dv=4)
    rng = np.random.default_rng(92)
    dO = rng.standard_normal(v.shape)
    dST = rng.standard_normal(S0.shape)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)

    def loss(a):
        o, S = orc.core(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"])
        return float((o * dO).sum() + (S * dST).sum())

    grads = orc.core_backward(q, k, v, g, beta, S0, dO, dST)
    h = 1e-6
    for name, grad in zip(("q", "k", "v", "g", "beta", "S0"), grads):
        x = args[name]
        assert grad.shape == x.shape
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            saved = x[idx]
            x[idx] = saved + h
            lp = loss(args)
            x[idx] = saved - h
            lm = loss(args)
            x[idx] = saved
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"d{name}")


# --------------------------------------------------------------------------
# Gradient of the prologue (for training): the hand-derived reverse pass
# against central finite differences of the forward prologue of the oracle,
# for every raw input element, conv weight and ring (history) element, on a
# linear functional of q^, k^ and v^.
def pin_prologue_backward_finite_differences(orc):
    q, k, v, g, beta, w, S0, ring = _rand_case(93, B=2, T=5, dk=3, dv=4)
    rng = np.random.default_rng(94)
    dqh, dkh, dvh = (rng.standard_normal(x.shape) for x in (q, k, v))
    args = dict(q=q, k=k, v=v, w=w, ring=ring)

    def loss(a):
        qh, kh, vh = orc.prologue(a["q"], a["k"], a["v"], a["w"], a["ring"])[:3]
        return float((qh * dqh).sum() + (kh * dkh).sum() + (vh * dvh).sum())

    grads = orc.prologue_backward(q, k, v, w, ring, dqh, dkh, dvh)
    h = 1e-6
    for name, grad in zip(("q", "k", "v", "w", "ring"), grads):
        x = args[name]
        assert grad.shape == x.shape
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            saved = x[idx]
            x[idx] = saved + h
            lp = loss(args)
            x[idx] = saved - h
            lm = loss(args)
            x[idx] = saved
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"d{name}")


ALL_PINS = [
    pin_worked_example,
    pin_zero_decay_is_delta_rule,
    pin_scalar_decay_is_gated_deltanet,
    pin_minus_inf_clears_memory,
    pin_chunked_equals_sequential,
    pin_kimi_linear_form,
    pin_exact_recall,
    pin_prologue_library,
    pin_split_calls,
    pin_stability_bound,
    pin_columns_and_linearity,
    pin_transition_product,
    pin_gated_rmsnorm_library,
    pin_gated_rmsnorm_closed_forms,
    pin_gates_from_raw,
    pin_core_backward_finite_differences,
    pin_prologue_backward_finite_differences,
]
